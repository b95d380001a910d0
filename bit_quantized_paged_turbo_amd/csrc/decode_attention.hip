// Paged single-token decode attention over a TurboQuant (or bf16) KV cache, gfx950.
//
// Method: "xInfer: Pure-Rust LLM Inference Without a Python Runtime" (hysenlabs.com):
//   section "What actually sits between the request and the tokens" — cached K/V rows are
//   Walsh-Hadamard rotated and absmax-quantized per head; section "TurboQuant is a memory
//   trade, and the README does not price it fully" — attention dequantizes the cache on
//   every step. Paging: infero landing page, section "Beyond plain text decode", item
//   "Continuous batching". Splitting one sequence over several workgroups and merging
//   with log-sum-exp mirrors the flash-attention split count of the infr page ("Introducing
//   infr: A Pure-Rust, Vulkan-First LLM Inference Engine", section "Configuration Without
//   Surprises").
//
// Because H is orthonormal, q.k = (Hq).(Hk): the query is rotated once (q' = Hq) and the
// scores are taken against the stored rotated rows; the value sum is formed in the rotated
// space and rotated back at the end (H is its own inverse).
//
// Kernel structure (one workgroup of 4 waves per (split, kv head, sequence)):
//   * the g = Hq/Hkv query heads of the kv head are rotated in LDS and quantized to
//     16-bit (turbo4/3: four signed 4-bit digits; turbo8: three signed 8-bit digits)
//     integers with one fp32 scale per head, so q'.c reduces to exact integer dot
//     products (v_dot8_i32_i4 / v_dot4_i32_i8 on the raw codes);
//   * every KV byte is read once per group: a wave step covers 16 tokens, lane l owns
//     token l/4 and dims [32*(l%4), +32) of it, so a step is one coalesced load of whole
//     code rows (a 1 KB turbo4 block at page size 16);
//   * the four partial dot products of a token are summed with two DPP quad exchanges;
//   * each lane keeps its own online-softmax state per head (running reference max m,
//     sum l, value sum acc[32]); m moves only when a score exceeds it by more than 2^8,
//     so rescaling is rare and exact in effect (any reference keeps the ratios);
//   * value codes are widened to fp32 with v_cvt_f32_ubyte after an offset-binary XOR,
//     the offset is removed once at the end from the sum of weights;
//   * at the end the 16 token lanes of each dim chunk and then the 4 waves are merged
//     with log-sum-exp; a sequence that fits one split is normalized, rotated back with
//     an in-LDS FWHT and stored; otherwise (m, l, acc) partials go to the workspace and
//     the combine kernel merges them.
#include "xq_internal.h"

namespace xq {
namespace {

constexpr int D = kHeadDim;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRotC = 0x1.6a09e6p-4f;   // fp32 nearest to 1/sqrt(128)
constexpr float kLazy = 8.0f;             // rescale only when a score beats m by > 2^8
constexpr float kQiMax4 = 30000.f;        // |q| bound for four signed 4-bit digits
constexpr float kQiMax8 = 8300000.f;      // |q| bound for three signed 8-bit digits

// Per-dtype geometry: bytes of a code row, bytes a lane loads per row, q digits and
// digit dwords per lane, and the offset-binary bias of value codes.
template <int DT> struct Fmt;
template <> struct Fmt<4> {
  static constexpr int kRow = 64, kLane = 16, kRaw = 4, kDig = 4, kQdw = 4, kQtot = 16;
  static constexpr float kOff = 8.f;
};
template <> struct Fmt<3> {
  static constexpr int kRow = 48, kLane = 12, kRaw = 3, kDig = 4, kQdw = 4, kQtot = 16;
  static constexpr float kOff = 8.f;
};
template <> struct Fmt<8> {
  static constexpr int kRow = 128, kLane = 32, kRaw = 8, kDig = 3, kQdw = 8, kQtot = 32;
  static constexpr float kOff = 128.f;
};
template <> struct Fmt<0> {
  static constexpr int kRow = 256, kLane = 64, kRaw = 16, kDig = 1, kQdw = 16, kQtot = 64;
  static constexpr float kOff = 0.f;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float half_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// DPP quad exchanges (lanes 4t..4t+3 hold the four dim chunks of one token)
__device__ __forceinline__ int quad_xor1(int v) { return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false); }
__device__ __forceinline__ int quad_xor2(int v) { return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false); }
__device__ __forceinline__ float quad_xor1f(float v) { return __int_as_float(quad_xor1(__float_as_int(v))); }
__device__ __forceinline__ float quad_xor2f(float v) { return __int_as_float(quad_xor2(__float_as_int(v))); }

// 3-bit fields [3k, 3k+3) of a 24-bit value -> sign-extended 4-bit nibbles k of a dword.
__device__ __forceinline__ uint32_t spread3to4(uint32_t x) {
  x = (x & 0xfffu) | ((x & 0xfff000u) << 4);            // 4 fields per 16-bit half
  x = (x & 0x003f003fu) | ((x & 0x0fc00fc0u) << 2);     // 2 fields per byte
  x = (x & 0x07070707u) | ((x & 0x38383838u) << 1);     // 1 field per nibble
  return x | ((x & 0x44444444u) << 1);                  // copy sign bit 2 -> bit 3
}

// Raw per-lane data of one 16-token step.
template <int DT> struct Raw {
  uint32_t k[Fmt<DT>::kRaw];
  uint32_t v[Fmt<DT>::kRaw];
  uint32_t ks, vs;
};

template <int DT>
__device__ __forceinline__ void load_raw(Raw<DT>& r, const uint8_t* kb, const uint8_t* vb,
                                         int slot, int c, int ps) {
  constexpr int RB = Fmt<DT>::kRow, LB = Fmt<DT>::kLane;
  const uint8_t* kp = kb + slot * RB + c * LB;
  const uint8_t* vp = vb + slot * RB + c * LB;
  if constexpr (DT == 3) {
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      r.k[i] = reinterpret_cast<const uint32_t*>(kp)[i];
      r.v[i] = reinterpret_cast<const uint32_t*>(vp)[i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < Fmt<DT>::kRaw / 4; ++i) {
      const uint4 a = reinterpret_cast<const uint4*>(kp)[i];
      const uint4 b = reinterpret_cast<const uint4*>(vp)[i];
      r.k[4 * i] = a.x; r.k[4 * i + 1] = a.y; r.k[4 * i + 2] = a.z; r.k[4 * i + 3] = a.w;
      r.v[4 * i] = b.x; r.v[4 * i + 1] = b.y; r.v[4 * i + 2] = b.z; r.v[4 * i + 3] = b.w;
    }
  }
  if constexpr (DT != 0) {
    r.ks = reinterpret_cast<const uint16_t*>(kb + ps * RB)[slot];
    r.vs = reinterpret_cast<const uint16_t*>(vb + ps * RB)[slot];
  } else {
    r.ks = r.vs = 0;
  }
}

template <int DT, int G>
struct State {
  float m[G], l[G], ws[G];
  float acc[G][32];
};

// One 16-token step for one lane: scores, online softmax, value accumulation.
template <int DT, int G>
__device__ __forceinline__ void process(const Raw<DT>& r, bool valid,
                                        const uint32_t (&qr)[G][Fmt<DT>::kDig][Fmt<DT>::kQdw],
                                        const float (&qs)[G], State<DT, G>& st) {
  // ---- scores z (log2 domain) ----------------------------------------------------------
  float z[G];
  if constexpr (DT == 4 || DT == 3) {
    uint32_t kc[4];
    if constexpr (DT == 4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) kc[i] = r.k[i];
    } else {
      kc[0] = r.k[0] & 0xffffffu;
      kc[1] = __builtin_amdgcn_alignbit(r.k[1], r.k[0], 24) & 0xffffffu;
      kc[2] = __builtin_amdgcn_alignbit(r.k[2], r.k[1], 16) & 0xffffffu;
      kc[3] = r.k[2] >> 8;
#pragma unroll
      for (int i = 0; i < 4; ++i) kc[i] = spread3to4(kc[i]);
    }
    const float sk = half_bits_to_f32(r.ks);
#pragma unroll
    for (int j = 0; j < G; ++j) {
      int a[4] = {0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int dg = 0; dg < 4; ++dg) a[dg] = __builtin_amdgcn_sdot8((int)qr[j][dg][i], (int)kc[i], a[dg], false);
      }
      int s = a[0] + (a[1] << 4) + (a[2] << 8) + (a[3] << 12);
      s += quad_xor1(s);
      s += quad_xor2(s);
      z[j] = valid ? (float)s * (sk * qs[j]) : -INFINITY;
    }
  } else if constexpr (DT == 8) {
    const float sk = half_bits_to_f32(r.ks);
#pragma unroll
    for (int j = 0; j < G; ++j) {
      int a[3] = {0, 0, 0};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int dg = 0; dg < 3; ++dg) a[dg] = __builtin_amdgcn_sdot4((int)qr[j][dg][i], (int)r.k[i], a[dg], false);
      }
#pragma unroll
      for (int dg = 0; dg < 3; ++dg) {
        a[dg] += quad_xor1(a[dg]);
        a[dg] += quad_xor2(a[dg]);
      }
      const float s = (float)a[2] * 65536.f + ((float)a[1] * 256.f + (float)a[0]);
      z[j] = valid ? s * (sk * qs[j]) : -INFINITY;
    }
  } else {  // bf16: q and k are bf16, exact products summed in fp32
#pragma unroll
    for (int j = 0; j < G; ++j) {
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
        a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, qr[j][0][i]),
                                            __builtin_bit_cast(v2bf, r.k[i]), a, false);
      }
      a += quad_xor1f(a);
      a += quad_xor2f(a);
      z[j] = valid ? a * qs[j] : -INFINITY;
    }
  }

  // ---- online softmax with a lazily moved reference ----------------------------------
  bool need = false;
#pragma unroll
  for (int j = 0; j < G; ++j) need |= z[j] > st.m[j] + kLazy;
  if (__builtin_expect(__any(need), 0)) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const bool up = z[j] > st.m[j] + kLazy;
      const float f = up ? __builtin_amdgcn_exp2f(st.m[j] - z[j]) : 1.f;
      st.m[j] = up ? z[j] : st.m[j];
      st.l[j] *= f;
      st.ws[j] *= f;
#pragma unroll
      for (int d = 0; d < 32; ++d) st.acc[j][d] *= f;
    }
  }
  float w[G];
  const float sv = (DT == 0) ? 1.f : half_bits_to_f32(r.vs);
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const float pj = valid ? __builtin_amdgcn_exp2f(z[j] - st.m[j]) : 0.f;
    st.l[j] += pj;
    w[j] = valid ? pj * sv : 0.f;
    st.ws[j] += w[j];
  }

  // ---- values --------------------------------------------------------------------------
  float v[32];
  if constexpr (DT == 4 || DT == 3) {
    uint32_t vc[4];
    if constexpr (DT == 4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) vc[i] = r.v[i];
    } else {
      vc[0] = r.v[0] & 0xffffffu;
      vc[1] = __builtin_amdgcn_alignbit(r.v[1], r.v[0], 24) & 0xffffffu;
      vc[2] = __builtin_amdgcn_alignbit(r.v[2], r.v[1], 16) & 0xffffffu;
      vc[3] = r.v[2] >> 8;
#pragma unroll
      for (int i = 0; i < 4; ++i) vc[i] = spread3to4(vc[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t x = vc[i] ^ 0x88888888u;     // code + 8, 0..15 per nibble
      const uint32_t e = x & 0x0f0f0f0fu;          // nibbles 0,2,4,6
      const uint32_t o = (x >> 4) & 0x0f0f0f0fu;   // nibbles 1,3,5,7
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[8 * i + 2 * k] = (float)((e >> (8 * k)) & 0xffu);
        v[8 * i + 2 * k + 1] = (float)((o >> (8 * k)) & 0xffu);
      }
    }
  } else if constexpr (DT == 8) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t x = r.v[i] ^ 0x80808080u;    // code + 128
#pragma unroll
      for (int k = 0; k < 4; ++k) v[4 * i + k] = (float)((x >> (8 * k)) & 0xffu);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t x = valid ? r.v[i] : 0u;     // unwritten slots may hold NaN patterns
      v[2 * i] = bf16_lo(x);
      v[2 * i + 1] = bf16_hi(x);
    }
  }
#pragma unroll
  for (int j = 0; j < G; ++j) {
#pragma unroll
    for (int d = 0; d < 32; ++d) st.acc[j][d] = fmaf(w[j], v[d], st.acc[j][d]);
  }
}

template <int G>
__device__ void fwht_lds(float (*x)[D + 4], int tid) {
  // in-place unnormalized FWHT of G rows of 128 floats; ends with a barrier
  for (int h = 1; h < D; h <<= 1) {
    __syncthreads();
    for (int k = tid; k < G * 64; k += kThreads) {
      const int j = k >> 6, r = k & 63;
      const int i = ((r / h) * 2 * h) + (r % h);
      const float a = x[j][i], b = x[j][i + h];
      x[j][i] = a + b;
      x[j][i + h] = a - b;
    }
  }
  __syncthreads();
}

template <int DT, int G>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeParams p) {
  using F = Fmt<DT>;
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int qh0 = kvh * G;
  const int L = min(p.context_lens[b], p.max_context_len);
  float* outp = p.out + ((int64_t)b * p.hq + qh0) * D;
  if (L <= 0) {
    if (split == 0)
      for (int i = tid; i < G * D; i += kThreads) outp[i] = 0.f;
    return;
  }
  const int tps = p.tokens_per_split;
  const int tok_begin = split * tps;
  if (tok_begin >= L) return;
  const int tok_end = min(L, tok_begin + tps);
  const int nsplit_b = (L + tps - 1) / tps;

  __shared__ float qf[G][D + 4];
  __shared__ uint32_t qd[G][F::kDig][F::kQtot];
  __shared__ float qsc[G];
  __shared__ float red[kWaves][G][D + 4];

  // ---- query: load, rotate, quantize -----------------------------------------------------
  const uint16_t* qp = p.q + ((int64_t)b * p.hq + qh0) * D;
  if constexpr (DT == 0) {
    for (int k = tid; k < G * 64; k += kThreads)
      qd[k >> 6][0][k & 63] = reinterpret_cast<const uint32_t*>(qp)[k];
    if (tid < G) qsc[tid] = p.softmax_scale * kLog2e;
    __syncthreads();
  } else {
    for (int k = tid; k < G * D; k += kThreads) qf[k >> 7][k & 127] = __uint_as_float((uint32_t)qp[k] << 16);
    fwht_lds<G>(qf, tid);
    constexpr float qimax = (DT == 8) ? kQiMax8 : kQiMax4;
    const int lane = tid & 63, wv = tid >> 6;
    for (int j = wv; j < G; j += kWaves) {
      const float a0 = qf[j][lane] * kRotC, a1 = qf[j][lane + 64] * kRotC;
      float am = fmaxf(fabsf(a0), fabsf(a1));
      for (int msk = 1; msk < 64; msk <<= 1) am = fmaxf(am, __shfl_xor(am, msk));
      const float inv = am > 0.f ? qimax / am : 0.f;
      // q integers, kept as floats (exact: |q| < 2^24)
      qf[j][lane] = rintf(a0 * inv);
      qf[j][lane + 64] = rintf(a1 * inv);
      if (lane == 0) qsc[j] = am > 0.f ? (am / qimax) * p.softmax_scale * kLog2e : 0.f;
    }
    __syncthreads();
    // pack digits: turbo4/3 -> dword i holds dims 8i..8i+7, one signed nibble each;
    // turbo8 -> dword i holds dims 4i..4i+3, one signed byte each
    for (int k = tid; k < G * F::kDig * F::kQtot; k += kThreads) {
      const int j = k / (F::kDig * F::kQtot);
      const int dg = (k / F::kQtot) % F::kDig;
      const int i = k % F::kQtot;
      uint32_t word = 0;
      if constexpr (DT == 8) {
        for (int e = 0; e < 4; ++e) {
          int q = (int)qf[j][4 * i + e];
          int dgt = 0;
          for (int t = 0; t <= dg; ++t) {
            dgt = ((q + 128) & 255) - 128;
            q = (q - dgt) >> 8;
          }
          word |= (uint32_t)(dgt & 0xff) << (8 * e);
        }
      } else {
        for (int e = 0; e < 8; ++e) {
          int q = (int)qf[j][8 * i + e];
          int dgt = 0;
          for (int t = 0; t <= dg; ++t) {
            dgt = ((q + 8) & 15) - 8;
            q = (q - dgt) >> 4;
          }
          word |= (uint32_t)(dgt & 0xf) << (4 * e);
        }
      }
      qd[j][dg][i] = word;
    }
    __syncthreads();
  }

  const int lane = tid & 63;
  const int t = lane >> 2, c = lane & 3;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint32_t qr[G][F::kDig][F::kQdw];
  float qs[G];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    qs[j] = qsc[j];
#pragma unroll
    for (int dg = 0; dg < F::kDig; ++dg)
#pragma unroll
      for (int i = 0; i < F::kQdw; ++i) qr[j][dg][i] = qd[j][dg][c * F::kQdw + i];
  }

  State<DT, G> st;
#pragma unroll
  for (int j = 0; j < G; ++j) {
    st.m[j] = -INFINITY;
    st.l[j] = 0.f;
    st.ws[j] = 0.f;
#pragma unroll
    for (int d = 0; d < 32; ++d) st.acc[j][d] = 0.f;
  }

  // ---- main loop: wave w takes 16-token steps w, w+4, ... ------------------------------
  const int nsteps = (tok_end - tok_begin + 15) >> 4;
  const int ps = p.page_size;
  const int64_t head_off = (int64_t)kvh * p.block_bytes;
  const int32_t* bt = p.block_tables + (int64_t)b * p.maxp;
  auto block_of = [&](int tok0, const uint8_t* pool) {
    const int phys = bt[tok0 >> p.page_shift];
    return pool + (int64_t)phys * p.page_stride + head_off;
  };
  int s = wave;
  if (s < nsteps) {
    Raw<DT> cur;
    int tok0 = tok_begin + (s << 4);
    load_raw<DT>(cur, block_of(tok0, p.k_pool), block_of(tok0, p.v_pool), (tok0 & (ps - 1)) + t, c, ps);
    for (; s < nsteps; s += kWaves) {
      Raw<DT> nxt;
      const int tok1 = tok0 + (kWaves << 4);
      const bool more = s + kWaves < nsteps;
      if (more)
        load_raw<DT>(nxt, block_of(tok1, p.k_pool), block_of(tok1, p.v_pool), (tok1 & (ps - 1)) + t, c, ps);
      process<DT, G>(cur, tok0 + t < tok_end, qr, qs, st);
      if (more) cur = nxt;
      tok0 = tok1;
    }
  }

  // ---- merge the 16 token lanes of each dim chunk ---------------------------------------
#pragma unroll
  for (int j = 0; j < G; ++j) {
    float mx = st.m[j];
#pragma unroll
    for (int msk = 4; msk < 64; msk <<= 1) mx = fmaxf(mx, __shfl_xor(mx, msk));
    const float f = (st.m[j] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(st.m[j] - mx);
    float l = st.l[j] * f;
    const float off = F::kOff * st.ws[j];
#pragma unroll
    for (int d = 0; d < 32; ++d) st.acc[j][d] = (st.acc[j][d] - off) * f;
#pragma unroll
    for (int msk = 4; msk < 64; msk <<= 1) {
      l += __shfl_xor(l, msk);
#pragma unroll
      for (int d = 0; d < 32; ++d) st.acc[j][d] += __shfl_xor(st.acc[j][d], msk);
    }
    if (t == 0) {
#pragma unroll
      for (int d = 0; d < 32; ++d) red[wave][j][32 * c + d] = st.acc[j][d];
      if (c == 0) {
        red[wave][j][D] = mx;
        red[wave][j][D + 1] = l;
      }
    }
  }
  __syncthreads();

  // ---- merge the 4 waves ------------------------------------------------------------------
  const bool single = nsplit_b == 1;
  for (int k = tid; k < G * D; k += kThreads) {
    const int j = k >> 7, d = k & 127;
    float mx = -INFINITY;
#pragma unroll
    for (int wv = 0; wv < kWaves; ++wv) mx = fmaxf(mx, red[wv][j][D]);
    float acc = 0.f, l = 0.f;
#pragma unroll
    for (int wv = 0; wv < kWaves; ++wv) {
      const float mw = red[wv][j][D];
      const float f = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - mx);
      acc += red[wv][j][d] * f;
      l += red[wv][j][D + 1] * f;
    }
    if (single) {
      qf[j][d] = acc / l;
    } else {
      float* part = p.partials + (((int64_t)b * p.hq + qh0 + j) * p.nsplits + split) * kPartialStride;
      part[4 + d] = acc;
      if (d == 0) {
        part[0] = mx;
        part[1] = l;
      }
    }
  }
  if (!single) return;
  if constexpr (DT != 0) {
    fwht_lds<G>(qf, tid);
    for (int k = tid; k < G * D; k += kThreads) outp[k] = qf[k >> 7][k & 127] * kRotC;
  } else {
    __syncthreads();
    for (int k = tid; k < G * D; k += kThreads) outp[k] = qf[k >> 7][k & 127];
  }
}

// Merge split partials of one (sequence, q head) and rotate back. 128 threads, one per dim.
template <int DT>
__global__ __launch_bounds__(128) void decode_combine_kernel(DecodeParams p) {
  const int qh = blockIdx.x, b = blockIdx.y;
  const int d = threadIdx.x;
  const int L = min(p.context_lens[b], p.max_context_len);
  const int nsplit_b = (L + p.tokens_per_split - 1) / p.tokens_per_split;
  if (nsplit_b <= 1) return;  // written by the split kernel
  const float* part = p.partials + ((int64_t)b * p.hq + qh) * p.nsplits * kPartialStride;
  float mx = -INFINITY;
  for (int s = 0; s < nsplit_b; ++s) mx = fmaxf(mx, part[s * kPartialStride]);
  float acc = 0.f, l = 0.f;
  for (int s = 0; s < nsplit_b; ++s) {
    const float ms = part[s * kPartialStride];
    const float f = (ms == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms - mx);
    acc += part[s * kPartialStride + 4 + d] * f;
    l += part[s * kPartialStride + 1] * f;
  }
  __shared__ float o[D];
  o[d] = acc / l;
  float* outp = p.out + ((int64_t)b * p.hq + qh) * D;
  if constexpr (DT != 0) {
    for (int h = 1; h < D; h <<= 1) {
      __syncthreads();
      float a = 0.f, c = 0.f;
      const bool lower = (d & h) == 0;
      if (lower) { a = o[d]; c = o[d + h]; }
      __syncthreads();
      if (lower) { o[d] = a + c; o[d + h] = a - c; }
    }
    __syncthreads();
    outp[d] = o[d] * kRotC;
  } else {
    outp[d] = o[d];
  }
}

template <int DT, int G>
hipError_t launch_g(const DecodeParams& p, hipStream_t stream) {
  dim3 grid(p.nsplits, p.hkv, p.batch);
  hipLaunchKernelGGL((decode_split_kernel<DT, G>), grid, dim3(kThreads), 0, stream, p);
  if (p.nsplits > 1) {
    hipLaunchKernelGGL((decode_combine_kernel<DT>), dim3(p.hq, p.batch), dim3(128), 0, stream, p);
  }
  return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(int g, const DecodeParams& p, hipStream_t stream) {
  switch (g) {
    case 1: return launch_g<DT, 1>(p, stream);
    case 2: return launch_g<DT, 2>(p, stream);
    case 3: return launch_g<DT, 3>(p, stream);
    case 4: return launch_g<DT, 4>(p, stream);
    case 5: return launch_g<DT, 5>(p, stream);
    case 6: return launch_g<DT, 6>(p, stream);
    case 7: return launch_g<DT, 7>(p, stream);
    case 8: return launch_g<DT, 8>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(int dtype, int group, const DecodeParams& p, hipStream_t stream) {
  switch (dtype) {
    case 0: return launch_dt<0>(group, p, stream);
    case 8: return launch_dt<8>(group, p, stream);
    case 4: return launch_dt<4>(group, p, stream);
    case 3: return launch_dt<3>(group, p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace xq
