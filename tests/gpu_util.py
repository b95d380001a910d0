"""Glue between the seeded workloads, the HIP library (through its C ABI) and the oracle.

Moves numpy inputs to the GPU, fills caches through xq_quantize_append and reads pool
bytes back for comparison. Holds no arithmetic of the method.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads
from bit_quantized_paged_turbo_amd.cache import PagedKVCache


def to_dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:                      # bf16 bit patterns
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def make_cache(W: workloads.Workload, fill_byte: int | None = 0xFF) -> PagedKVCache:
    return PagedKVCache(W.dtype, W.num_kv_heads, W.page_size, W.num_pages, fill_byte=fill_byte)


def upload_tables(W: workloads.Workload):
    bt = to_dev(W.block_tables.astype(np.int32))
    cl = to_dev(W.context_lens.astype(np.int32))
    return bt, cl


def fill(cache: PagedKVCache, W: workloads.Workload, bt: torch.Tensor, seqs=None,
         max_rows: int = 1 << 20, kv=None, last=None):
    """Append every position of the given sequences (default: all, incl. a chunk sequence).
    `kv` optionally maps seq -> (k_bits, v_bits) already drawn; `last`, a dict, receives each
    sequence's last K and V rows (seq -> (k_row, v_row))."""
    seqs = range(W.num_seqs) if seqs is None else seqs
    pend_k, pend_v, pend_s, pend_p, n = [], [], [], [], 0

    def flush():
        nonlocal pend_k, pend_v, pend_s, pend_p, n
        if not n:
            return
        k = to_dev(np.concatenate(pend_k))
        v = to_dev(np.concatenate(pend_v))
        s = to_dev(np.concatenate(pend_s).astype(np.int32))
        p = to_dev(np.concatenate(pend_p).astype(np.int32))
        cache.append(k, v, s, p, bt)
        pend_k, pend_v, pend_s, pend_p, n = [], [], [], [], 0

    for b in seqs:
        L = W.seq_len(b)
        if L == 0:
            continue
        k, v = kv[b] if kv is not None and b in kv else W.kv_bits(b)
        if last is not None:
            last[b] = (k[-1].copy(), v[-1].copy())
        pend_k.append(k)
        pend_v.append(v)
        pend_s.append(np.full(L, b, np.int32))
        pend_p.append(np.arange(L, dtype=np.int32))
        n += L
        if n >= max_rows:
            flush()
    flush()


def gather(pool: np.ndarray, W: workloads.Workload, block_bytes: int, b: int, positions):
    """Read (code bytes [n, Hkv, rowb], scale bits [n, Hkv]) of sequence b out of a pool."""
    ps, hkv = W.page_size, W.num_kv_heads
    rowb = 256 if W.dtype == 0 else 128 if W.dtype == workloads.FP8 else 16 * W.dtype
    blocks = pool.reshape(W.num_pages, hkv, block_bytes)
    positions = np.asarray(positions)
    pages = W.block_tables[b, positions // ps]
    slots = positions % ps
    codes = np.stack([blocks[pages, h][np.arange(len(positions))[:, None],
                                      slots[:, None] * rowb + np.arange(rowb)[None, :]]
                      for h in range(hkv)], axis=1)
    if W.dtype in (0, workloads.FP8):
        return codes, None
    sc = np.stack([blocks[pages, h][np.arange(len(positions))[:, None],
                                   ps * rowb + 2 * slots[:, None] + np.arange(2)[None, :]]
                   for h in range(hkv)], axis=1)
    scales = sc[..., 0].astype(np.uint16) | (sc[..., 1].astype(np.uint16) << 8)
    return codes, scales


def hadamard_sign_rows(ks) -> np.ndarray:
    """Rows k of the unnormalised Sylvester sign pattern, (-1)^popcount(i & k) over i < 128: a
    query shaped like this rotates to a multiple of one basis vector (test input only)."""
    i = np.arange(128)
    par = np.zeros((len(ks), 128), np.int64)
    x = np.asarray(ks)[:, None] & i[None, :]
    while np.any(x):
        par ^= x & 1
        x >>= 1
    return np.where(par == 1, -1.0, 1.0)


def dominant_queries(qb: np.ndarray, kind, seed: int) -> np.ndarray:
    """Queries whose rotation has one dominant element: the draw plus a constant (which rotates
    to offset * sqrt(128) on element 0), or a signed Hadamard row plus N(0, 0.3^2) noise (which
    rotates to +-sqrt(128) on another element). bf16 bits of qb's shape."""
    q = oracle.bf16_bits_to_f32(qb)
    if kind == "had":
        r = np.random.default_rng(seed)
        rows = hadamard_sign_rows(r.integers(0, 128, size=q.shape[:-1]).reshape(-1))
        sign = r.choice([-1.0, 1.0], size=(rows.shape[0], 1))
        q = (sign * rows).reshape(q.shape) + 0.3 * r.standard_normal(q.shape)
    else:
        q = q + np.float32(kind)
    return workloads.round_to_bf16_bits(q.astype(np.float32))
