"""Seeded synthetic decode workloads for the TurboQuant paged KV cache.

This module only draws inputs: query/key/value rows as bf16 bit patterns, context
lengths and page tables. It holds none of the method's arithmetic, and it is the one
thing both the oracle (oracle/) and the HIP library (bit_quantized_paged_turbo_amd/)
are fed from, through the tests and bench.py.

The five presets stand in for the workloads the pages measure on model runs; real
activations would need trained weights, so K/V/Q are N(0,1) draws with the structure
listed per preset (outlier channels in K, a slow drift in the mean, length mixes).

Randomness: numpy PCG64 streams keyed by SeedSequence([20261202, cfg, stream, *extra]).
Streams: 0 context lengths, 1 page permutation, 2 outlier channels, 3 Q,
4 K (extra = sequence index), 5 V (extra = sequence index), 6/7 K/V of an appended chunk.
Values are drawn in fp32, shaped (outliers, drift), then rounded once to bf16 (RNE).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

SEED = 20261202
HEAD_DIM = 128

BF16 = 0
TURBO8 = 8
TURBO4 = 4
TURBO3 = 3
TURBO2 = 2
FP8 = 16        # OCP FP8 E4M3 elements, no rotation, no scale
DTYPE_NAMES = {BF16: "bf16", TURBO8: "turbo8", TURBO4: "turbo4", TURBO3: "turbo3", TURBO2: "turbo2",
               FP8: "fp8"}


def rng(cfg: int, stream: int, *extra: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED, cfg, stream, *extra])))


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns with round-half-even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


@dataclass
class Workload:
    """One decode-attention workload (one layer).

    Sequences 0..batch-1 are decoded. When `chunk_tokens` > 0 an extra sequence (index
    `batch`) receives a freshly prefilled chunk of that many tokens in the same step.
    """
    name: str
    cfg: int
    dtype: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    page_size: int
    context_lens: np.ndarray            # int32 [batch]
    num_pages: int
    block_tables: np.ndarray            # int32 [num_seqs][max_pages_per_seq]
    outlier_channels: int = 4
    outlier_scale: float = 20.0
    drift_amplitude: float = 0.0
    drift_period: int = 262144
    num_splits: int = 0
    chunk_tokens: int = 0
    note: str = ""
    _outliers: np.ndarray | None = field(default=None, repr=False)

    # -- shape helpers --------------------------------------------------------------
    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(HEAD_DIM)

    @property
    def max_pages_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.batch else 0

    @property
    def num_seqs(self) -> int:
        return int(self.block_tables.shape[0])

    def seq_len(self, b: int) -> int:
        return self.chunk_tokens if b == self.batch else int(self.context_lens[b])

    # -- draws ------------------------------------------------------------------------
    def outliers(self) -> np.ndarray:
        """Distinct outlier channels per kv head, int [Hkv, outlier_channels]."""
        if self._outliers is None:
            g = rng(self.cfg, 2)
            self._outliers = np.stack([
                np.sort(g.choice(HEAD_DIM, size=self.outlier_channels, replace=False))
                for _ in range(self.num_kv_heads)]) if self.outlier_channels else \
                np.zeros((self.num_kv_heads, 0), dtype=np.int64)
        return self._outliers

    def q_bits(self) -> np.ndarray:
        """Queries, bf16 bits [batch, Hq, 128]."""
        x = rng(self.cfg, 3).standard_normal((self.batch, self.num_q_heads, HEAD_DIM),
                                             dtype=np.float32)
        return round_to_bf16_bits(x)

    def _rows(self, stream: int, b: int, n: int, is_k: bool, t0: int = 0) -> np.ndarray:
        x = rng(self.cfg, stream, b).standard_normal((n, self.num_kv_heads, HEAD_DIM),
                                                     dtype=np.float32)
        if is_k and self.outlier_channels:
            ch = self.outliers()
            for h in range(self.num_kv_heads):
                x[:, h, ch[h]] *= np.float32(self.outlier_scale)
        if self.drift_amplitude:
            t = np.arange(t0, t0 + n, dtype=np.float64)
            d = (self.drift_amplitude * np.sin(2.0 * np.pi * t / self.drift_period))
            x += d.astype(np.float32)[:, None, None]
        return round_to_bf16_bits(x)

    def kv_bits(self, b: int):
        """K and V rows of sequence b, bf16 bits [L_b, Hkv, 128] each (positions 0..L_b-1)."""
        n = self.seq_len(b)
        if b == self.batch:
            return self._rows(6, b, n, True), self._rows(7, b, n, False)
        return self._rows(4, b, n, True), self._rows(5, b, n, False)

    def total_tokens(self) -> int:
        return int(self.context_lens.sum())


# ------------------------------------------------------------------------------------
# page tables
# ------------------------------------------------------------------------------------
def _assign_pages(seq_lens, page_size, num_pages, order):
    """Block tables giving each sequence's logical pages the next physical pages of `order`."""
    pages = [max(1, -(-int(n) // page_size)) if n > 0 else 0 for n in seq_lens]
    maxp = max(1, max(pages) if pages else 1)
    bt = np.zeros((len(seq_lens), maxp), dtype=np.int32)
    k = 0
    for s, n in enumerate(pages):
        bt[s, :n] = order[k:k + n]
        k += n
    if k > num_pages:
        raise ValueError("pool too small")
    return bt


def make(name: str, cfg: int, dtype: int, context_lens, num_q_heads: int,
         num_kv_heads: int, page_size: int, *, permute: bool = True,
         pool_pages: int | None = None, chunk_tokens: int = 0, **kw) -> Workload:
    context_lens = np.asarray(context_lens, dtype=np.int32)
    seq_lens = list(context_lens) + ([chunk_tokens] if chunk_tokens else [])
    needed = sum(-(-int(n) // page_size) for n in seq_lens)
    num_pages = max(1, pool_pages if pool_pages is not None else needed)
    order = rng(cfg, 1).permutation(num_pages) if permute else np.arange(num_pages)
    bt = _assign_pages(seq_lens, page_size, num_pages, order)
    return Workload(name=name, cfg=cfg, dtype=dtype, batch=len(context_lens),
                    num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                    page_size=page_size, context_lens=context_lens, num_pages=num_pages,
                    block_tables=bt, chunk_tokens=chunk_tokens, **kw)


# ------------------------------------------------------------------------------------
# the five presets
# ------------------------------------------------------------------------------------
def c1_context_lens(batch: int = 256) -> np.ndarray:
    return rng(1, 0).integers(64, 1024, size=batch, endpoint=True).astype(np.int32)


def c4_context_lens(batch: int = 64) -> np.ndarray:
    u = rng(4, 0).uniform(math.log(1024), math.log(32768), size=batch)
    return np.floor(np.exp(u)).astype(np.int32)


def config(i: int, dtype: int | None = None, batch: int | None = None,
           context_scale: float = 1.0) -> Workload:
    """Preset i (0..4). `batch` and `context_scale` shrink it for quick parity runs while
    keeping head counts, page size, dtype and value distributions."""
    def scaled(lens):
        lens = np.asarray(lens)
        return np.maximum(1, np.floor(lens * context_scale)).astype(np.int32)

    if i == 0:
        return make("tiny-gqa4-turbo4", 0, TURBO4 if dtype is None else dtype,
                    scaled([256] * (batch or 1)), 8, 2, 16,
                    note="B=1, 8q/2kv, ctx 256, ps 16, permuted pages, K outliers 4x20")
    if i == 1:
        lens = c1_context_lens()[: (batch or 256)]
        return make("batched-16q8kv-turbo4", 1, TURBO4 if dtype is None else dtype,
                    scaled(lens), 16, 8, 16,
                    note="B=256, 16q/8kv, ctx U[64,1024], ps 16, permuted pages")
    if i == 2:
        return make("8b-32q8kv-ctx8192", 2, TURBO8 if dtype is None else dtype,
                    scaled([8192] * (batch or 32)), 32, 8, 16, permute=False,
                    outlier_channels=8, outlier_scale=30.0,
                    note="B=32, 32q/8kv, ctx 8192, ps 16, K outliers 8x30; turbo8 and bf16")
    if i == 3:
        return make("longctx-40q8kv-turbo3", 3, TURBO3 if dtype is None else dtype,
                    scaled([262144] * (batch or 1)), 40, 8, 64, permute=False,
                    drift_amplitude=0.5, num_splits=256,
                    note="B=1, 40q/8kv, ctx 262144, ps 64, 256 splits, drift 0.5 sin")
    if i == 4:
        lens = c4_context_lens()[: (batch or 64)]
        pool = 131072 if context_scale == 1.0 and batch is None else None
        return make("mixed-32q8kv-turbo4", 4, TURBO4 if dtype is None else dtype,
                    scaled(lens), 32, 8, 16, pool_pages=pool,
                    chunk_tokens=max(16, int(2048 * context_scale)),
                    note="chunk append 2048 + decode B=64, ctx logU[1024,32768], ps 16, "
                         "pages shuffled over a 2M-token pool")
    raise ValueError(f"no preset {i}")
