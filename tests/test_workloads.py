"""The seeded generators are deterministic and have the preset shapes (CPU only)."""
import numpy as np

import workloads


def test_presets_shapes_and_sums():
    c1 = workloads.config(1)
    assert c1.batch == 256 and c1.total_tokens() == 139593
    assert c1.context_lens.min() >= 64 and c1.context_lens.max() <= 1024
    c4 = workloads.config(4)
    assert c4.batch == 64 and c4.total_tokens() == 589302 and c4.num_pages == 131072
    assert c4.num_seqs == 65 and c4.chunk_tokens == 2048
    c3 = workloads.config(3)
    assert c3.page_size == 64 and c3.num_splits == 256 and c3.group == 5


def test_page_tables_are_injective():
    for i in (0, 1, 4):
        W = workloads.config(i)
        used = np.concatenate([W.block_tables[s, : -(-W.seq_len(s) // W.page_size)]
                               for s in range(W.num_seqs)])
        assert len(np.unique(used)) == len(used)
        assert used.max() < W.num_pages


def test_draws_are_deterministic():
    W = workloads.config(0)
    a, b = W.kv_bits(0), W.kv_bits(0)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert np.array_equal(W.q_bits(), workloads.config(0).q_bits())


def test_bf16_rounding_is_half_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5], np.float32)
    assert list(workloads.round_to_bf16_bits(x)) == [0x3F80, 0x3F80, 0x3F82, 0xC020]
