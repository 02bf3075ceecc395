"""Seeded input generator: determinism, structure of each workload family."""
import numpy as np
import pytest

from top_sparse_decode_amd import synth


def test_same_seed_same_bits_other_seed_differs():
    a = synth.make_workload(2, batch=2, kv_len=200)
    b = synth.make_workload(2, batch=2, kv_len=200)
    c = synth.make_workload(2, seed=99, batch=2, kv_len=200)
    for x, y in ((a.k, b.k), (a.q, b.q), (a.block_table, b.block_table)):
        assert np.array_equal(x, y)
    assert not np.array_equal(a.q, c.q)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5], np.float32)
    got = synth.bf16_bits_to_f32(synth.to_bf16_bits(x))
    # 1+2^-8 is a tie between 1 and 1+2^-7 -> even (1); 1+3*2^-8 -> 1+2^-6 (even)
    assert got.tolist() == [1.0, 1.0, 1.0 + 2 ** -6, 1.0, -2.5]


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_block_table_is_a_page_permutation(cfg):
    kw = {1: {}, 2: dict(batch=2), 3: dict(batch=2, kv_len=700), 4: dict(batch=2, kv_len=300)}[cfg]
    w = synth.make_workload(cfg, **kw)
    P = w.page_size
    used = []
    for b in range(w.batch):
        n = (int(w.kv_lens[b]) + P - 1) // P
        used += list(w.block_table[b, :n])
        assert np.all(w.block_table[b, n:] == -1)
    assert len(set(used)) == len(used)
    assert min(used) >= 0 and max(used) < w.num_pages


def test_mixed_lengths_pool_has_slack_and_canaries():
    w = synth.make_workload(5, batch=6, min_len=70, max_len=900, idx_heads=4, heads=2)
    P = w.page_size
    need = sum((int(L) + P - 1) // P for L in w.kv_lens)
    assert w.num_pages == int(np.ceil(1.25 * need))
    assert np.all((w.kv_lens >= 70) & (w.kv_lens <= 900))
    lat = synth.bf16_bits_to_f32(w.k)
    for b in range(w.batch):
        L = int(w.kv_lens[b])
        last = w.block_table[b, (L - 1) // P]
        assert np.all(np.isfinite(lat[last, 0, (L - 1) % P]))
        if L % P:
            assert np.all(np.isnan(lat[last, 0, L % P:]))


def test_mixed_lengths_key_bias_fraction():
    w = synth.make_workload(5, batch=2, kv_lens=[6000, 5000], idx_heads=4, heads=2)
    ki = synth.bf16_bits_to_f32(w.score_k)
    P = w.page_size
    biased = 0
    total = 0
    for b in range(2):
        for t in range(int(w.kv_lens[b])):
            row = ki[w.block_table[b, t // P], 0, t % P]
            biased += row.mean() > 2.0
            total += 1
    assert 0.006 < biased / total < 0.014


def test_tiny_heavy_tokens_are_shifted_along_query_sum():
    w = synth.make_workload(1)
    plain = synth.make_workload(1, heavy=0)
    diff = (w.k.astype(np.float64) - plain.k).reshape(-1, 64)
    moved = np.nonzero(np.abs(diff).max(axis=1) > 0)[0]
    assert len(moved) == 8
    qbar = w.q[0].astype(np.float64).sum(axis=0)
    shift = 3 * qbar / np.linalg.norm(qbar)
    for r in moved:
        np.testing.assert_allclose(diff[r], shift, atol=1e-5)
