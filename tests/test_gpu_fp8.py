"""GPU parity of the FP8 E4M3 indexer cache (one binary32 scale per row)
against the CPU oracle: exact scores bit for bit, fast scores within their
reported bound, fused indices bit for bit and outputs within tolerance."""
import numpy as np
import pytest
import torch

import oracle
from top_sparse_decode_amd import api, synth

from parity_util import assert_outputs_close, oracle_run, out_to_numpy

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def say(*a):
    print(*a, flush=True)


SMALL = {
    "dsa_fp8": (4, dict(batch=2, kv_len=[9000, 4100], topk=2048)),
    "dsa_fp8_short": (4, dict(batch=3, kv_len=[1, 100, 2047], topk=2048)),
    "dsa_fp8_mixed": (5, dict(batch=3, min_len=2000, max_len=9000, topk=2048)),
    "dsa_fp8_h16_p16": (4, dict(batch=3, kv_len=[3000, 1500, 17], topk=512, idx_heads=16, page_size=16)),
    "dsa_fp8_h32_p32": (4, dict(batch=2, kv_len=[7000, 33], topk=1024, idx_heads=32, page_size=32)),
}


def make(name):
    cfg, kw = SMALL[name]
    return synth.make_workload(cfg, index_dtype="fp8", **kw)


def scores_on_gpu(w, precision):
    step = api.prepare(w, precision=precision)
    groups = w.score_k.shape[1]
    scores = torch.empty((w.batch, groups, w.max_kv_len), dtype=torch.float32, device="cuda")
    bound = torch.zeros((w.batch, groups), dtype=torch.float32, device="cuda")
    api.sparse_score_paged(step.args.pages, step.args.score_k, step.score_q, w.score_q.shape[1],
                           step.head_weights, api.MODES[w.mode], w.head_scale, precision, scores, bound)
    torch.cuda.synchronize()
    return scores.cpu().numpy(), bound.cpu().numpy()


def oracle_scores(w):
    return oracle.score(w.block_table, w.kv_lens, w.score_k, w.score_q, w.head_weights, w.mode,
                        w.head_scale, w.max_kv_len, w.score_k_scale)


def format_cap(w, b):
    """A rounding-level ceiling for the reported bound: 1e-4 of the largest
    value the row's inputs allow, 448 max|sigma| sum_h |w_h| sum_d |q_hd|."""
    P = w.page_size
    L = int(w.kv_lens[b])
    t = np.arange(L)
    sig = np.abs(w.score_k_scale[w.block_table[b, t // P], 0, t % P]).max()
    q = synth.bf16_bits_to_f32(w.score_q[b]).astype(np.float64)
    return 1e-4 * 448.0 * sig * float(np.abs(w.head_weights[b]) @ np.abs(q).sum(axis=1))


def assert_within_bound(w, got, d, ref):
    for b in range(w.batch):
        L = int(w.kv_lens[b])
        err = np.abs(got[b, 0, :L].astype(np.float64) - ref[b, 0, :L])
        assert np.all(err <= d[b, 0]), (b, float(err.max()), float(d[b, 0]))
        assert np.all(got[b, 0, L:] == -np.inf)
        if L:
            # a rounding-level quantity, not a loose one
            assert d[b, 0] <= format_cap(w, b), (b, float(d[b, 0]), format_cap(w, b))


@pytest.mark.parametrize("name", list(SMALL))
def test_fp8_exact_scores_bitwise(name):
    w = make(name)
    say(f"[fp8 exact scores] {name}")
    got, d = scores_on_gpu(w, api.EXACT)
    ref = oracle_scores(w)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert np.all(d == 0)


@pytest.mark.parametrize("name", list(SMALL))
def test_fp8_fast_scores_within_bound(name):
    w = make(name)
    say(f"[fp8 fast scores] {name}")
    got, d = scores_on_gpu(w, api.FAST)
    assert_within_bound(w, got, d, oracle_scores(w))


def every_code_workload(idx_heads):
    """Token t of 254 holds the t-th non-NaN E4M3 code in all 128 dims, with
    a row scale that is a power of two on even tokens and 0.3 on odd ones;
    half the query heads are +1, half -1, all weights 1/H.  Every code meets
    both signs, so no code hides behind the ReLU."""
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    n = codes.size
    w = synth.make_workload(4, batch=1, kv_len=n, topk=64, idx_heads=idx_heads, index_dtype="fp8")
    P = w.page_size
    for t in range(n):
        pg, sl = w.block_table[0, t // P], t % P
        w.score_k[pg, 0, sl, :] = codes[t]
        w.score_k_scale[pg, 0, sl] = np.float32(2.0 ** ((t % 9) - 4)) if t % 2 == 0 else np.float32(0.3)
    q = np.full((1, idx_heads, 128), 0x3F80, np.uint16)        # bf16 +1
    q[:, idx_heads // 2:, :] = 0xBF80                            # bf16 -1
    w.score_q[...] = q
    w.head_weights[...] = np.float32(1.0 / idx_heads)
    return w


@pytest.mark.parametrize("idx_heads", [16, 64])
def test_fp8_every_code(idx_heads):
    w = every_code_workload(idx_heads)
    say(f"[fp8 every code] heads={idx_heads}")
    ref = oracle_scores(w)
    got, _ = scores_on_gpu(w, api.EXACT)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    got, d = scores_on_gpu(w, api.FAST)
    assert_within_bound(w, got, d, ref)
    # power-of-two scales: every step is exact, so the fast score is too
    L = int(w.kv_lens[0])
    even = np.arange(0, L, 2)
    assert np.array_equal(got[0, 0, even], ref[0, 0, even])


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("precision", [api.EXACT, api.FAST])
def test_fp8_fused_small(name, precision):
    w = make(name)
    say(f"[fp8 fused] {name} precision={precision}")
    step = api.prepare(w, precision=precision)
    step.run()
    torch.cuda.synchronize()
    ref = oracle_run(w)
    assert np.array_equal(step.indices.cpu().numpy(), ref["indices"]), "indices differ"
    assert np.array_equal(step.counts.cpu().numpy(), ref["counts"]), "counts differ"
    assert_outputs_close(out_to_numpy(step.out), ref["out"], w.out_dtype, name)


def test_fp8_band_overflow_falls_back_exactly():
    # one request whose indexer rows are all the same codes and scale: every
    # score ties, the band overflows and the single-block fallback re-scores
    # in the exact order
    w = synth.make_workload(4, batch=2, kv_len=[6000, 5000], topk=2048, index_dtype="fp8")
    P = w.page_size
    pg0 = w.block_table[0, 0]
    row0, sc0 = w.score_k[pg0, 0, 0].copy(), w.score_k_scale[pg0, 0, 0]
    for t in range(6000):
        pg, sl = w.block_table[0, t // P], t % P
        w.score_k[pg, 0, sl] = row0
        w.score_k_scale[pg, 0, sl] = sc0
    say("[fp8 band overflow]")
    step = api.prepare(w, precision=api.FAST)
    step.run()
    torch.cuda.synchronize()
    ref = oracle_run(w)
    assert np.array_equal(step.indices.cpu().numpy(), ref["indices"])
    assert_outputs_close(out_to_numpy(step.out), ref["out"], w.out_dtype, "fp8 band overflow")


def test_fp8_full_dsa_all_requests():
    w = synth.make_workload(4, index_dtype="fp8")
    say("[fp8 DSA-MLA 16 x 64K, all requests]")
    step = api.prepare(w, precision=api.FAST)
    step.run()
    torch.cuda.synchronize()
    ref = oracle_run(w)
    assert np.array_equal(step.indices.cpu().numpy(), ref["indices"])
    assert np.array_equal(step.counts.cpu().numpy(), ref["counts"])
    worst = assert_outputs_close(out_to_numpy(step.out), ref["out"], w.out_dtype, "fp8 DSA-MLA 16 x 64K")
    say(f"fp8 DSA-MLA 16 x 64K: worst row rel-L2 {worst:.3e}")
