"""GPU parity of multi-query decode (next_n query tokens per request, each
with its causal length) against the oracle's single-query rows."""
import numpy as np
import pytest
import torch

from top_sparse_decode_amd import api, synth

from parity_util import assert_outputs_close, oracle_run, out_to_numpy

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def say(*a):
    print(*a, flush=True)


def check(w, precision, reqs=None, what=""):
    say(f"[mq] {what} next_n={w.next_n} B={w.batch} precision={precision}")
    step = api.prepare(w, precision=precision)
    step.run()
    torch.cuda.synchronize()
    ref = oracle_run(w, reqs)
    n = w.next_n
    rows = slice(None) if reqs is None else [b * n + j for b in reqs for j in range(n)]
    assert np.array_equal(step.indices.cpu().numpy()[rows], ref["indices"]), f"{what}: indices differ"
    assert np.array_equal(step.counts.cpu().numpy()[rows], ref["counts"]), f"{what}: counts differ"
    return assert_outputs_close(out_to_numpy(step.out)[rows], ref["out"], w.out_dtype, what), step


@pytest.mark.parametrize("next_n", [2, 4])
@pytest.mark.parametrize("precision", [api.EXACT, api.FAST])
def test_mq_small(next_n, precision):
    w = synth.make_workload(4, batch=3, kv_len=[9000, 2050, 3], topk=2048, next_n=next_n)
    check(w, precision, what="dsa")


def test_mq_fp8_and_small_pages():
    w = synth.make_workload(4, batch=2, kv_len=[5000, 1500], topk=512, idx_heads=16, page_size=16,
                            next_n=3, index_dtype="fp8")
    check(w, api.FAST, what="fp8 h16 p16")


def test_mq_mixed_lengths():
    w = synth.make_workload(5, batch=3, min_len=2000, max_len=9000, topk=2048, next_n=2)
    check(w, api.FAST, what="mixed")


def test_mq_with_hint_writeback():
    w = synth.make_workload(4, batch=2, kv_len=[7000, 4000], topk=1024, next_n=2)
    ref = oracle_run(w)
    step = api.prepare(w, precision=api.FAST, hint=True)
    for it in range(2):
        step.run()
        torch.cuda.synchronize()
        assert np.array_equal(step.indices.cpu().numpy(), ref["indices"])
        assert torch.equal(step.hint, step.indices)


def test_mq_full_dsa_all_requests():
    w = synth.make_workload(4, next_n=2)
    worst, step = check(w, api.FAST, what="DSA-MLA 16 x 64K next_n 2 (all requests)")
    say(f"DSA-MLA 16 x 64K next_n 2: worst row rel-L2 {worst:.3e}")
    assert torch.isfinite(step.out.float()).all()
