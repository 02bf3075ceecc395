"""The allocation-free fused step (sd_sparse_decode_noalloc) against the
fused step with a caller workspace (sd_sparse_decode), through the C ABI on
the same inputs: two calls in a row, the second with a smaller input, so the
second runs on scratch that still holds the first call's contents."""
import numpy as np
import pytest
import torch

from top_sparse_decode_amd import api, synth

from parity_util import assert_outputs_close, out_to_numpy

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def say(*a):
    print(*a, flush=True)


def both(w, precision):
    """(indices, counts, out) from sd_sparse_decode and from the no-alloc call."""
    step = api.prepare(w, precision=precision)
    step.run()
    torch.cuda.synchronize()
    ref = (step.indices.clone(), step.counts.clone(), step.out.clone())
    # clobber the outputs, then the same step on the library's scratch
    step.indices.fill_(-7)
    step.counts.fill_(-7)
    step.out.fill_(float("nan"))
    api.sparse_decode_noalloc(step.args)
    torch.cuda.synchronize()
    return ref, (step.indices, step.counts, step.out), step


@pytest.mark.parametrize("precision", [api.FAST, api.EXACT])
def test_noalloc_matches_workspace_entry_point(precision):
    cap = api.sparse_decode_noalloc_max_bytes()
    cases = [
        # DSA-MLA shapes (8 requests of 64K), then a smaller call
        synth.make_workload(4, batch=8, kv_len=[65536, 40000, 65536, 9000, 30000, 65536, 2047, 50000]),
        synth.make_workload(4, batch=3, kv_len=[5000, 100, 4100], topk=512, idx_heads=32, heads=64),
    ]
    for i, w in enumerate(cases):
        need = api.sparse_decode_workspace_size(api.prepare(w, precision=precision).args)
        say(f"[noalloc] call {i} {w.name} B={w.batch} precision={precision} workspace {need} of {cap}")
        assert need <= cap
        (ri, rc, ro), (gi, gc, go), step = both(w, precision)
        # the same kernels on the same inputs: identical indices and counts,
        # outputs within the bf16 tolerance of each other (and in fact equal)
        assert torch.equal(gi, ri), f"call {i}: indices differ"
        assert torch.equal(gc, rc), f"call {i}: counts differ"
        assert_outputs_close(out_to_numpy(go), out_to_numpy(ro).astype(np.float64), w.out_dtype, f"call {i}")
        assert torch.equal(go.view(torch.int16), ro.view(torch.int16)), f"call {i}: output bits differ"
