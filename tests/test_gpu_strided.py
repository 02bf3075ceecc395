"""GPU parity with pools that are not densely packed: every token row padded
(token stride > head_dim) and the pages interleaved with unused ones (page
stride = twice the page's size), the padding filled with NaN / NaN codes so
that any read of it spoils the result.  The page-table resolution of every
kernel (exact and fast scorers, selection re-score, vector and MLA attention)
goes through the strides; results must equal the oracle's on the packed
logical pool.  Also: exact scores for row sizes that are not staged through
LDS (512-byte f32 rows, 64-byte bf16 rows)."""
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


def strided_copy(t):
    """The same logical pool [pages, heads, page_size, dim] inside a buffer
    with 16 bytes of padding after every row and an unused page after every
    page; padding holds NaN (floats) or the NaN code 0x7F (fp8)."""
    P, H, S, D = t.shape
    pad = 16 // t.element_size()
    big = torch.empty((2 * P, H, S, D + pad), dtype=t.dtype, device=t.device)
    if t.dtype == torch.uint8:
        big.fill_(0x7F)
    else:
        big.fill_(float("nan"))
    view = big[::2, :, :, :D]
    view.copy_(t)
    assert view.stride(2) == D + pad and view.stride(0) == 2 * H * S * (D + pad)
    return big, view


def restride(step):
    """Point the step's pools at strided copies (kept alive on the step)."""
    keep = []
    a = step.args
    bk, vk = strided_copy(step.k)
    keep.append(bk)
    a.k = api.pool(vk)
    if step.v is step.k:
        a.v = a.k
    else:
        bv, vv = strided_copy(step.v)
        keep.append(bv)
        a.v = api.pool(vv)
    if step.score_k is step.k:
        a.score_k = a.k
    else:
        bs, vs = strided_copy(step.score_k)
        keep.append(bs)
        a.score_k = api.pool(vs, step.score_k_scale)
    step.keep = keep
    return step


CASES = {
    "tiny_f32": (1, dict(batch=2, kv_len=[1000, 300], topk=128), {}),
    "mha_bf16": (2, dict(batch=2, kv_len=[1024, 700], topk=408), {}),
    "gqa_bf16": (3, dict(batch=2, kv_len=[3000, 2049], topk=2048), {}),
    "dsa": (4, dict(batch=2, kv_len=[9000, 4100], topk=2048), {}),
    "dsa_fp8": (4, dict(batch=2, kv_len=[7000, 3000], topk=1024), dict(index_dtype="fp8")),
}


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("precision", [api.EXACT, api.FAST])
def test_fused_strided_pools(name, precision):
    cfg, kw, extra = CASES[name]
    w = synth.make_workload(cfg, **kw, **extra)
    say(f"[strided fused] {name} precision={precision}")
    step = restride(api.prepare(w, precision=precision))
    step.run()
    torch.cuda.synchronize()
    ref = oracle_run(w)
    assert np.array_equal(step.indices.cpu().numpy(), ref["indices"]), "indices differ"
    assert np.array_equal(step.counts.cpu().numpy(), ref["counts"]), "counts differ"
    assert_outputs_close(out_to_numpy(step.out), ref["out"], w.out_dtype, name)


@pytest.mark.parametrize("name", ["tiny_f32", "gqa_bf16", "dsa", "dsa_fp8"])
def test_exact_scores_strided_bitwise(name):
    cfg, kw, extra = CASES[name]
    w = synth.make_workload(cfg, **kw, **extra)
    say(f"[strided exact scores] {name}")
    step = restride(api.prepare(w, precision=api.EXACT))
    G = w.score_k.shape[1]
    scores = torch.empty((w.batch, G, w.max_kv_len), dtype=torch.float32, device="cuda")
    api.sparse_score_paged(step.args.pages, step.args.score_k, step.score_q, w.score_q.shape[1],
                           step.head_weights, api.MODES[w.mode], w.head_scale, api.EXACT, scores)
    torch.cuda.synchronize()
    ref = oracle.score(w.block_table, w.kv_lens, w.score_k, w.score_q, w.head_weights, w.mode,
                       w.head_scale, w.max_kv_len, w.score_k_scale)
    assert np.array_equal(scores.cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("dtype,head_dim", [("f32", 128), ("bf16", 32)])
def test_exact_scores_unstaged_rows_bitwise(dtype, head_dim):
    # rows of 512 and 64 bytes are read by each lane from memory directly
    w = synth.make_workload(1, batch=2, kv_len=[700, 1000], topk=64, head_dim=head_dim)
    if dtype == "bf16":
        for attr in ("k", "q"):
            a = getattr(w, attr)
            setattr(w, attr, synth.to_bf16_bits(a))
        w.score_k, w.score_q = w.k, w.q
    say(f"[unstaged exact scores] {dtype} D={head_dim}")
    k = api.to_device_array(w.score_k)
    q = api.to_device_array(w.score_q)
    pg = api.pages(api.to_device_array(w.block_table), api.to_device_array(w.kv_lens), w.max_kv_len)
    scores = torch.empty((w.batch, w.score_k.shape[1], w.max_kv_len), dtype=torch.float32, device="cuda")
    api.sparse_score_paged(pg, api.pool(k), q, w.score_q.shape[1], None, api.MODES[w.mode], w.head_scale,
                           api.EXACT, scores)
    torch.cuda.synchronize()
    ref = oracle.score(w.block_table, w.kv_lens, w.score_k, w.score_q, None, w.mode, w.head_scale,
                       w.max_kv_len, None)
    assert np.array_equal(scores.cpu().numpy().view(np.uint32), ref.view(np.uint32))
