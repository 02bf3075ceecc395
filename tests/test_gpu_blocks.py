"""GPU parity of attention over block-granular selections against the
oracle's token expansion."""
import numpy as np
import pytest
import torch

import oracle
from top_sparse_decode_amd import api, synth

from parity_util import assert_outputs_close, out_to_numpy

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def say(*a):
    print(*a, flush=True)


def block_lists(rs, kv_lens, groups, k_blocks, bs):
    """distinct blocks per row, some -1, some past kv_len"""
    B = len(kv_lens)
    out = np.full((B, groups, k_blocks), -1, np.int32)
    for b in range(B):
        nblk = max(1, (int(kv_lens[b]) + bs - 1) // bs + 2)   # a couple past the cache
        for g in range(groups):
            pick = rs.permutation(nblk)[:k_blocks]
            out[b, g, :len(pick)] = pick
            out[b, g, rs.random(k_blocks) < 0.1] = -1
    return out


def run_blocks(w, blocks, bs):
    step = api.prepare(w, precision=api.EXACT)
    kb = blocks.shape[-1]
    n = api.sparse_decode_attn_blocks_workspace_size(step.args.pages, w.q.shape[1], step.args.k, w.v_dim, kb, bs)
    ws = torch.empty(max(n, 16), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(step.out)
    api.sparse_decode_attn_blocks(step.args.pages, step.q, w.q.shape[1], step.args.k, step.args.v, w.v_dim,
                                  torch.from_numpy(blocks).cuda(), kb, bs, w.softmax_scale, out, ws)
    torch.cuda.synchronize()
    return step, out


@pytest.mark.parametrize("cfg,kw,kb,bs", [
    (4, dict(batch=3, kv_len=[9000, 2000, 37], topk=64), 40, 16),     # MLA
    (4, dict(batch=2, kv_len=[5000, 300], topk=64), 128, 8),
    (3, dict(batch=3, kv_len=[3000, 2049, 100], topk=64), 30, 32),    # GQA vector path
    (2, dict(batch=2, kv_len=[1024, 700], topk=64), 50, 4),           # MHA
])
def test_block_attention_matches_oracle(cfg, kw, kb, bs):
    w = synth.make_workload(cfg, **kw)
    rs = np.random.default_rng(cfg * 100 + bs)
    G = w.k.shape[1]
    blocks = block_lists(rs, w.kv_lens, G, kb, bs)
    say(f"[blocks] cfg {cfg} k_blocks {kb} block_size {bs}")
    _, out = run_blocks(w, blocks, bs)
    tok = oracle.expand_blocks(blocks, w.kv_lens, bs)
    ref = oracle.attention(w.block_table, w.kv_lens, w.q, w.k, w.v, w.v_dim, tok, w.softmax_scale)
    assert_outputs_close(out_to_numpy(out), ref, w.out_dtype, f"blocks cfg {cfg}")


def test_block_size_one_is_token_attention_bitwise():
    w = synth.make_workload(4, batch=2, kv_len=[6000, 3000], topk=512)
    rs = np.random.default_rng(9)
    idx = np.stack([np.sort(rs.permutation(int(L))[:512]) for L in w.kv_lens]).astype(np.int32)[:, None, :]
    step, out = run_blocks(w, idx, 1)
    n = api.sparse_decode_attn_workspace_size(step.args.pages, w.q.shape[1], step.args.k, w.v_dim, 512)
    ws = torch.empty(max(n, 16), dtype=torch.uint8, device="cuda")
    tok_out = torch.empty_like(step.out)
    api.sparse_decode_attn(step.args.pages, step.q, w.q.shape[1], step.args.k, step.args.v, w.v_dim,
                           torch.from_numpy(idx).cuda(), 512, w.softmax_scale, tok_out, ws)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), tok_out.view(torch.int16))
