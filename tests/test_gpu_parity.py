"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs.  Indices must match bit for bit; outputs within 1e-5
(fp32) / 2e-2 (bf16) relative L2 per (request, head) row; exact-mode scores
bit for bit; fast scores within their reported bound."""
import numpy as np
import pytest
import torch

import oracle
from top_sparse_decode_amd import api, synth

from parity_util import TOL, assert_outputs_close, oracle_run, out_to_numpy, subset

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def say(*a):
    print(*a, flush=True)


def run_fused(w, precision):
    step = api.prepare(w, precision=precision)
    step.run()
    torch.cuda.synchronize()
    return step


def check_fused(w, precision, reqs=None, what=""):
    say(f"[fused] {what} {w.name} B={w.batch} precision={precision}")
    step = run_fused(w, precision)
    ref = oracle_run(w, reqs)
    sel = slice(None) if reqs is None else list(reqs)
    idx = step.indices.cpu().numpy()[sel]
    cnt = step.counts.cpu().numpy()[sel]
    assert np.array_equal(idx, ref["indices"]), f"{what}: indices differ"
    assert np.array_equal(cnt, ref["counts"]), f"{what}: counts differ"
    got = out_to_numpy(step.out)[sel]
    return assert_outputs_close(got, ref["out"], w.out_dtype, what), step


# ---------------------------------------------------------------- small cases

SMALL = {
    "tiny_f32": (1, dict(kv_len=1000, topk=128)),
    "tiny_f32_multi": (1, dict(batch=3, kv_len=[1000, 77, 1024], topk=100)),
    "mha_bf16": (2, dict(batch=2, kv_len=[1024, 700], topk=408)),
    "gqa_bf16": (3, dict(batch=3, kv_len=[3000, 2049, 5000], topk=2048)),
    "dsa": (4, dict(batch=2, kv_len=[9000, 4100], topk=2048)),
    "dsa_short": (4, dict(batch=3, kv_len=[1, 100, 2047], topk=2048)),
    "dsa_mixed": (5, dict(batch=3, min_len=2000, max_len=9000, topk=2048)),
    # the matrix-core scorer at 16 and 32 indexer heads and small pages
    "dsa_h16_p16": (4, dict(batch=2, kv_len=[3000, 1500], topk=512, idx_heads=16, page_size=16)),
    "dsa_h32": (4, dict(batch=3, kv_len=[7000, 64, 4097], topk=256, idx_heads=32)),
    "dsa_h32_p32": (4, dict(batch=2, kv_len=[5000, 33], topk=1024, idx_heads=32, page_size=32)),
}


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("precision", [api.EXACT, api.FAST])
def test_fused_small(name, precision):
    cfg, kw = SMALL[name]
    w = synth.make_workload(cfg, **kw)
    check_fused(w, precision, what=name)


@pytest.mark.parametrize("name", ["tiny_f32", "mha_bf16", "gqa_bf16", "dsa", "dsa_mixed"])
def test_exact_scores_bitwise(name):
    cfg, kw = SMALL[name]
    w = synth.make_workload(cfg, **kw)
    say(f"[scores] {name}")
    step = api.prepare(w, precision=api.EXACT)
    groups = w.score_k.shape[1]
    scores = torch.empty((w.batch, groups, w.max_kv_len), dtype=torch.float32, device="cuda")
    bound = torch.full((w.batch, groups), -1.0, device="cuda")  # exact scores leave it alone
    api.sparse_score_paged(step.args.pages, step.args.score_k, step.score_q, w.score_q.shape[1],
                           step.head_weights, api.MODES[w.mode], w.head_scale, api.EXACT, scores, bound)
    torch.cuda.synchronize()
    ref = oracle.score(w.block_table, w.kv_lens, w.score_k, w.score_q, w.head_weights, w.mode,
                       w.head_scale, w.max_kv_len)
    got = scores.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert torch.all(bound == -1.0)


# bf16 K with groups of 4, 8 and 16 heads and 64- or 128-dim rows: the
# exact scorer that holds the query in registers (one variant per group and
# row size), ragged lengths, page sizes below and above the 64-token tile
GROUP_SHAPES = {
    "g8_d128": dict(batch=3, q_heads=32, kv_heads=4, head_dim=128, kv_len=[3000, 64, 2049], topk=512),
    "g4_d64_p16": dict(batch=2, q_heads=8, kv_heads=2, head_dim=64, kv_len=[1500, 777], topk=256, page_size=16),
    "g8_d64": dict(batch=2, q_heads=16, kv_heads=2, head_dim=64, kv_len=[4096, 1], topk=128),
    "g16_d64_p128": dict(batch=2, q_heads=32, kv_heads=2, head_dim=64, kv_len=[2500, 1300], topk=300,
                         page_size=128),
}


@pytest.mark.parametrize("name", list(GROUP_SHAPES))
def test_exact_scores_bitwise_head_groups(name):
    w = synth.make_workload(3, **GROUP_SHAPES[name])
    say(f"[scores] {name}")
    # scores alone (a group of 16 heads has no attention path, so no fused step)
    bt = api.to_device_array(w.block_table, "cuda")
    kl = api.to_device_array(w.kv_lens, "cuda")
    sk = api.to_device_array(w.score_k, "cuda")
    sq = api.to_device_array(w.score_q, "cuda")
    groups = w.score_k.shape[1]
    scores = torch.empty((w.batch, groups, w.max_kv_len), dtype=torch.float32, device="cuda")
    bound = torch.full((w.batch, groups), -1.0, device="cuda")
    api.sparse_score_paged(api.pages(bt, kl, w.max_kv_len), api.pool(sk), sq, w.score_q.shape[1], None,
                           api.MODES[w.mode], w.head_scale, api.EXACT, scores, bound)
    torch.cuda.synchronize()
    ref = oracle.score(w.block_table, w.kv_lens, w.score_k, w.score_q, w.head_weights, w.mode,
                       w.head_scale, w.max_kv_len)
    assert np.array_equal(scores.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_fused_gqa_group_of_eight():
    w = synth.make_workload(3, **GROUP_SHAPES["g8_d128"])
    check_fused(w, api.EXACT, what="g8_d128")


@pytest.mark.parametrize("kw", [dict(batch=2, kv_len=[9000, 4100]),
                                dict(batch=2, kv_lens=[6000, 3000], bias_frac=0.01),
                                dict(batch=2, kv_len=[3000, 1500], idx_heads=16, page_size=16),
                                dict(batch=3, kv_len=[5000, 700, 1], idx_heads=32, page_size=32)])
def test_fast_scores_within_bound(kw):
    cfg = 5 if "kv_lens" in kw else 4
    w = synth.make_workload(cfg, **kw)
    say(f"[fast bound] {kw}")
    step = api.prepare(w, precision=api.FAST)
    scores = torch.empty((w.batch, 1, w.max_kv_len), dtype=torch.float32, device="cuda")
    bound = torch.zeros((w.batch, 1), dtype=torch.float32, device="cuda")  # max-accumulated
    api.sparse_score_paged(step.args.pages, step.args.score_k, step.score_q, w.score_q.shape[1], step.head_weights,
                           api.RELU_WEIGHTED, 1.0, api.FAST, scores, bound)
    torch.cuda.synchronize()
    ref = oracle.score(w.block_table, w.kv_lens, w.score_k, w.score_q, w.head_weights, w.mode, 1.0,
                       w.max_kv_len)
    got = scores.cpu().numpy()
    d = bound.cpu().numpy()
    for b in range(w.batch):
        L = int(w.kv_lens[b])
        err = np.abs(got[b, 0, :L].astype(np.float64) - ref[b, 0, :L])
        assert np.all(err <= d[b, 0]), (b, float(err.max()), float(d[b, 0]))
        assert np.all(got[b, 0, L:] == -np.inf)
        # the bound is its derivation's value, not a looser one
        f = bound_formula(w, b)
        assert f * (1 - 1e-3) <= d[b, 0] <= f * 1.01, (b, float(d[b, 0]), f)


def bound_formula(w, b):
    """The rigorous bound on |fast - exact| for request b, from its
    derivation: every |dot_h| error is at most gamma_D sum_d |q_hd||k_d| on
    either side (matrix-core sums counted with unit 2^-23, D = 128), the
    head sum adds gamma_{H+1} (unit 2^-24) of the weighted terms, so
      |s~ - s| <= B_t (2 gamma_{H+1} (1 + gamma_D) + 2 gamma_D),
      B_t = sum_d a_d |k_td|,  a_d = sum_h |w_h| |q_hd|,
    maximised over the row's tokens.  The kernel evaluates B_t with a_d
    rounded up to bfloat16 (at most 2^-7 above) and adds 1e-3 of slack, so
    its reported bound lies in [1, 1.01] times this value."""
    P = w.page_size
    L = int(w.kv_lens[b])
    if L == 0:
        return 0.0
    t = np.arange(L)
    rows = synth.bf16_bits_to_f32(w.score_k[w.block_table[b, t // P], 0, t % P]).astype(np.float64)
    q = synth.bf16_bits_to_f32(w.score_q[b]).astype(np.float64)
    a = np.abs(w.head_weights[b]).astype(np.float64) @ np.abs(q)
    bmax = float((np.abs(rows) @ a).max())

    def gamma(n, u):
        return n * u / (1 - n * u)

    H, D = q.shape
    gD, gH = gamma(D, 2.0 ** -23), gamma(H + 1, 2.0 ** -24)
    return bmax * (2 * gH * (1 + gD) + 2 * gD)


def test_topk_select_heavy_ties():
    # integer-valued scores: many exact ties, settled by lowest position
    rs = np.random.default_rng(1)
    B, G, S = 3, 4, 5000
    s = rs.integers(-20, 20, size=(B, G, S)).astype(np.float32)
    s[0, 0, ::3] = -0.0
    s[1, 2, :] = 7.0                       # a whole row of equal scores
    kv = np.array([5000, 4321, 300], np.int32)
    for k in (1, 17, 1024, 4321, 6000):
        say(f"[topk ties] k={k}")
        idx = torch.empty((B, G, k), dtype=torch.int32, device="cuda")
        cnt = torch.empty((B, G), dtype=torch.int32, device="cuda")
        ws = torch.empty(api.topk_workspace_size(B, G, S, k), dtype=torch.uint8, device="cuda")
        api.topk_select(torch.from_numpy(s).cuda(), B, G, S, torch.from_numpy(kv).cuda(), k, idx, cnt,
                        ws, ws.numel())
        torch.cuda.synchronize()
        ref_i, ref_c = oracle.topk(s, kv, k)
        assert np.array_equal(idx.cpu().numpy(), ref_i)
        assert np.array_equal(cnt.cpu().numpy(), ref_c)


def test_topk_select_long_rows_random_scores():
    rs = np.random.default_rng(2)
    B, S = 2, 131072
    s = rs.standard_normal((B, 1, S)).astype(np.float32) * 30 + 100
    kv = np.array([131072, 99999], np.int32)
    idx = torch.empty((B, 1, 2048), dtype=torch.int32, device="cuda")
    ws = torch.empty(api.topk_workspace_size(B, 1, S, 2048), dtype=torch.uint8, device="cuda")
    api.topk_select(torch.from_numpy(s).cuda(), B, 1, S, torch.from_numpy(kv).cuda(), 2048, idx, None,
                    ws, ws.numel())
    torch.cuda.synchronize()
    ref_i, _ = oracle.topk(s, kv, 2048)
    assert np.array_equal(idx.cpu().numpy(), ref_i)


def test_topk_select_edge_rows():
    # constant rows, rows with -inf (absent) tokens that must fill the quota,
    # a row of distinct scores with one huge outlier, and a long row past
    # the register-resident size
    S = 70000
    rows = np.zeros((5, 1, S), np.float32)
    rows[0, 0, :] = 3.5
    rows[1, 0, :] = -np.inf
    rows[1, 0, 100:130] = np.arange(30, dtype=np.float32)
    rows[2, 0, :] = np.random.default_rng(4).standard_normal(S).astype(np.float32)
    rows[2, 0, 777] = 1e30
    rows[3, 0, :] = np.random.default_rng(5).integers(0, 3, S).astype(np.float32)
    rows[4, 0, :] = np.random.default_rng(6).standard_normal(S).astype(np.float32)
    kv = np.array([S, 5000, S, S, 66000], np.int32)
    for k in (64, 2048):
        say(f"[topk edges] k={k}")
        idx = torch.empty((5, 1, k), dtype=torch.int32, device="cuda")
        ws = torch.empty(api.topk_workspace_size(5, 1, S, k), dtype=torch.uint8, device="cuda")
        api.topk_select(torch.from_numpy(rows).cuda(), 5, 1, S, torch.from_numpy(kv).cuda(), k, idx, None,
                        ws, ws.numel())
        torch.cuda.synchronize()
        ref_i, _ = oracle.topk(rows, kv, k)
        assert np.array_equal(idx.cpu().numpy(), ref_i)


@pytest.mark.parametrize("name", ["tiny_f32", "mha_bf16", "gqa_bf16", "dsa"])
def test_attention_on_oracle_indices(name):
    cfg, kw = SMALL[name]
    w = synth.make_workload(cfg, **kw)
    say(f"[attn] {name}")
    ref = oracle_run(w)
    step = api.prepare(w, precision=api.EXACT)
    # shuffle the order of each index list and pad with -1: the attention
    # result does not depend on the order
    idx = ref["indices"].copy()
    rs = np.random.default_rng(0)
    for r in idx.reshape(-1, idx.shape[-1]):
        rs.shuffle(r)
    d_idx = torch.from_numpy(idx).cuda()
    n = api.sparse_decode_attn_workspace_size(step.args.pages, w.q.shape[1], step.args.k, w.v_dim, w.topk)
    ws = torch.empty(max(n, 16), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(step.out)
    api.sparse_decode_attn(step.args.pages, step.q, w.q.shape[1], step.args.k, step.args.v, w.v_dim, d_idx,
                           w.topk, w.softmax_scale, out, ws)
    torch.cuda.synchronize()
    assert_outputs_close(out_to_numpy(out), ref["out"], w.out_dtype, name)


def test_fast_and_exact_agree_and_repeat_bitwise():
    w = synth.make_workload(4, batch=2, kv_len=[9000, 4100])
    say("[determinism]")
    a = run_fused(w, api.FAST)
    b = run_fused(w, api.EXACT)
    assert torch.equal(a.indices, b.indices)
    assert torch.equal(a.out.view(torch.int16), b.out.view(torch.int16))
    first = a.out.clone()
    a.run()
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int16), a.out.view(torch.int16))


def test_fast_path_band_overflow_falls_back_exactly():
    # Identical indexer keys on one request: every fast score is equal, so the
    # whole row is one band (far more than the band list holds); selection
    # must still be the exact one (all-equal exact scores -> lowest positions).
    w = synth.make_workload(4, batch=2, kv_len=[6000, 5000], topk=2048)
    P = w.page_size
    row0 = w.score_k[w.block_table[0, 0], 0, 0].copy()
    for t in range(6000):
        w.score_k[w.block_table[0, t // P], 0, t % P] = row0
    say("[band overflow]")
    check_fused(w, api.FAST, what="band overflow")


def test_empty_request_and_k_one():
    w = synth.make_workload(3, batch=3, kv_len=[0, 500, 64], topk=1)
    say("[empty, k=1]")
    step = run_fused(w, api.EXACT)
    ref = oracle_run(w)
    assert np.array_equal(step.indices.cpu().numpy(), ref["indices"])
    got = out_to_numpy(step.out)
    assert np.all(got[0] == 0)
    assert_outputs_close(got, ref["out"], "bf16", "k=1")


def test_local_to_global_matches_oracle():
    w = synth.make_workload(5, batch=4, min_len=100, max_len=3000, topk=64, idx_heads=16, heads=32)
    say("[local_to_global]")
    rs = np.random.default_rng(3)
    local = rs.integers(-3, 3100, size=(4, 2, 64)).astype(np.int32)
    bt = w.block_table.copy()
    bt[1, 0] = w.num_pages + 5          # a page outside the pool
    d_bt = torch.from_numpy(bt).cuda()
    pg = api.pages(d_bt, torch.from_numpy(w.kv_lens).cuda(), w.max_kv_len)
    out = torch.empty((4, 2, 64), dtype=torch.int64, device="cuda")
    api.local_to_global(pg, w.page_size, w.num_pages, torch.from_numpy(local).cuda(), out)
    torch.cuda.synchronize()
    ref = oracle.local_to_global(bt, w.page_size, w.num_pages, local)
    assert np.array_equal(out.cpu().numpy(), ref)


# ---------------------------------------------------------------- full sizes

@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_full_config_all_requests(cfg):
    w = synth.make_workload(cfg)
    worst, _ = check_fused(w, api.FAST, what=f"config {cfg}")
    say(f"config {cfg}: worst row rel-L2 {worst:.3e}")


@pytest.fixture(scope="module")
def dsa_full():
    return synth.make_workload(4)


@pytest.fixture(scope="module")
def dsa_mixed_full():
    return synth.make_workload(5)


def test_full_dsa_all_requests(dsa_full):
    worst, step = check_fused(dsa_full, api.FAST, what="DSA-MLA 16 x 64K (all 16 requests)")
    say(f"DSA-MLA 16 x 64K: worst row rel-L2 {worst:.3e}")
    assert torch.isfinite(step.out.float()).all()


def test_full_dsa_mixed_all_requests(dsa_mixed_full):
    w = dsa_mixed_full
    worst, step = check_fused(w, api.FAST, what="mixed-length DSA-MLA (all 64 requests)")
    say(f"mixed-length DSA-MLA: worst row rel-L2 {worst:.3e}, lengths {int(w.kv_lens.min())}..{int(w.kv_lens.max())}")
    assert torch.isfinite(step.out.float()).all()


# ---------------------------------------------------------------- MLA head counts

# The sparse MLA kernel runs one wave per 32 query heads (32, 64 or 128 heads
# per latent KV row) and the combine one block per (request, 32 heads,
# quarter of the value columns).  Several splits and a partial last split
# (k not a multiple of the 128-row split) for each head count, through the
# attention entry point on oracle indices and through the fused call.
@pytest.mark.parametrize("heads", [32, 64])
@pytest.mark.parametrize("topk", [1000, 2048])
def test_mla_head_counts(heads, topk):
    w = synth.make_workload(4, batch=3, kv_len=[9000, 4100, 1500], topk=topk, heads=heads)
    assert w.q.shape[1] == heads
    check_fused(w, api.FAST, what=f"MLA {heads} heads k={topk}")
    ref = oracle_run(w)
    step = api.prepare(w, precision=api.EXACT)
    d_idx = torch.from_numpy(ref["indices"]).cuda()
    n = api.sparse_decode_attn_workspace_size(step.args.pages, heads, step.args.k, w.v_dim, w.topk)
    ws = torch.empty(max(n, 16), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(step.out)
    api.sparse_decode_attn(step.args.pages, step.q, heads, step.args.k, step.args.v, w.v_dim, d_idx,
                           w.topk, w.softmax_scale, out, ws)
    torch.cuda.synchronize()
    assert_outputs_close(out_to_numpy(out), ref["out"], w.out_dtype, f"MLA attention {heads} heads")
