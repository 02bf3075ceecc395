"""GPU parity of the TriAttention selection modes (normalize -> reduce ->
top-k) against the oracle: reduced rows bit for bit, indices and counts
exactly."""
import numpy as np
import pytest
import torch

import oracle
from top_sparse_decode_amd import api, synth

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

MODES = ["per_layer_perhead", "per_head", "union"]


def say(*a):
    print(*a, flush=True)


def run_tri(scores, kv, mode, k):
    layers, B, G, S = scores.shape
    out_rows = {"per_layer_perhead": layers * B * G, "per_head": B * G, "union": B}[mode]
    d = torch.from_numpy(np.ascontiguousarray(scores)).cuda()
    idx = torch.empty((out_rows, k), dtype=torch.int32, device="cuda")
    cnt = torch.empty((out_rows,), dtype=torch.int32, device="cuda")
    red = torch.empty((out_rows, S), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(api.triattention_select_workspace_size(layers, B, G, S, mode, k), 16),
                     dtype=torch.uint8, device="cuda")
    api.triattention_select(d, torch.from_numpy(kv).cuda(), mode, k, idx, cnt, red, ws)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), cnt.cpu().numpy(), red.cpu().numpy()


def check(scores, kv, mode, k, what):
    say(f"[tri] {what} mode={mode} shape={scores.shape} k={k}")
    ref = oracle.tri_select(scores, kv, mode, k)
    idx, cnt, red = run_tri(scores, kv, mode, k)
    assert np.array_equal(red.view(np.uint32), ref["reduced"].view(np.uint32)), f"{what}: reduced rows differ"
    assert np.array_equal(idx, ref["indices"]), f"{what}: indices differ"
    assert np.array_equal(cnt, ref["counts"]), f"{what}: counts differ"


def random_scores(seed, layers, B, G, S):
    rs = np.random.default_rng(seed)
    loc = rs.uniform(-50, 50, size=(layers, B, G, 1))
    scale = np.exp(rs.uniform(-3, 3, size=(layers, B, G, 1)))
    return (rs.standard_normal((layers, B, G, S)) * scale + loc).astype(np.float32)


@pytest.mark.parametrize("mode", MODES)
def test_tri_modes_random_rows(mode):
    s = random_scores(41, 3, 4, 4, 6000)
    kv = np.array([6000, 4096, 333, 5001], np.int32)   # resident and streamed rows, ragged
    check(s, kv, mode, 512, "random")


@pytest.mark.parametrize("mode", MODES)
def test_tri_modes_edge_rows(mode):
    rs = np.random.default_rng(42)
    s = rs.integers(-4, 5, size=(2, 3, 2, 3000)).astype(np.float32)   # heavy ties
    s[0, 0, 0, :] = 2.5                                                # constant row
    s[1, 1, 1, 10:400] = -np.inf                                       # absent tokens
    s[1, 2, 0, :] = -np.inf                                            # no finite score
    kv = np.array([3000, 1024, 17], np.int32)
    check(s, kv, mode, 64, "edges")
    kv0 = np.array([3000, 0, 2], np.int32)                             # empty and short rows
    check(s, kv0, mode, 4, "empty")


@pytest.mark.parametrize("mode", MODES)
def test_tri_long_rows(mode):
    s = random_scores(43, 2, 2, 2, 70000)
    kv = np.array([70000, 65537], np.int32)
    check(s, kv, mode, 2048, "long")


def test_tri_from_paged_group_mean_scores():
    # the whole TriAttention step: per-layer paged GQA scores (group mean over
    # 4 query heads per KV head, exact scorer) stacked, then union selection
    layers = [synth.make_workload(3, seed=50 + l, batch=3, kv_len=[4096, 3000, 1111], topk=256)
              for l in range(3)]
    S = layers[0].max_kv_len
    gpu, ref = [], []
    for w in layers:
        step = api.prepare(w, precision=api.EXACT)
        G = w.score_k.shape[1]
        sc = torch.empty((w.batch, G, S), dtype=torch.float32, device="cuda")
        api.sparse_score_paged(step.args.pages, step.args.score_k, step.score_q, w.score_q.shape[1],
                               step.head_weights, api.MODES[w.mode], w.head_scale, api.EXACT, sc)
        gpu.append(sc)
        ref.append(oracle.score(w.block_table, w.kv_lens, w.score_k, w.score_q, w.head_weights, w.mode,
                                w.head_scale, S))
    torch.cuda.synchronize()
    stacked = torch.stack(gpu).cpu().numpy()
    assert np.array_equal(stacked.view(np.uint32), np.stack(ref).view(np.uint32))
    for mode in MODES:
        check(stacked, layers[0].kv_lens, mode, 256, "paged")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("S", [3000, 3001])
def test_tri_many_members_both_reduce_paths(mode, S):
    # 20 members per union row (the sliced reduce); a row stride that is a
    # multiple of four takes the 16-byte-load reduce, an odd one the scalar one
    s = random_scores(44, 5, 2, 4, S)
    kv = np.array([S, 1234], np.int32)
    check(s, kv, mode, 256, f"members S={S}")


def wide_range_rows(seed, layers, B, G, S):
    # binary32 scores whose magnitudes span 2^-120 .. 2^60 within a row, exact
    # cancellations of large values, and rows where a few scores sit far from
    # the rest: sums the grid extraction cannot take whole, so the long
    # accumulation decides them
    rs = np.random.default_rng(seed)
    mant = rs.uniform(1, 2, size=(layers, B, G, S)) * rs.choice([-1.0, 1.0], size=(layers, B, G, S))
    s = np.ldexp(mant, rs.integers(-120, 61, size=(layers, B, G, S))).astype(np.float32)
    big = np.float32(2.0 ** 60)
    s[0, 0, 0, :4] = [big, 1.0, -big, 3.0]                      # exact mean of the four: 1
    s[0, 0, 0, 4:] = 0.0
    s[-1, -1, -1, :] = np.float32(7.0)
    s[-1, -1, -1, ::97] = np.float32(7.0 + 2.0 ** -21)          # deviations 2^-21 and tiny means
    return s


@pytest.mark.parametrize("mode", MODES)
def test_tri_exact_sums_on_wide_range_rows(mode):
    s = wide_range_rows(45, 2, 2, 3, 4096)
    kv = np.array([4096, 2999], np.int32)
    check(s, kv, mode, 300, "wide range")


@pytest.mark.parametrize("S", [1000, 2048, 4096, 4100, 12000, 4099])
def test_tri_every_row_layout(S):
    # rows held in registers by one wave (up to 1024, 2048, 4096 tokens) or
    # by four (up to 8192, 16384), and rows read again in every pass (a
    # stride that is not a multiple of four)
    s = random_scores(46, 2, 3, 2, S)
    kv = np.array([S, S - 1, 1], np.int32)
    check(s, kv, "per_layer_perhead", 64, f"layout S={S}")


@pytest.mark.parametrize("S", [1000, 4096, 6000, 4099])
def test_tri_long_accumulation_forced(S, monkeypatch):
    # SD_TRI_EXACT_SLOW=1: every sum through the long accumulator
    monkeypatch.setenv("SD_TRI_EXACT_SLOW", "1")
    s = random_scores(47, 2, 2, 2, S)
    s[1, 1, 1, :] = wide_range_rows(48, 3, 1, 1, S)[1, 0, 0]   # a random wide-range row
    kv = np.array([S, S - 3], np.int32)
    check(s, kv, "per_layer_perhead", 64, f"forced long S={S}")
    check(s, kv, "union", 64, f"forced long S={S}")


@pytest.mark.parametrize("ragged", [False, True])
def test_tri_full_size_all_modes(ragged):
    # the benchmarked shape: 36 layers x 32 requests x 8 KV heads x 4096
    # tokens (151 MB), per-row location U(-50, 50), spread exp(U(-2, 2)),
    # keep 2048; every reduced row, index and count compared
    rs = np.random.default_rng(2048)
    layers, B, G, S, k = 36, 32, 8, 4096, 2048
    loc = rs.uniform(-50, 50, size=(layers, B, G, 1))
    spread = np.exp(rs.uniform(-2, 2, size=(layers, B, G, 1)))
    s = (rs.standard_normal((layers, B, G, S), dtype=np.float32) * spread + loc).astype(np.float32)
    kv = rs.integers(2049, S + 1, size=B).astype(np.int32) if ragged else np.full(B, S, np.int32)
    for mode in MODES:
        check(s, kv, mode, k, f"full size ragged={ragged}")


@pytest.mark.parametrize("S", [1000, 2048, 4096, 3001])
def test_tri_selection_without_reduced_rows(S):
    # no reduced rows asked for: per layer and head the statistics kernel
    # selects without writing z rows; indices and counts still exact
    s = random_scores(49, 3, 2, 4, S)
    s[0, 0, 0, :] = np.float32(1.5)                                   # one value
    s[1, 1, 1, ::5] = -np.inf
    kv = np.array([S, S // 2 + 1], np.int32)
    layers, B, G, _ = s.shape
    for mode, k in (("per_layer_perhead", 64), ("per_layer_perhead", S // 2), ("union", 128)):
        out_rows = {"per_layer_perhead": layers * B * G, "per_head": B * G, "union": B}[mode]
        idx = torch.empty((out_rows, k), dtype=torch.int32, device="cuda")
        cnt = torch.empty((out_rows,), dtype=torch.int32, device="cuda")
        ws = torch.empty(api.triattention_select_workspace_size(layers, B, G, S, mode, k), dtype=torch.uint8,
                         device="cuda")
        say(f"[tri] no reduced rows mode={mode} S={S} k={k}")
        api.triattention_select(torch.from_numpy(s).cuda(), torch.from_numpy(kv).cuda(), mode, k, idx, cnt, None,
                                ws)
        torch.cuda.synchronize()
        ref = oracle.tri_select(s, kv, mode, k)
        assert np.array_equal(idx.cpu().numpy(), ref["indices"]), mode
        assert np.array_equal(cnt.cpu().numpy(), ref["counts"]), mode
