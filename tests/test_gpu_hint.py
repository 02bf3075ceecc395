"""GPU parity of hinted top-k and its write-back: for any hint the selection
equals the oracle's top-k (the hint only narrows the search), and the
write-back buffer receives exactly the selected indices."""
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


def hinted(scores, kv, k, hint, writeback_extra=3):
    B, G, S = scores.shape
    d_s = torch.from_numpy(scores).cuda()
    idx = torch.empty((B, G, k), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B, G), dtype=torch.int32, device="cuda")
    # a write-back row longer than k: the tail must stay untouched
    wb = torch.full((B, G, k + writeback_extra), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(api.topk_workspace_size(B, G, S, k), dtype=torch.uint8, device="cuda")
    h = None if hint is None else torch.from_numpy(np.ascontiguousarray(hint, dtype=np.int32)).cuda()
    api.topk_select_hinted(d_s, B, G, S, torch.from_numpy(kv).cuda(), k, h, idx, cnt, wb, ws, ws.numel())
    torch.cuda.synchronize()
    wbn = wb.cpu().numpy()
    assert np.array_equal(wbn[..., :k], idx.cpu().numpy()), "write-back differs from the selection"
    assert np.all(wbn[..., k:] == -7), "write-back wrote past k"
    return idx.cpu().numpy(), cnt.cpu().numpy()


def hint_cases(scores, kv, k, rs):
    """A set of hints for the same rows: perfect, shuffled, perturbed,
    duplicated, out of range, short, long and garbage."""
    B, G, S = scores.shape
    ref, _ = oracle.topk(scores, kv, k)
    perfect = ref.copy()
    shuffled = ref.copy()
    for r in shuffled.reshape(-1, k):
        rs.shuffle(r)
    perturbed = ref.copy()
    m = rs.random(perturbed.shape) < 0.1               # 10% replaced by random positions
    perturbed[m] = rs.integers(0, S, size=int(m.sum()))
    dup = np.repeat(ref[..., :1], k, axis=-1)          # one position k times: certifies nothing
    oob = ref.copy()
    oob[..., ::7] = -1
    oob[..., 1::7] = S + 5                            # past kv_len and the row
    short = ref[..., : max(1, k // 2)]                 # fewer than k entries
    long = np.concatenate([ref, rs.integers(0, S, size=(B, G, 17)).astype(np.int32)], axis=-1)
    garbage = rs.integers(-3, S + 3, size=(B, G, k)).astype(np.int32)
    return {"perfect": perfect, "shuffled": shuffled, "perturbed": perturbed, "duplicates": dup,
            "out_of_range": oob, "short": short, "long": long, "garbage": garbage, "none": None}


@pytest.mark.parametrize("kind", ["normal", "ties", "long_rows"])
def test_hinted_topk_equals_oracle_for_any_hint(kind):
    rs = np.random.default_rng({"normal": 11, "ties": 12, "long_rows": 13}[kind])
    if kind == "normal":
        B, G, S, k = 3, 2, 20000, 1024
        s = (rs.standard_normal((B, G, S)) * 25 + 100).astype(np.float32)
        kv = np.array([20000, 13001, 900], np.int32)
    elif kind == "ties":
        B, G, S, k = 2, 2, 9000, 700
        s = rs.integers(-5, 6, size=(B, G, S)).astype(np.float32)
        kv = np.array([9000, 4321], np.int32)
    else:
        B, G, S, k = 2, 1, 131072, 2048
        s = rs.standard_normal((B, G, S)).astype(np.float32)
        kv = np.array([131072, 70000], np.int32)
    ref_i, ref_c = oracle.topk(s, kv, k)
    for name, h in hint_cases(s, kv, k, rs).items():
        say(f"[hinted topk] {kind} hint={name}")
        idx, cnt = hinted(s, kv, k, h)
        assert np.array_equal(idx, ref_i), f"{kind}/{name}: indices differ"
        assert np.array_equal(cnt, ref_c), f"{kind}/{name}: counts differ"


def test_hint_from_other_scores_still_exact():
    # a hint taken from an unrelated score set: its floor is low but valid
    rs = np.random.default_rng(21)
    s1 = rs.standard_normal((2, 1, 30000)).astype(np.float32)
    s2 = rs.standard_normal((2, 1, 30000)).astype(np.float32)
    kv = np.array([30000, 29999], np.int32)
    h, _ = oracle.topk(s1, kv, 512)
    idx, _ = hinted(s2, kv, 512, h)
    assert np.array_equal(idx, oracle.topk(s2, kv, 512)[0])


@pytest.mark.parametrize("precision", [api.EXACT, api.FAST])
@pytest.mark.parametrize("index_dtype", ["bf16", "fp8"])
def test_fused_steps_with_hint_feedback(precision, index_dtype):
    # step 1 starts from an empty hint (-1), writes its selection back; step 2
    # consumes it; a foreign hint follows.  Every step equals the oracle.
    w = synth.make_workload(4, batch=3, kv_len=[9000, 4100, 1500], topk=1024, index_dtype=index_dtype)
    ref = oracle_run(w)
    step = api.prepare(w, precision=precision, hint=True)
    for it in range(3):
        if it == 2:  # foreign hint: another request's selection, shifted
            step.hint.copy_(torch.roll(step.hint, 1, dims=0))
        say(f"[fused hint] {index_dtype} precision={precision} step {it}")
        step.run()
        torch.cuda.synchronize()
        idx = step.indices.cpu().numpy()
        assert np.array_equal(idx, ref["indices"]), f"step {it}: indices differ"
        assert np.array_equal(step.hint.cpu().numpy(), idx), f"step {it}: write-back differs"
        assert_outputs_close(out_to_numpy(step.out), ref["out"], w.out_dtype, f"hint step {it}")


def test_full_dsa_with_hint_all_requests():
    w = synth.make_workload(4)
    step = api.prepare(w, precision=api.FAST, hint=True)
    step.run()
    step.run()  # the second step uses the first one's write-back
    torch.cuda.synchronize()
    ref = oracle_run(w)
    assert np.array_equal(step.indices.cpu().numpy(), ref["indices"])
    assert_outputs_close(out_to_numpy(step.out), ref["out"], w.out_dtype, "DSA-MLA 16 x 64K hinted")
    assert torch.equal(step.hint, step.indices)
