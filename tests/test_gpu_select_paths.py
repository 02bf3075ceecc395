"""The selection's launch shapes against the oracle: one launch with row
barriers (grids that fit on the device at once), three launches (the
histogram, classify and emit passes), and the one-launch kernel with a tiny
wait at its row barriers, so that blocks give up waiting and finish their
rows alone (the path that guarantees progress when other work holds the
CUs).  Indices and counts must equal the oracle's in every shape."""
import os
from contextlib import contextmanager

import numpy as np
import pytest
import torch

import oracle
from top_sparse_decode_amd import api, synth

from parity_util import assert_outputs_close, oracle_run, out_to_numpy

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

SHAPES = {"one_launch": {}, "three_launches": {"SD_SELECT_ONE_LAUNCH": "0"},
          "solo_fallback": {"SD_SELECT_SPIN_TICKS": "1"}}


def say(*a):
    print(*a, flush=True)


@contextmanager
def shape(name):
    env = SHAPES[name]
    old = {k: os.environ.get(k) for k in env}
    os.environ.update(env)
    try:
        yield
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def topk_gpu(s, kv, k):
    B, G, S = s.shape
    idx = torch.empty((B, G, k), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B, G), dtype=torch.int32, device="cuda")
    ws = torch.empty(api.topk_workspace_size(B, G, S, k), dtype=torch.uint8, device="cuda")
    api.topk_select(torch.from_numpy(s).cuda(), B, G, S, torch.from_numpy(kv).cuda(), k, idx, cnt, ws, ws.numel())
    torch.cuda.synchronize()
    return idx.cpu().numpy(), cnt.cpu().numpy()


def rows_cases():
    rs = np.random.default_rng(11)
    ties = rs.integers(-20, 20, size=(3, 4, 5000)).astype(np.float32)
    ties[1, 2, :] = 7.0
    long = (rs.standard_normal((2, 1, 131072)) * 30 + 100).astype(np.float32)
    S = 70000
    edge = np.zeros((4, 1, S), np.float32)
    edge[0, 0, :] = 3.5
    edge[1, 0, :] = -np.inf
    edge[1, 0, 100:130] = np.arange(30, dtype=np.float32)
    edge[2, 0, :] = rs.standard_normal(S).astype(np.float32)
    edge[2, 0, 777] = 1e30
    edge[3, 0, :] = rs.integers(0, 3, S).astype(np.float32)
    return [("ties", ties, np.array([5000, 4321, 300], np.int32), (1, 17, 1024, 6000)),
            ("long", long, np.array([131072, 99999], np.int32), (2048,)),
            ("edge", edge, np.array([S, 5000, S, 66000], np.int32), (64, 2048))]


@pytest.mark.parametrize("name", list(SHAPES))
def test_standalone_selection_shapes(name):
    for what, s, kv, ks in rows_cases():
        for k in ks:
            say(f"[select {name}] {what} k={k}")
            with shape(name):
                idx, cnt = topk_gpu(s, kv, k)
            ri, rc = oracle.topk(s, kv, k)
            assert np.array_equal(idx, ri), f"{what} k={k}: indices differ"
            assert np.array_equal(cnt, rc), f"{what} k={k}: counts differ"


@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("index_dtype", ["bf16", "fp8"])
def test_fused_step_selection_shapes(name, index_dtype):
    # DSA-MLA shapes (64K rows, top-k 2048) with fast scores: the band re-score inside the one launch
    w = synth.make_workload(4, batch=4, kv_len=[65536, 40000, 9000, 2047], topk=2048, index_dtype=index_dtype)
    ref = oracle_run(w)
    for hint in (False, True):
        say(f"[fused {name}] {index_dtype} hint={hint}")
        step = api.prepare(w, precision=api.FAST, hint=hint)
        with shape(name):
            step.run()
            if hint:
                step.run()  # the second step uses the first one's write-back as its hint
            torch.cuda.synchronize()
        assert np.array_equal(step.indices.cpu().numpy(), ref["indices"]), "indices differ"
        assert np.array_equal(step.counts.cpu().numpy(), ref["counts"]), "counts differ"
        assert_outputs_close(out_to_numpy(step.out), ref["out"], w.out_dtype, f"{name} {index_dtype}")
