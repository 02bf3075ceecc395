"""The one-wave-per-row selection (rows of at most 4096 tokens with exact
scores, taken when there are many rows) against the oracle: indices and
counts exactly.  SD_SELECT_WAVE_ROWS=1 sends every short-row selection down
this path, whatever the row count."""
import os

import numpy as np
import pytest
import torch

import oracle
from top_sparse_decode_amd import api

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def say(*a):
    print(*a, flush=True)


def topk_gpu(s, kv, k):
    B, G, S = s.shape
    idx = torch.empty((B, G, k), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B, G), dtype=torch.int32, device="cuda")
    ws = torch.empty(api.topk_workspace_size(B, G, S, k), dtype=torch.uint8, device="cuda")
    api.topk_select(torch.from_numpy(np.ascontiguousarray(s)).cuda(), B, G, S, torch.from_numpy(kv).cuda(), k,
                    idx, cnt, ws, ws.numel())
    torch.cuda.synchronize()
    return idx.cpu().numpy(), cnt.cpu().numpy()


def check(s, kv, k, what):
    say(f"[select wave] {what} shape={s.shape} k={k}")
    idx, cnt = topk_gpu(s, kv, k)
    ri, rc = oracle.topk(s, kv, k)
    assert np.array_equal(idx, ri), f"{what} k={k}: indices differ"
    assert np.array_equal(cnt, rc), f"{what} k={k}: counts differ"


def rows(seed, B, G, S):
    rs = np.random.default_rng(seed)
    s = (rs.standard_normal((B, G, S)) * np.exp(rs.uniform(-3, 3, size=(B, G, 1)))
         + rs.uniform(-50, 50, size=(B, G, 1))).astype(np.float32)
    s[0, 0, :] = rs.integers(-3, 4, size=S).astype(np.float32)       # heavy ties
    s[0, 1, :] = 2.5                                                   # one value
    s[1, 0, ::3] = -np.inf                                             # absent tokens
    s[1, 1, :] = rs.choice(np.array([0.0, -0.0, 1.0, -1.0], np.float32), size=S)   # signed zeros tie
    s[2, 0, :] = -np.inf
    s[2, 0, 5:9] = np.inf                                              # infinities rank at the ends
    s[2, 1, :] = np.ldexp(rs.uniform(1, 2, S), rs.integers(-120, 120, S)).astype(np.float32)
    return s


@pytest.mark.parametrize("S", [1000, 2048, 4096, 3001])
def test_wave_selection_forced(S, monkeypatch):
    monkeypatch.setenv("SD_SELECT_WAVE_ROWS", "1")
    s = rows(61, 3, 3, S)
    kv = np.array([S, S - 1, S // 2 + 1], np.int32)
    for k in (1, 17, S // 2, S - 2):
        check(s, kv, k, f"forced S={S}")
    kv2 = np.array([0, 1, S // 3], np.int32)                           # empty and short rows
    check(s, kv2, S // 3, f"forced short S={S}")
    check(s, kv2, S // 3 + 5, f"forced padded S={S}")


def test_wave_selection_by_row_count():
    # 2048 rows of 1024 tokens: the one-wave path without forcing
    assert os.environ.get("SD_SELECT_WAVE_ROWS") is None
    rs = np.random.default_rng(62)
    s = rs.standard_normal((64, 32, 1024)).astype(np.float32)
    s[3, :, :] = rs.integers(0, 5, size=(32, 1024)).astype(np.float32)
    kv = rs.integers(1, 1025, size=64).astype(np.int32)
    kv[0] = 1024
    check(s, kv, 512, "rows=2048")
