"""Shared helpers for the GPU parity tests: run the CPU oracle on (a subset
of) a workload and compare with the device results."""
import dataclasses

import numpy as np

import oracle

TOL = {"f32": 1e-5, "bf16": 2e-2}


def subset(w, reqs):
    """The same workload restricted to requests `reqs` (pools shared)."""
    reqs = list(reqs)
    n = int(getattr(w, "next_n", 1))
    rows = [b * n + j for b in reqs for j in range(n)]   # query rows of the requests
    return dataclasses.replace(
        w, block_table=w.block_table[reqs], kv_lens=w.kv_lens[reqs], score_q=w.score_q[rows],
        head_weights=None if w.head_weights is None else w.head_weights[rows], q=w.q[rows])


def oracle_run(w, reqs=None):
    ws = w if reqs is None else subset(w, reqs)
    return oracle.sparse_decode(ws)


def row_rel_l2(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Relative L2 per (request, head) row; rows whose reference is zero
    must be zero themselves (reported as 0 or inf)."""
    got = got.astype(np.float64)
    num = np.linalg.norm(got - ref, axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    out = np.where(den > 0, num / np.where(den > 0, den, 1), np.where(num > 0, np.inf, 0.0))
    return out


def out_to_numpy(t) -> np.ndarray:
    import torch

    return t.detach().to(torch.float32).cpu().numpy()


def assert_outputs_close(got: np.ndarray, ref: np.ndarray, out_dtype: str, what=""):
    err = row_rel_l2(got, ref)
    tol = TOL[out_dtype]
    worst = float(err.max()) if err.size else 0.0
    assert worst <= tol, f"{what}: max per-row rel-L2 {worst:.3e} > {tol:g}"
    return worst
