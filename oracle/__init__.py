"""Plain CPU oracle for top-k sparse decode attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the HIP library: the arithmetic lives in ``oracle.c`` (plain C, built with
``-O2 -ffp-contract=off``), and this module only marshals numpy arrays into it.

Functions and the passages they follow:

* :func:`score` -- every cached token scored through the page table ("Add
  TriAttention KV-cache compression method", Key Design Decisions: direct
  paged-pool scoring; for the DSA indexer mode see "Overlap DSA heuristic
  prev_topk write-back on the aux stream", Description).
* :func:`topk` -- full sort by (score desc, index asc), the deterministic tie
  settlement of "Add TriAttention ...", Summary / Test Plan.
* :func:`attention` -- float64 softmax attention over the selected rows, the
  eager golden reference of "Add DSA Vanilla sparse attention", Walkthrough.
* :func:`local_to_global` -- the global index conversion of "Unify sparse
  attention framework with clean backend interfaces", Dev Engineer Review.

Parity pins (tests/test_oracle_pins.py) tie each function to closed forms,
brute force, a library routine (SDPA) and invariants; see the test module.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F32, BF16, FP8 = 0, 1, 2
GROUP_SUM, GROUP_MEAN, RELU_WEIGHTED = 0, 1, 2
_MODES = {"group_sum": GROUP_SUM, "group_mean": GROUP_MEAN, "relu_weighted": RELU_WEIGHTED}
_ERRORS = {1: "bad argument", 2: "page id out of range", 3: "NaN score", 4: "index out of range"}

CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-std=c11", "-fopenmp"]


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so next to it (gcc, plain C)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Pool(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_stride", ctypes.c_int64),
        ("head_stride", ctypes.c_int64),
        ("token_stride", ctypes.c_int64),
        ("scale", ctypes.c_void_p),
    ]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        P, I32, I64, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        PP = ctypes.POINTER(_Pool)
        lib.orc_score.argtypes = [P, I32, P, I32, PP, P, I32, I32, P, I32, F, P, I32]
        lib.orc_topk.argtypes = [P, I32, I32, I32, P, I32, P, P]
        lib.orc_attention.argtypes = [P, I32, P, I32, P, I32, I32, PP, PP, I32, P, I32, F, P]
        lib.orc_local_to_global.argtypes = [P, I32, I32, I32, I32, P, I32, I32, P]
        lib.orc_tri_select.argtypes = [P, I32, I32, I32, I32, P, I32, I32, P, P, P, P]
        lib.orc_exact_sum.argtypes = [P, I64, P]
        lib.orc_set_threads.argtypes = [I32]
        lib.orc_set_threads.restype = ctypes.c_int
        for f in (lib.orc_score, lib.orc_topk, lib.orc_attention, lib.orc_local_to_global, lib.orc_tri_select,
                  lib.orc_exact_sum):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def set_threads(n: int = 0) -> int:
    """Threads the oracle's row loops use (n > 0 sets them); returns the count
    in effect.  Results are bit-identical for every count."""
    return int(_load().orc_set_threads(int(n)))


def exact_sum(values) -> float:
    """The exactly rounded sum of finite binary64 values: their exact real sum
    rounded once to the nearest binary64, ties to even (the sums of the
    TriAttention normalization)."""
    v = np.ascontiguousarray(np.asarray(values, dtype=np.float64))
    out = np.zeros(1, dtype=np.float64)
    _check(_load().orc_exact_sum(v.ctypes.data, v.size, out.ctypes.data), "exact_sum")
    return float(out[0])


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {what}: {_ERRORS.get(rc, rc)}")


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.uint8:
        return FP8
    raise TypeError(f"oracle takes float32, bfloat16 bits (uint16) or FP8 E4M3 codes (uint8), got {a.dtype}")


@dataclass
class PoolView:
    """A paged pool in host memory.  ``data`` is a numpy array (float32 or
    uint16 bfloat16 bits); its shape is [num_pages, num_kv_heads, page_size,
    head_dim] in any memory order, the element strides are taken from it."""

    data: np.ndarray
    scale: Optional[np.ndarray] = None  # FP8 pools: [num_pages, num_kv_heads, page_size] float32

    def struct(self) -> _Pool:
        a = self.data
        if a.ndim != 4:
            raise ValueError("pool must be 4-D [pages, kv_heads, page_size, head_dim]")
        es = a.itemsize
        st = [s // es for s in a.strides]
        if st[3] != 1:
            raise ValueError("pool rows must be contiguous")
        sc = None
        if a.dtype == np.uint8:
            if self.scale is None or self.scale.shape != (a.shape[0], a.shape[1], a.shape[2]):
                raise ValueError("an FP8 pool needs scales [num_pages, num_kv_heads, page_size]")
            self._scale_c = np.ascontiguousarray(self.scale, dtype=np.float32)  # kept alive with the view
            sc = self._scale_c.ctypes.data
        return _Pool(a.ctypes.data, _dtype_code(a), a.shape[0], a.shape[2], a.shape[1],
                     a.shape[3], st[0], st[1], st[2], sc)


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def score(block_table, kv_lens, k_pool: np.ndarray, q: np.ndarray, weights, mode: int,
          head_scale: float, row_len: int, k_scale: Optional[np.ndarray] = None) -> np.ndarray:
    """Scores [batch, num_kv_heads, row_len] float32 (-inf past kv_len).  An
    FP8 pool (uint8 codes) comes with its row scales ``k_scale``."""
    lib = _load()
    bt = _c(block_table, np.int32)
    kl = _c(kv_lens, np.int32)
    view = PoolView(k_pool, k_scale)
    pool = view.struct()
    qa = np.ascontiguousarray(q)
    batch, q_heads = qa.shape[0], qa.shape[1]
    w = None if weights is None else _c(weights, np.float32)
    mode = _MODES[mode] if isinstance(mode, str) else int(mode)
    out = np.empty((batch, k_pool.shape[1], row_len), dtype=np.float32)
    rc = lib.orc_score(bt.ctypes.data, bt.shape[1], kl.ctypes.data, batch, ctypes.byref(pool),
                       qa.ctypes.data, _dtype_code(qa), q_heads,
                       None if w is None else w.ctypes.data, mode, float(head_scale),
                       out.ctypes.data, row_len)
    _check(rc, "score")
    return out


def topk(scores: np.ndarray, kv_lens, k: int):
    """Returns (indices [batch, groups, k] int32, counts [batch, groups] int32)."""
    lib = _load()
    s = _c(scores, np.float32)
    kl = _c(kv_lens, np.int32)
    batch, groups, row_len = s.shape
    idx = np.empty((batch, groups, k), dtype=np.int32)
    cnt = np.empty((batch, groups), dtype=np.int32)
    rc = lib.orc_topk(s.ctypes.data, batch, groups, row_len, kl.ctypes.data, k,
                      idx.ctypes.data, cnt.ctypes.data)
    _check(rc, "topk")
    return idx, cnt


def attention(block_table, kv_lens, q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
              v_dim: int, indices: np.ndarray, scale: float) -> np.ndarray:
    """Float64 output [batch, q_heads, v_dim]."""
    lib = _load()
    bt = _c(block_table, np.int32)
    kl = _c(kv_lens, np.int32)
    qa = np.ascontiguousarray(q)
    kp, vp = PoolView(k_pool).struct(), PoolView(v_pool).struct()
    ind = _c(indices, np.int32)
    batch, q_heads = qa.shape[0], qa.shape[1]
    out = np.empty((batch, q_heads, v_dim), dtype=np.float64)
    rc = lib.orc_attention(bt.ctypes.data, bt.shape[1], kl.ctypes.data, batch, qa.ctypes.data,
                           _dtype_code(qa), q_heads, ctypes.byref(kp), ctypes.byref(vp), v_dim,
                           ind.ctypes.data, ind.shape[2], float(scale), out.ctypes.data)
    _check(rc, "attention")
    return out


def local_to_global(block_table, page_size: int, num_pages: int, local: np.ndarray) -> np.ndarray:
    lib = _load()
    bt = _c(block_table, np.int32)
    loc = _c(local, np.int32)
    batch, groups, k = loc.shape
    out = np.empty(loc.shape, dtype=np.int64)
    rc = lib.orc_local_to_global(bt.ctypes.data, bt.shape[1], batch, page_size, num_pages,
                                 loc.ctypes.data, groups, k, out.ctypes.data)
    _check(rc, "local_to_global")
    return out


def expand_blocks(block_indices: np.ndarray, kv_lens, block_size: int) -> np.ndarray:
    """Block-granular selections as token lists: entry e >= 0 of a row
    names tokens e*block_size .. e*block_size + block_size - 1 that lie below
    the request's kv_len, -1 stands for the others and for negative entries
    ("Unify sparse attention framework with clean backend interfaces": the
    runtime carrier's indices block size).  [batch, groups, k_blocks] ->
    [batch, groups, k_blocks * block_size]."""
    bi = np.asarray(block_indices, dtype=np.int64)
    B, G, kb = bi.shape
    tok = bi[..., None] * block_size + np.arange(block_size)
    L = np.asarray(kv_lens, dtype=np.int64)[:, None, None, None]
    ok = (bi[..., None] >= 0) & (tok < L)
    return np.where(ok, tok, -1).reshape(B, G, kb * block_size).astype(np.int32)


TRI_MODES = {"per_layer_perhead": 0, "per_head": 1, "union": 2}


def tri_select(scores: np.ndarray, kv_lens, mode, k: int) -> dict:
    """TriAttention normalize -> reduce -> top-k (see oracle.h).  scores is
    [layers, batch, groups, row_len] float32; returns z (same shape), the
    reduced rows, indices and counts ([out_rows, k] / [out_rows] with
    out_rows = layers*batch*groups, batch*groups or batch by mode)."""
    lib = _load()
    s = _c(scores, np.float32)
    kl = _c(kv_lens, np.int32)
    layers, batch, groups, row_len = s.shape
    m = TRI_MODES[mode] if isinstance(mode, str) else int(mode)
    out_rows = {0: layers * batch * groups, 1: batch * groups, 2: batch}[m]
    z = np.empty(s.shape, dtype=np.float32)
    red = np.empty((out_rows, row_len), dtype=np.float32)
    idx = np.empty((out_rows, k), dtype=np.int32)
    cnt = np.empty((out_rows,), dtype=np.int32)
    rc = lib.orc_tri_select(s.ctypes.data, layers, batch, groups, row_len, kl.ctypes.data, m, k,
                            z.ctypes.data, red.ctypes.data, idx.ctypes.data, cnt.ctypes.data)
    _check(rc, "tri_select")
    return {"z": z, "reduced": red, "indices": idx, "counts": cnt}


def multi_query_rows(block_table, kv_lens, next_n: int):
    """Multi-query decode as single-query rows: request b's query j (of
    next_n, the last next_n positions of its kv_len tokens) is row
    b*next_n + j, with request b's page table and the causal length
    kv_len - (next_n - 1 - j) ("Overlap DSA heuristic prev_topk write-back on
    the aux stream", Performance: the MTP decode setting)."""
    bt = np.repeat(np.asarray(block_table), next_n, axis=0)
    j = np.tile(np.arange(next_n), len(kv_lens))
    kl = np.maximum(np.repeat(np.asarray(kv_lens, dtype=np.int64), next_n) - (next_n - 1 - j), 0)
    return bt.astype(np.int32), kl.astype(np.int32)


def sparse_decode(w) -> dict:
    """The whole path on a workload object (see top_sparse_decode_amd.synth):
    score -> top-k -> attention.  Returns scores, indices, counts and the
    float64 output.  A multi-query workload (next_n > 1) runs as its
    single-query rows (multi_query_rows); outputs are request-major rows."""
    n = int(getattr(w, "next_n", 1))
    if n > 1:
        import dataclasses
        bt, kl = multi_query_rows(w.block_table, w.kv_lens, n)
        w = dataclasses.replace(w, block_table=bt, kv_lens=kl, next_n=1)
    s = score(w.block_table, w.kv_lens, w.score_k, w.score_q, w.head_weights, w.mode,
              w.head_scale, w.max_kv_len, getattr(w, "score_k_scale", None))
    idx, cnt = topk(s, w.kv_lens, w.topk)
    out = attention(w.block_table, w.kv_lens, w.q, w.k, w.v, w.v_dim, idx, w.softmax_scale)
    return {"scores": s, "indices": idx, "counts": cnt, "out": out}
