"""Thin Python binding of libsparse_decode.so (include/sparse_decode.h).

Argument marshalling only: every step of the path runs in the HIP kernels of
the library.  PyTorch provides device memory and streams.  Function names
follow the C ABI without the ``sd_`` prefix; each takes torch tensors (device
memory) and enqueues on the current torch stream unless ``stream`` is given.

The library is loaded on first use and a missing library is an error -- there
is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsparse_decode.so")

OK, ERR_INVALID_ARGUMENT, ERR_UNSUPPORTED, ERR_WORKSPACE_TOO_SMALL, ERR_HIP = range(5)
F32, BF16, FP8_E4M3 = 0, 1, 2
GROUP_SUM, GROUP_MEAN, RELU_WEIGHTED = 0, 1, 2
EXACT, FAST = 0, 1
SELECT_MODES = {"per_layer_perhead": 0, "per_head": 1, "union": 2}
MODES = {"group_sum": GROUP_SUM, "group_mean": GROUP_MEAN, "relu_weighted": RELU_WEIGHTED}


class SparseDecodeError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({detail})")
        self.status = status


class sd_pool(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int), ("num_pages", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_stride", ctypes.c_int64),
                ("head_stride", ctypes.c_int64), ("token_stride", ctypes.c_int64),
                ("scale", ctypes.c_void_p)]


class sd_pages(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("kv_lens", ctypes.c_void_p),
                ("batch", ctypes.c_int32), ("max_pages", ctypes.c_int32),
                ("max_kv_len", ctypes.c_int32)]


class sd_sparse_decode_args(ctypes.Structure):
    _fields_ = [("pages", sd_pages), ("score_k", sd_pool), ("score_q", ctypes.c_void_p),
                ("score_q_dtype", ctypes.c_int), ("score_heads", ctypes.c_int32),
                ("head_weights", ctypes.c_void_p), ("mode", ctypes.c_int),
                ("head_scale", ctypes.c_float), ("precision", ctypes.c_int),
                ("topk", ctypes.c_int32), ("q", ctypes.c_void_p), ("q_dtype", ctypes.c_int),
                ("q_heads", ctypes.c_int32), ("k", sd_pool), ("v", sd_pool),
                ("v_dim", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("out", ctypes.c_void_p), ("out_dtype", ctypes.c_int),
                ("indices_out", ctypes.c_void_p), ("counts_out", ctypes.c_void_p),
                ("topk_hint", ctypes.c_void_p), ("hint_len", ctypes.c_int32),
                ("hint_stride", ctypes.c_int64), ("topk_writeback", ctypes.c_void_p),
                ("writeback_stride", ctypes.c_int64), ("next_n", ctypes.c_int32)]


EXPORTS = ["sd_sparse_score_paged", "sd_topk_workspace_size", "sd_topk_select", "sd_topk_select_hinted",
           "sd_sparse_decode_attn_workspace_size", "sd_sparse_decode_attn",
           "sd_sparse_decode_workspace_size", "sd_sparse_decode", "sd_local_to_global",
           "sd_triattention_select_workspace_size", "sd_triattention_select",
           "sd_sparse_decode_attn_blocks_workspace_size", "sd_sparse_decode_attn_blocks",
           "sd_sparse_decode_noalloc_max_bytes", "sd_sparse_decode_noalloc",
           "sd_status_string", "sd_last_error", "sd_version"]

_lib = None


def load(path: str = LIB_PATH):
    """Open the library (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing; build it with `python -m top_sparse_decode_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, F, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    PP = ctypes.POINTER(sd_pages)
    PL = ctypes.POINTER(sd_pool)
    PA = ctypes.POINTER(sd_sparse_decode_args)
    E = ctypes.c_int
    sig = {
        "sd_sparse_score_paged": [PP, PL, P, E, I32, P, E, F, E, P, P, P],
        "sd_topk_workspace_size": [I32, I32, I32, I32, ctypes.POINTER(SZ)],
        "sd_topk_select": [P, I32, I32, I32, P, I32, P, P, P, SZ, P],
        "sd_topk_select_hinted": [P, I32, I32, I32, P, I32, P, I32, ctypes.c_int64, P, P, P, ctypes.c_int64,
                                  P, SZ, P],
        "sd_sparse_decode_attn_workspace_size": [PP, I32, PL, I32, I32, ctypes.POINTER(SZ)],
        "sd_sparse_decode_attn": [PP, P, E, I32, PL, PL, I32, P, I32, F, P, E, P, SZ, P],
        "sd_sparse_decode_workspace_size": [PA, ctypes.POINTER(SZ)],
        "sd_sparse_decode": [PA, P, SZ, P],
        "sd_sparse_decode_noalloc": [PA, P],
        "sd_local_to_global": [PP, I32, I32, P, I32, I32, P, P],
        "sd_triattention_select_workspace_size": [I32, I32, I32, I32, E, I32, ctypes.POINTER(SZ)],
        "sd_sparse_decode_attn_blocks_workspace_size": [PP, I32, PL, I32, I32, I32, ctypes.POINTER(SZ)],
        "sd_sparse_decode_attn_blocks": [PP, P, E, I32, PL, PL, I32, P, I32, I32, F, P, E, P, SZ, P],
        "sd_triattention_select": [P, I32, I32, I32, I32, P, E, I32, P, P, P, P, SZ, P],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.sd_status_string.argtypes = [ctypes.c_int]
    lib.sd_status_string.restype = ctypes.c_char_p
    lib.sd_last_error.argtypes = []
    lib.sd_last_error.restype = ctypes.c_char_p
    lib.sd_version.argtypes = []
    lib.sd_version.restype = ctypes.c_int32
    lib.sd_sparse_decode_noalloc_max_bytes.argtypes = []
    lib.sd_sparse_decode_noalloc_max_bytes.restype = ctypes.c_size_t
    _lib = lib
    return lib


def _check(rc: int, where: str) -> None:
    if rc != OK:
        lib = load()
        raise SparseDecodeError(rc, where, lib.sd_last_error().decode() or lib.sd_status_string(rc).decode())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch

    return torch.cuda.current_stream().cuda_stream


def dtype_code(t) -> int:
    import torch

    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype in (torch.uint8, getattr(torch, "float8_e4m3fn", None)):
        return FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


# ------------------------------------------------------------------ descriptors

def pool(t, scale=None) -> sd_pool:
    """Describe a 4-D paged pool tensor [pages, kv_heads, page_size, head_dim]
    (HND; any strides with a contiguous last dim).  An FP8 E4M3 pool (uint8
    codes) takes its float32 row scales [pages, kv_heads, page_size]."""
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("pool must be 4-D [pages, kv_heads, page_size, head_dim] with contiguous rows")
    code = dtype_code(t)
    if code == FP8_E4M3:
        import torch

        if scale is None or scale.dtype != torch.float32 or tuple(scale.shape) != (t.shape[0], t.shape[1], t.shape[2]) \
                or not scale.is_contiguous():
            raise ValueError("an FP8 pool needs contiguous float32 scales [pages, kv_heads, page_size]")
    elif scale is not None:
        raise ValueError("scales are for FP8 pools only")
    return sd_pool(t.data_ptr(), code, t.shape[0], t.shape[2], t.shape[1], t.shape[3],
                   t.stride(0), t.stride(1), t.stride(2), None if scale is None else scale.data_ptr())


def pages(block_table, kv_lens, max_kv_len: int) -> sd_pages:
    return sd_pages(block_table.data_ptr(), kv_lens.data_ptr(), kv_lens.shape[0],
                    block_table.shape[1], int(max_kv_len))


# ------------------------------------------------------------------ entry points

def sparse_score_paged(pg: sd_pages, k_pool: sd_pool, q, q_heads: int, head_weights, mode: int,
                       head_scale: float, precision: int, scores, row_bound=None, stream=None):
    lib = load()
    rc = lib.sd_sparse_score_paged(ctypes.byref(pg), ctypes.byref(k_pool), _ptr(q), dtype_code(q),
                                   q_heads, _ptr(head_weights), mode, head_scale, precision,
                                   _ptr(scores), _ptr(row_bound), _stream(stream))
    _check(rc, "sd_sparse_score_paged")


def topk_workspace_size(batch: int, groups: int, row_stride: int, k: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().sd_topk_workspace_size(batch, groups, row_stride, k, ctypes.byref(n)),
           "sd_topk_workspace_size")
    return n.value


def topk_select(scores, batch: int, groups: int, row_stride: int, kv_lens, k: int, indices,
                counts=None, workspace=None, workspace_bytes: int = 0, stream=None):
    rc = load().sd_topk_select(_ptr(scores), batch, groups, row_stride, _ptr(kv_lens), k,
                               _ptr(indices), _ptr(counts), _ptr(workspace), workspace_bytes,
                               _stream(stream))
    _check(rc, "sd_topk_select")


def topk_select_hinted(scores, batch: int, groups: int, row_stride: int, kv_lens, k: int, hint,
                       indices, counts=None, writeback=None, workspace=None, workspace_bytes: int = 0,
                       stream=None):
    """hint and writeback are [batch, groups, n] int32 tensors (or None)."""
    hl = 0 if hint is None else int(hint.shape[-1])
    hs = 0 if hint is None else int(hint.stride(1))
    ws_ = 0 if writeback is None else int(writeback.stride(1))
    rc = load().sd_topk_select_hinted(_ptr(scores), batch, groups, row_stride, _ptr(kv_lens), k, _ptr(hint), hl,
                                      hs, _ptr(indices), _ptr(counts), _ptr(writeback), ws_, _ptr(workspace),
                                      workspace_bytes, _stream(stream))
    _check(rc, "sd_topk_select_hinted")


def sparse_decode_attn_workspace_size(pg: sd_pages, q_heads: int, k_pool: sd_pool, v_dim: int,
                                      k_sel: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().sd_sparse_decode_attn_workspace_size(ctypes.byref(pg), q_heads, ctypes.byref(k_pool),
                                                        v_dim, k_sel, ctypes.byref(n)),
           "sd_sparse_decode_attn_workspace_size")
    return n.value


def sparse_decode_attn(pg: sd_pages, q, q_heads: int, k_pool: sd_pool, v_pool: sd_pool, v_dim: int,
                       indices, k_sel: int, softmax_scale: float, out, workspace,
                       workspace_bytes: Optional[int] = None, stream=None):
    wb = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    rc = load().sd_sparse_decode_attn(ctypes.byref(pg), _ptr(q), dtype_code(q), q_heads,
                                      ctypes.byref(k_pool), ctypes.byref(v_pool), v_dim,
                                      _ptr(indices), k_sel, softmax_scale, _ptr(out), dtype_code(out),
                                      _ptr(workspace), wb, _stream(stream))
    _check(rc, "sd_sparse_decode_attn")


def sparse_decode_attn_blocks_workspace_size(pg: sd_pages, q_heads: int, k_pool: sd_pool, v_dim: int,
                                             k_blocks: int, block_size: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().sd_sparse_decode_attn_blocks_workspace_size(ctypes.byref(pg), q_heads, ctypes.byref(k_pool),
                                                               v_dim, k_blocks, block_size, ctypes.byref(n)),
           "sd_sparse_decode_attn_blocks_workspace_size")
    return n.value


def sparse_decode_attn_blocks(pg: sd_pages, q, q_heads: int, k_pool: sd_pool, v_pool: sd_pool, v_dim: int,
                              block_indices, k_blocks: int, block_size: int, softmax_scale: float, out,
                              workspace, workspace_bytes: Optional[int] = None, stream=None):
    wb = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    rc = load().sd_sparse_decode_attn_blocks(ctypes.byref(pg), _ptr(q), dtype_code(q), q_heads,
                                             ctypes.byref(k_pool), ctypes.byref(v_pool), v_dim,
                                             _ptr(block_indices), k_blocks, block_size, softmax_scale, _ptr(out),
                                             dtype_code(out), _ptr(workspace), wb, _stream(stream))
    _check(rc, "sd_sparse_decode_attn_blocks")


def sparse_decode_workspace_size(args: sd_sparse_decode_args) -> int:
    n = ctypes.c_size_t(0)
    _check(load().sd_sparse_decode_workspace_size(ctypes.byref(args), ctypes.byref(n)),
           "sd_sparse_decode_workspace_size")
    return n.value


def sparse_decode(args: sd_sparse_decode_args, workspace, workspace_bytes: Optional[int] = None,
                  stream=None):
    wb = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    rc = load().sd_sparse_decode(ctypes.byref(args), _ptr(workspace), wb, _stream(stream))
    _check(rc, "sd_sparse_decode")


def sparse_decode_noalloc_max_bytes() -> int:
    return int(load().sd_sparse_decode_noalloc_max_bytes())


def sparse_decode_noalloc(args: sd_sparse_decode_args, stream=None):
    """sd_sparse_decode on the library's own per-device scratch (no caller
    workspace, no allocation)."""
    rc = load().sd_sparse_decode_noalloc(ctypes.byref(args), _stream(stream))
    _check(rc, "sd_sparse_decode_noalloc")


def local_to_global(pg: sd_pages, page_size: int, num_pages: int, local, out, stream=None):
    b, g, k = local.shape
    rc = load().sd_local_to_global(ctypes.byref(pg), page_size, num_pages, _ptr(local), g, k,
                                   _ptr(out), _stream(stream))
    _check(rc, "sd_local_to_global")


def _select_mode(mode) -> int:
    return SELECT_MODES[mode] if isinstance(mode, str) else int(mode)


def triattention_select_workspace_size(layers: int, batch: int, groups: int, row_stride: int, mode,
                                       k: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().sd_triattention_select_workspace_size(layers, batch, groups, row_stride, _select_mode(mode),
                                                        k, ctypes.byref(n)),
           "sd_triattention_select_workspace_size")
    return n.value


def triattention_select(scores, kv_lens, mode, k: int, indices, counts=None, reduced=None, workspace=None,
                        workspace_bytes: Optional[int] = None, stream=None):
    """scores: [layers, batch, groups, row_stride] float32 tensor."""
    layers, batch, groups, row_stride = scores.shape
    wb = (0 if workspace is None else workspace.numel() * workspace.element_size()) \
        if workspace_bytes is None else workspace_bytes
    rc = load().sd_triattention_select(_ptr(scores), layers, batch, groups, row_stride, _ptr(kv_lens),
                                       _select_mode(mode), k, _ptr(indices), _ptr(counts), _ptr(reduced),
                                       _ptr(workspace), wb, _stream(stream))
    _check(rc, "sd_triattention_select")


def version() -> int:
    return int(load().sd_version())


# ------------------------------------------------------------------ workloads on the device

def to_device_array(a: np.ndarray, device="cuda"):
    """numpy float32 / uint16 (bfloat16 bits) / uint8 (FP8 codes) / int32 -> torch tensor on device."""
    import torch

    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


@dataclass
class DeviceStep:
    """Device copies of a workload and the argument block of one decode step."""

    block_table: object
    kv_lens: object
    score_k: object
    score_k_scale: object
    score_q: object
    head_weights: object
    q: object
    k: object
    v: object
    out: object
    indices: object
    counts: object
    workspace: object
    args: sd_sparse_decode_args
    workload: object
    hint: object = None

    def run(self, stream=None):
        sparse_decode(self.args, self.workspace, stream=stream)


def prepare(w, precision: int = FAST, device="cuda", out_dtype=None, hint: bool = False) -> DeviceStep:
    """Upload a host workload (see synth.Workload) and build the fused-step
    arguments, output buffers and workspace.  hint=True adds a persistent
    [batch, groups, topk] buffer that each step reads as its hint and
    overwrites with its own selection (the next step's hint); it starts at -1
    (no hint)."""
    import torch

    bt = to_device_array(w.block_table, device)
    kl = to_device_array(w.kv_lens, device)
    sk = to_device_array(w.score_k, device)
    sks = None if getattr(w, "score_k_scale", None) is None else to_device_array(w.score_k_scale, device)
    sq = to_device_array(w.score_q, device)
    hw = None if w.head_weights is None else to_device_array(w.head_weights, device)
    if w.score_k is w.k:
        k, q = sk, (sq if w.score_q is w.q else to_device_array(w.q, device))
    else:
        k, q = to_device_array(w.k, device), to_device_array(w.q, device)
    v = k if w.v is w.k else to_device_array(w.v, device)
    odt = out_dtype or (torch.float32 if w.out_dtype == "f32" else torch.bfloat16)
    n = int(getattr(w, "next_n", 1))
    B, Hq = w.q.shape[0], w.q.shape[1]   # B = requests * next_n decode rows
    groups = w.score_k.shape[1]
    out = torch.empty((B, Hq, w.v_dim), dtype=odt, device=device)
    idx = torch.empty((B, groups, w.topk), dtype=torch.int32, device=device)
    cnt = torch.empty((B, groups), dtype=torch.int32, device=device)
    pg = pages(bt, kl, w.max_kv_len)
    args = sd_sparse_decode_args()
    args.pages = pg
    args.score_k = pool(sk, sks)
    args.score_q = sq.data_ptr()
    args.score_q_dtype = dtype_code(sq)
    args.score_heads = w.score_q.shape[1]
    args.head_weights = None if hw is None else hw.data_ptr()
    args.mode = MODES[w.mode]
    args.head_scale = float(w.head_scale)
    args.precision = precision
    args.topk = w.topk
    args.q = q.data_ptr()
    args.q_dtype = dtype_code(q)
    args.q_heads = Hq
    args.k = pool(k)
    args.v = pool(v)
    args.v_dim = w.v_dim
    args.softmax_scale = float(w.softmax_scale)
    args.out = out.data_ptr()
    args.out_dtype = dtype_code(out)
    args.indices_out = idx.data_ptr()
    args.counts_out = cnt.data_ptr()
    args.next_n = n
    hbuf = None
    if hint:
        hbuf = torch.full((B, groups, w.topk), -1, dtype=torch.int32, device=device)
        args.topk_hint = hbuf.data_ptr()
        args.hint_len = w.topk
        args.hint_stride = w.topk
        args.topk_writeback = hbuf.data_ptr()
        args.writeback_stride = w.topk
    nbytes = sparse_decode_workspace_size(args)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)
    return DeviceStep(bt, kl, sk, sks, sq, hw, q, k, v, out, idx, cnt, ws, args, w, hbuf)
