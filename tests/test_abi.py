"""The C ABI: the library loads, exports every entry point the header
declares, and rejects bad host-visible arguments before any GPU work (these
calls return before touching HIP, so they run without a GPU)."""
import ctypes
import os
import re

import pytest

from top_sparse_decode_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_decode.h")


def _lib():
    if not os.path.exists(api.LIB_PATH):
        from top_sparse_decode_amd import build
        build.build()
    return api.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:sd_status|const char\*|int32_t|size_t)\s+(sd_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("sd_sparse_score_paged", "sd_topk_select", "sd_sparse_decode_attn",
                 "sd_sparse_decode", "sd_local_to_global"):
        assert want in names
    assert sorted(api.EXPORTS) == names


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert lib.sd_version() == 2
    assert lib.sd_status_string(0) == b"ok"
    assert lib.sd_status_string(3) == b"workspace too small"


def _pool(data=4096, dtype=api.BF16, pages=8, P=64, H=1, D=128, scale=None):
    return api.sd_pool(data, dtype, pages, P, H, D, H * P * D, P * D, D, scale)


def _pages(batch=2, max_pages=4, max_kv_len=256):
    return api.sd_pages(8192, 12288, batch, max_pages, max_kv_len)


def _rc_score(pg, pool, q=16384, heads=64, w=20480, mode=api.RELU_WEIGHTED, scores=24576, q_dtype=None):
    lib = _lib()
    if q_dtype is None:
        q_dtype = api.BF16 if pool.dtype == api.FP8_E4M3 else pool.dtype
    return lib.sd_sparse_score_paged(ctypes.byref(pg), ctypes.byref(pool), q, q_dtype, heads, w,
                                     mode, 1.0, api.FAST, scores, None, 0)


def test_score_argument_validation():
    lib = _lib()
    assert _rc_score(_pages(), _pool(data=None)) == api.ERR_INVALID_ARGUMENT
    assert b"data is NULL" in lib.sd_last_error()
    assert _rc_score(_pages(), _pool(data=4104)) == api.ERR_INVALID_ARGUMENT     # misaligned
    assert _rc_score(_pages(), _pool(), q=None) == api.ERR_INVALID_ARGUMENT
    assert _rc_score(_pages(), _pool(), w=None) == api.ERR_INVALID_ARGUMENT
    assert _rc_score(_pages(), _pool(), heads=63) == api.ERR_UNSUPPORTED
    assert _rc_score(_pages(), _pool(H=2), heads=63) == api.ERR_INVALID_ARGUMENT
    assert _rc_score(_pages(max_kv_len=1000), _pool()) == api.ERR_INVALID_ARGUMENT  # > pages*P
    assert _rc_score(_pages(), _pool(), mode=7) == api.ERR_INVALID_ARGUMENT
    assert _rc_score(_pages(), _pool(), scores=None) == api.ERR_INVALID_ARGUMENT
    # zero-size batch is a no-op that needs no GPU
    assert _rc_score(_pages(batch=0), _pool()) == api.OK


def test_fp8_pool_validation():
    lib = _lib()
    fp8 = dict(dtype=api.FP8_E4M3)
    assert _rc_score(_pages(), _pool(**fp8)) == api.ERR_INVALID_ARGUMENT          # no scales
    assert b"scales" in lib.sd_last_error()
    assert _rc_score(_pages(), _pool(scale=4104, **fp8)) == api.ERR_INVALID_ARGUMENT  # misaligned
    assert _rc_score(_pages(), _pool(scale=8192)) == api.ERR_INVALID_ARGUMENT     # scales on a bf16 pool
    assert _rc_score(_pages(), _pool(D=120, scale=8192, **fp8)) == api.ERR_INVALID_ARGUMENT  # 120-byte rows
    assert _rc_score(_pages(), _pool(scale=8192, **fp8), q_dtype=api.F32) == api.ERR_UNSUPPORTED
    assert _rc_score(_pages(), _pool(scale=8192, **fp8), q_dtype=api.FP8_E4M3) == api.ERR_UNSUPPORTED
    assert _rc_score(_pages(batch=0), _pool(scale=8192, **fp8)) == api.OK
    # FP8 pools are scored, never attended
    n = ctypes.c_size_t(0)
    kp = _pool(D=576, scale=8192, **fp8)
    assert lib.sd_sparse_decode_attn_workspace_size(ctypes.byref(_pages()), 128, ctypes.byref(kp), 512,
                                                     2048, ctypes.byref(n)) == api.ERR_UNSUPPORTED
    # the fused step accepts an FP8 indexer pool beside a bf16 latent pool
    a = api.sd_sparse_decode_args()
    a.pages = _pages(batch=4, max_pages=64, max_kv_len=4096)
    a.score_k = api.sd_pool(4096, api.FP8_E4M3, 512, 64, 1, 128, 64 * 128, 64 * 128, 128, 8192)
    a.score_q_dtype, a.score_heads, a.mode, a.head_scale = api.BF16, 64, api.RELU_WEIGHTED, 1.0
    a.precision, a.topk = api.FAST, 2048
    a.q_dtype, a.q_heads = api.BF16, 128
    a.k = api.sd_pool(8192, api.BF16, 512, 64, 1, 576, 64 * 576, 64 * 576, 576)
    a.v = a.k
    a.v_dim, a.softmax_scale, a.out_dtype = 512, 0.0721, api.BF16
    assert lib.sd_sparse_decode_workspace_size(ctypes.byref(a), ctypes.byref(n)) == api.OK
    a.score_q_dtype = api.FP8_E4M3
    assert lib.sd_sparse_decode_workspace_size(ctypes.byref(a), ctypes.byref(n)) == api.ERR_UNSUPPORTED


def test_hinted_topk_argument_validation():
    lib = _lib()
    f = lib.sd_topk_select_hinted
    # (scores, batch, groups, row_stride, kv_lens, k, hint, hint_len, hint_stride, indices, counts,
    #  writeback, writeback_stride, workspace, workspace_bytes, stream)
    n = ctypes.c_size_t(0)
    assert lib.sd_topk_workspace_size(2, 1, 100, 8, ctypes.byref(n)) == api.OK
    def call(h=32, hl=8, hs=8, wb=48, wbs=8):
        return f(16, 2, 1, 100, 64, 8, h, hl, hs, 80, None, wb, wbs, 4096, n.value, 0)
    assert call(hl=-1) == api.ERR_INVALID_ARGUMENT          # negative hint length
    assert call(hl=9, hs=8) == api.ERR_INVALID_ARGUMENT     # stride below the length
    assert call(wbs=7) == api.ERR_INVALID_ARGUMENT          # write-back row shorter than k
    assert b"write-back" in lib.sd_last_error()
    # batch 0 is a no-op that needs no GPU, with or without a hint
    assert f(None, 0, 1, 100, None, 8, 32, 8, 8, None, None, 48, 8, None, 0, 0) == api.OK
    assert f(None, 0, 1, 100, None, 8, None, 0, 0, None, None, None, 0, None, 0, 0) == api.OK


def test_triattention_select_validation():
    lib = _lib()
    n = ctypes.c_size_t(0)
    ws = lib.sd_triattention_select_workspace_size
    assert ws(4, 2, 8, 4096, 2, 2048, ctypes.byref(n)) == api.OK
    assert n.value >= 2 * 4096 * 4            # the two reduced union rows at least
    assert ws(0, 2, 8, 4096, 2, 2048, ctypes.byref(n)) == api.ERR_INVALID_ARGUMENT   # no layers
    assert ws(4, 2, 8, 4096, 3, 2048, ctypes.byref(n)) == api.ERR_INVALID_ARGUMENT   # bad mode
    assert ws(4, 2, 8, 4096, 2, 0, ctypes.byref(n)) == api.ERR_INVALID_ARGUMENT      # k = 0
    assert ws(4, 2, 8, 300000, 2, 16, ctypes.byref(n)) == api.ERR_UNSUPPORTED        # row too long
    f = lib.sd_triattention_select
    assert ws(4, 2, 8, 4096, 1, 2048, ctypes.byref(n)) == api.OK
    assert f(16, 4, 2, 8, 4096, 32, 1, 2048, 48, None, None, 4096, n.value - 1, 0) == api.ERR_WORKSPACE_TOO_SMALL
    assert f(None, 4, 2, 8, 4096, 32, 1, 2048, 48, None, None, 4096, n.value, 0) == api.ERR_INVALID_ARGUMENT
    assert f(None, 4, 0, 8, 4096, None, 1, 2048, None, None, None, None, 0, 0) == api.OK  # empty batch


def test_block_attention_validation():
    lib = _lib()
    n = ctypes.c_size_t(0)
    kp = _pool(D=576)
    f = lib.sd_sparse_decode_attn_blocks_workspace_size
    assert f(ctypes.byref(_pages()), 128, ctypes.byref(kp), 512, 64, 32, ctypes.byref(n)) == api.OK
    assert n.value >= 2 * 64 * 32 * 4                                  # the expanded token lists
    assert f(ctypes.byref(_pages()), 128, ctypes.byref(kp), 512, 64, 0, ctypes.byref(n)) == api.ERR_INVALID_ARGUMENT
    assert f(ctypes.byref(_pages()), 128, ctypes.byref(kp), 512, 0, 32, ctypes.byref(n)) == api.ERR_INVALID_ARGUMENT
    assert f(ctypes.byref(_pages()), 128, ctypes.byref(kp), 512, 1 << 13, 1 << 12, ctypes.byref(n)) == api.ERR_INVALID_ARGUMENT
    g = lib.sd_sparse_decode_attn_blocks
    assert f(ctypes.byref(_pages()), 128, ctypes.byref(kp), 512, 64, 32, ctypes.byref(n)) == api.OK
    args = (ctypes.byref(_pages(max_kv_len=256)), 16384, api.BF16, 128, ctypes.byref(kp), ctypes.byref(kp), 512)
    assert g(*args, None, 64, 32, 0.07, 24576, api.BF16, 4096, n.value, 0) == api.ERR_INVALID_ARGUMENT
    assert g(*args, 20480, 64, 32, 0.07, 24576, api.BF16, 4096, n.value - 1, 0) == api.ERR_WORKSPACE_TOO_SMALL


def test_topk_argument_validation():
    lib = _lib()
    f = lib.sd_topk_select
    assert f(None, 2, 1, 100, 8, 10, 16, None, None, 0, 0) == api.ERR_INVALID_ARGUMENT
    assert f(16, 2, 1, 100, 8, 0, 16, None, None, 0, 0) == api.ERR_INVALID_ARGUMENT
    assert f(16, 2, 0, 100, 8, 4, 16, None, None, 0, 0) == api.ERR_INVALID_ARGUMENT
    assert f(None, 0, 1, 100, None, 4, None, None, None, 0, 0) == api.OK
    n = ctypes.c_size_t(7)
    assert lib.sd_topk_workspace_size(4, 2, 100, 8, ctypes.byref(n)) == api.OK
    assert n.value >= 4 * 2 * 100 * 4           # one key per score
    assert f(16, 4, 2, 100, 32, 8, 48, None, 4096, n.value - 1, 0) == api.ERR_WORKSPACE_TOO_SMALL
    assert f(16, 4, 2, 300000, 32, 8, 48, None, 4096, 1 << 30, 0) == api.ERR_UNSUPPORTED


def _attn(k=None, v=None, heads=128, v_dim=512, k_sel=2048, ws_bytes=0, q=16384, idx=20480, out=24576):
    lib = _lib()
    kp = k or _pool(D=576)
    vp = v or kp
    return lib.sd_sparse_decode_attn(ctypes.byref(_pages(max_kv_len=256)), q, api.BF16, heads,
                                     ctypes.byref(kp), ctypes.byref(vp), v_dim, idx, k_sel, 0.07,
                                     out, api.BF16, 4096 if ws_bytes else None, ws_bytes, 0)


def test_attention_argument_validation_and_workspace():
    lib = _lib()
    n = ctypes.c_size_t(0)
    kp = _pool(D=576)
    assert lib.sd_sparse_decode_attn_workspace_size(ctypes.byref(_pages()), 128, ctypes.byref(kp), 512,
                                                     2048, ctypes.byref(n)) == api.OK
    need = n.value
    assert need > 0
    assert _attn(ws_bytes=need - 1) == api.ERR_WORKSPACE_TOO_SMALL
    assert _attn(ws_bytes=need, q=None) == api.ERR_INVALID_ARGUMENT
    assert _attn(ws_bytes=need, k_sel=0) == api.ERR_INVALID_ARGUMENT
    assert _attn(ws_bytes=need, v_dim=600) == api.ERR_INVALID_ARGUMENT
    assert _attn(ws_bytes=need, heads=96) == api.ERR_UNSUPPORTED        # MLA wants 32/64/128 heads
    assert _attn(ws_bytes=need, v=_pool(data=8192, D=576)) == api.ERR_UNSUPPORTED  # MLA pools must alias
    assert _attn(ws_bytes=need, v=_pool(D=576, P=32)) == api.ERR_INVALID_ARGUMENT  # page sizes differ
    assert _attn(ws_bytes=need, k=_pool(D=64, H=2), v=_pool(D=64, H=2), heads=6, v_dim=64) == api.ERR_UNSUPPORTED


def test_fused_workspace_and_validation():
    lib = _lib()
    a = api.sd_sparse_decode_args()
    a.pages = _pages(batch=16, max_pages=1024, max_kv_len=65536)
    a.score_k = api.sd_pool(4096, api.BF16, 16384, 64, 1, 128, 64 * 128, 64 * 128, 128, None)
    a.score_q_dtype, a.score_heads, a.mode, a.head_scale = api.BF16, 64, api.RELU_WEIGHTED, 1.0
    a.precision, a.topk = api.FAST, 2048
    a.q_dtype, a.q_heads = api.BF16, 128
    a.k = api.sd_pool(8192, api.BF16, 16384, 64, 1, 576, 64 * 576, 64 * 576, 576, None)
    a.v = a.k
    a.v_dim, a.softmax_scale, a.out_dtype = 512, 0.0721, api.BF16
    n = ctypes.c_size_t(0)
    assert lib.sd_sparse_decode_workspace_size(ctypes.byref(a), ctypes.byref(n)) == api.OK
    # scores + refined scores (2 x 16 x 65536 floats) dominate
    assert n.value >= 2 * 16 * 65536 * 4
    # running needs the pointers the size query does not
    assert lib.sd_sparse_decode(ctypes.byref(a), 4096, n.value, 0) == api.ERR_INVALID_ARGUMENT
    a.topk = 0
    assert lib.sd_sparse_decode_workspace_size(ctypes.byref(a), ctypes.byref(n)) == api.ERR_INVALID_ARGUMENT
    a.topk = 2048
    a.k.page_size = 32
    a.v = a.k
    assert lib.sd_sparse_decode_workspace_size(ctypes.byref(a), ctypes.byref(n)) == api.ERR_INVALID_ARGUMENT


def test_noalloc_rejects_calls_beyond_its_scratch():
    # host-side checks only: nothing reaches a device.  Mixed-length DSA-MLA sizes (64
    # requests up to 131072 tokens) need more scratch than the library holds.
    lib = _lib()
    cap = lib.sd_sparse_decode_noalloc_max_bytes()
    assert cap == 64 << 20
    a = api.sd_sparse_decode_args()
    a.pages = api.sd_pages(8192, 12288, 64, 2048, 131072)
    a.score_k = api.sd_pool(4096, api.BF16, 140000, 64, 1, 128, 64 * 128, 64 * 128, 128, None)
    a.score_q, a.score_q_dtype, a.score_heads, a.head_weights = 16384, api.BF16, 64, 20480
    a.mode, a.head_scale, a.precision, a.topk = api.RELU_WEIGHTED, 1.0, api.FAST, 2048
    a.q, a.q_dtype, a.q_heads = 24576, api.BF16, 128
    a.k = api.sd_pool(8192, api.BF16, 140000, 64, 1, 576, 64 * 576, 64 * 576, 576, None)
    a.v = a.k
    a.v_dim, a.softmax_scale, a.out, a.out_dtype = 512, 0.0721, 32768, api.BF16
    n = ctypes.c_size_t(0)
    assert lib.sd_sparse_decode_workspace_size(ctypes.byref(a), ctypes.byref(n)) == api.OK
    assert n.value > cap
    assert lib.sd_sparse_decode_noalloc(ctypes.byref(a), None) == api.ERR_WORKSPACE_TOO_SMALL
    assert b"64 MiB" in lib.sd_last_error() or str(cap).encode() in lib.sd_last_error()
    # argument errors are reported before any size or device question
    a.topk = 0
    assert lib.sd_sparse_decode_noalloc(ctypes.byref(a), None) == api.ERR_INVALID_ARGUMENT


def test_local_to_global_validation():
    lib = _lib()
    pg = _pages()
    assert lib.sd_local_to_global(ctypes.byref(pg), 0, 8, 16, 1, 4, 32, 0) == api.ERR_INVALID_ARGUMENT
    assert lib.sd_local_to_global(ctypes.byref(pg), 64, 8, None, 1, 4, 32, 0) == api.ERR_INVALID_ARGUMENT


def test_missing_library_is_an_error(tmp_path):
    saved = api._lib
    api._lib = None
    try:
        with pytest.raises(RuntimeError, match="missing"):
            api.load(str(tmp_path / "nope.so"))
    finally:
        api._lib = saved
