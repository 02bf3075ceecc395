"""Pins for the CPU oracle: each check ties it to something other than itself
(hand-derived closed forms, exact rational arithmetic, brute-force rank
definitions, a library SDPA, and invariants the method implies), chosen so
that a plausible slip -- a dropped term, a wrong index or sign, a transposed
operand, a different summation order, FMA contraction, the wrong tie rule --
fails at least one of them.  CPU only."""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from top_sparse_decode_amd import synth

F32 = np.float32


# ----------------------------------------------------------------- helpers

def paged(rows: np.ndarray, page_size: int, perm=None, num_pages=None, fill=np.nan):
    """Lay logical rows [B, Hkv, L, D] into an HND pool through a block table.
    perm: physical page for each (b, logical page) in order; default identity."""
    B, H, L, D = rows.shape
    npg = (L + page_size - 1) // page_size
    total = B * npg
    if perm is None:
        perm = np.arange(total)
    num_pages = num_pages or total
    if rows.dtype == np.uint16 and isinstance(fill, float):
        fill = synth.BF16_NAN
    pool = np.full((num_pages, H, page_size, D), fill, dtype=rows.dtype)
    bt = np.asarray(perm, dtype=np.int32).reshape(B, npg)
    for b in range(B):
        for t in range(L):
            pool[bt[b, t // page_size], :, t % page_size, :] = rows[b, :, t, :]
    return pool, bt


def bf16(x):
    return synth.to_bf16_bits(np.asarray(x, dtype=F32))


def exact_dot(q, k):
    return sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(q, k))


def rank_select(s, k):
    """O(L^2) definition: t is kept iff fewer than k tokens beat it under
    (score desc, index asc)."""
    L = len(s)
    keep = [t for t in range(L)
            if sum(1 for u in range(L) if s[u] > s[t] or (s[u] == s[t] and u < t)) < k]
    return keep


# ----------------------------------------------------------------- scoring

def _score_1tok(q_rows, k_row, mode="group_sum", head_scale=1.0, w=None, dtype=F32):
    q = np.asarray(q_rows, dtype=F32)[None]                 # [1, H, D]
    k = np.asarray(k_row, dtype=F32)[None, None, None, :]   # [1 page, 1 kvh, 1 slot, D]
    if dtype == np.uint16:
        q, k = bf16(q), bf16(k)
    bt = np.zeros((1, 1), dtype=np.int32)
    s = oracle.score(bt, [1], k, q, None if w is None else np.asarray(w, F32)[None], mode,
                     head_scale, 1)
    return s[0, 0, 0]


def test_sequential_order_closed_form():
    # terms 1e8, 1, -1e8, 1 (all exact in fp32).  Left to right, each sum
    # rounded: 1e8; 1e8+1 -> 1e8 (ulp 8); 0; 1.  A pairwise tree gives 0, the
    # exact value is 2.
    s = _score_1tok([[1, 1, 1, 1]], [1e8, 1, -1e8, 1])
    assert s == F32(1.0)
    # 2^24 followed by 63 ones: each +1 is a tie that rounds to even (2^24),
    # so the left-to-right result stays 2^24 (blocked orders give 2^24+64).
    k = [2.0 ** 24] + [1.0] * 63
    assert _score_1tok([[1.0] * 64], k) == F32(2.0 ** 24)


def test_no_fma_contraction_closed_form():
    # q = [1, 1+2^-12], k = [-(1+2^-11), 1+2^-12].  q1*k1 = 1+2^-11+2^-24 is a
    # tie that rounds to even 1+2^-11, so the separately rounded sum is +0; an
    # FMA would keep the 2^-24.
    a = 1.0 + 2.0 ** -12
    s = _score_1tok([[1.0, a]], [-(1.0 + 2.0 ** -11), a])
    assert s == F32(0.0)


@pytest.mark.parametrize("mode", ["group_sum", "group_mean", "relu_weighted"])
def test_integer_inputs_exact(mode):
    # integer q, k in [-3, 3]: every partial sum is a small integer, exact in
    # fp32 in any order, so the oracle must equal exact rational arithmetic.
    rs = np.random.default_rng(7)
    B, Hq, Hkv, L, D, P = 2, 8, 2, 37, 64, 8
    G = Hq // Hkv
    q = rs.integers(-3, 4, size=(B, Hq, D)).astype(F32)
    rows = rs.integers(-3, 4, size=(B, Hkv, L, D)).astype(F32)
    w = (rs.integers(0, 9, size=(B, Hq)) / 8.0).astype(F32)       # dyadic: products exact
    pool, bt = paged(bf16(rows), P, perm=rs.permutation(B * ((L + P - 1) // P)))
    hs = 0.125 if mode == "group_sum" else 1.0
    got = oracle.score(bt, [L] * B, pool, bf16(q), w if mode == "relu_weighted" else None, mode,
                       hs, L)
    for b in range(B):
        for g in range(Hkv):
            for t in range(L):
                dots = [exact_dot(q[b, g * G + j], rows[b, g, t]) for j in range(G)]
                if mode == "group_sum":
                    ref = sum(d * Fraction(hs) for d in dots)
                elif mode == "group_mean":
                    ref = sum(dots) / G
                else:
                    ref = sum(Fraction(float(w[b, g * G + j])) * max(d, 0) for j, d in enumerate(dots))
                assert Fraction(float(got[b, g, t])) == ref, (b, g, t)


def test_random_scores_within_rounding_bound():
    # Real-valued fp32 inputs: |oracle - exact| <= gamma_D * sum|q_d k_d| per
    # head, the bound any binary32 evaluation of the sum obeys.  Catches a
    # dropped or doubled term, a sign slip, or the wrong operand pairing.
    rs = np.random.default_rng(11)
    B, Hq, L, D = 1, 4, 50, 64
    q = rs.standard_normal((B, Hq, D)).astype(F32)
    rows = rs.standard_normal((B, 1, L, D)).astype(F32)
    pool, bt = paged(rows, 16, perm=[3, 0, 2, 1])
    got = oracle.score(bt, [L], pool, q, None, "group_sum", 0.125, L)
    u = 2.0 ** -24
    gam = lambda n: n * u / (1 - n * u)
    for t in range(L):
        ex = sum(exact_dot(q[0, h], rows[0, 0, t]) * Fraction(1, 8) for h in range(Hq))
        mag = sum(sum(abs(float(a) * float(c)) for a, c in zip(q[0, h], rows[0, 0, t])) / 8
                  for h in range(Hq))
        assert abs(float(Fraction(float(got[0, 0, t])) - ex)) <= gam(D + Hq) * mag * 1.01


def test_dsa_unit_weight_reduces_to_single_head_relu():
    # w = e_j: the DSA score is exactly max(q_j . k, 0) with that head's dot
    # product; every token with a non-positive dot ties at 0.
    rs = np.random.default_rng(3)
    B, H, L, D, P = 1, 6, 40, 16, 8
    j = 4
    q = rs.integers(-3, 4, size=(B, H, D)).astype(F32)
    rows = rs.integers(-3, 4, size=(B, 1, L, D)).astype(F32)
    w = np.zeros((B, H), F32)
    w[0, j] = 1.0
    pool, bt = paged(bf16(rows), P)
    got = oracle.score(bt, [L], pool, bf16(q), w, "relu_weighted", 1.0, L)[0, 0]
    ref = [max(int(exact_dot(q[0, j], rows[0, 0, t])), 0) for t in range(L)]
    assert [float(x) for x in got] == [float(r) for r in ref]
    # selection on those scores follows the rank definition, ties by lowest index
    idx, cnt = oracle.topk(got[None, None], [L], 10)
    assert list(idx[0, 0]) == rank_select(ref, 10)


def test_scores_past_kv_len_are_minus_inf():
    rs = np.random.default_rng(5)
    rows = rs.standard_normal((1, 1, 20, 8)).astype(F32)
    pool, bt = paged(rows, 8)
    s = oracle.score(bt, [13], pool, rs.standard_normal((1, 1, 8)).astype(F32), None,
                     "group_sum", 1.0, 24)
    assert np.all(np.isfinite(s[0, 0, :13])) and np.all(s[0, 0, 13:] == -np.inf)


# ----------------------------------------------------------------- selection

@pytest.mark.parametrize("L,k,levels", [(40, 7, 3), (64, 64, 5), (33, 1, 4), (50, 49, 2),
                                        (17, 30, 3), (64, 16, 1000)])
def test_topk_matches_rank_definition(L, k, levels):
    rs = np.random.default_rng(L * 100 + k)
    s = (rs.integers(0, levels, size=(2, 3, L)) - levels // 2).astype(F32)
    s[0, 0, ::5] = -0.0          # -0 and +0 must compare equal
    idx, cnt = oracle.topk(s, [L, L - 3], k)
    for b, LL in enumerate([L, L - 3]):
        for g in range(3):
            keep = rank_select(list(s[b, g, :LL]), k)
            n = len(keep)
            assert cnt[b, g] == n == min(k, LL)
            assert list(idx[b, g, :n]) == keep
            assert np.all(idx[b, g, n:] == -1)


def test_topk_all_equal_takes_first_k_and_k1_is_lowest_argmax():
    s = np.zeros((1, 1, 30), F32)
    idx, _ = oracle.topk(s, [30], 5)
    assert list(idx[0, 0]) == [0, 1, 2, 3, 4]
    s = np.array([[[1, 5, 2, 5, 5, -1]]], F32)
    idx, _ = oracle.topk(s, [6], 1)
    assert list(idx[0, 0]) == [1]


def test_topk_dense_equivalent_and_empty():
    s = np.random.default_rng(0).standard_normal((2, 1, 16)).astype(F32)
    idx, cnt = oracle.topk(s, [5, 0], 8)
    assert list(idx[0, 0]) == [0, 1, 2, 3, 4, -1, -1, -1] and cnt[0, 0] == 5
    assert np.all(idx[1, 0] == -1) and cnt[1, 0] == 0


def test_topk_rejects_nan_inside_kv_len():
    s = np.zeros((1, 1, 8), F32)
    s[0, 0, 3] = np.nan
    with pytest.raises(ValueError):
        oracle.topk(s, [8], 2)
    s[0, 0, 3] = 0
    s[0, 0, 6:] = np.nan   # past kv_len: ignored
    oracle.topk(s, [6], 2)


# ----------------------------------------------------------------- attention

def _gather_logical(pool, bt, L, g):
    """numpy gather of the logical rows [L, D] of one (request 0, KV head g)."""
    P = pool.shape[2]
    return np.stack([pool[bt[0, t // P], g, t % P] for t in range(L)])


def _sdpa64(q, k, v, scale):
    qt = torch.from_numpy(q.astype(np.float64))[None, None, None]
    kt = torch.from_numpy(k.astype(np.float64))[None, None]
    vt = torch.from_numpy(v.astype(np.float64))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)[0, 0, 0].numpy()


@pytest.mark.parametrize("mla", [False, True])
def test_full_selection_equals_sdpa(mla):
    # k >= L: sparse attention is dense attention; compare with PyTorch SDPA in
    # float64 over contiguously gathered rows.
    rs = np.random.default_rng(21 + mla)
    L, P = 45, 16
    Hq, Hkv, D, Dv = (8, 1, 96, 64) if mla else (4, 2, 32, 32)
    rows_k = rs.standard_normal((1, Hkv, L, D)).astype(F32)
    rows_v = rows_k if mla else rs.standard_normal((1, Hkv, L, Dv)).astype(F32)
    q = rs.standard_normal((1, Hq, D)).astype(F32)
    perm = rs.permutation(3)
    kp, bt = paged(bf16(rows_k), P, perm=perm)
    vp = kp if mla else paged(bf16(rows_v), P, perm=perm)[0]
    qb = bf16(q)
    idx = np.tile(np.arange(64, dtype=np.int32), (1, Hkv, 1))
    idx[idx >= L] = -1
    scale = 1.0 / np.sqrt(D)
    out = oracle.attention(bt, [L], qb, kp, vp, Dv, idx, scale)
    G = Hq // Hkv
    for h in range(Hq):
        g = h // G
        K = synth.bf16_bits_to_f32(_gather_logical(kp, bt, L, g))
        V = synth.bf16_bits_to_f32(_gather_logical(vp, bt, L, g))[:, :Dv]
        ref = _sdpa64(synth.bf16_bits_to_f32(qb[0, h]), K, V, float(F32(scale)))
        np.testing.assert_allclose(out[0, h], ref, rtol=1e-12, atol=1e-12)


def test_single_selection_returns_that_value_row():
    rs = np.random.default_rng(2)
    rows = rs.standard_normal((1, 1, 24, 16)).astype(F32)
    vrows = rs.standard_normal((1, 1, 24, 16)).astype(F32)
    kp, bt = paged(rows, 8, perm=[2, 0, 1])
    vp, _ = paged(vrows, 8, perm=[2, 0, 1])
    idx = np.full((1, 1, 4), -1, np.int32)
    idx[0, 0, 2] = 17
    out = oracle.attention(bt, [24], rs.standard_normal((1, 3, 16)).astype(F32), kp, vp, 16, idx, 0.3)
    for h in range(3):
        assert np.array_equal(out[0, h], vrows[0, 0, 17].astype(np.float64))


def test_value_pool_with_its_own_layout():
    # V in an NHD pool ([pages, page_size, kv_heads, width] memory order) of a
    # different row width than K: every value read must go through V's own
    # strides.  k >= L again, so the result is SDPA over the gathered rows.
    rs = np.random.default_rng(31)
    L, P, Hkv, Hq, D, W, Dv = 24, 8, 2, 4, 16, 24, 20
    rows_k = rs.standard_normal((1, Hkv, L, D)).astype(F32)
    rows_v = rs.standard_normal((1, Hkv, L, W)).astype(F32)
    kp, bt = paged(rows_k, P, perm=[2, 0, 1])
    vh, _ = paged(rows_v, P, perm=[2, 0, 1])
    vp = np.ascontiguousarray(vh.transpose(0, 2, 1, 3)).transpose(0, 2, 1, 3)   # NHD strides
    assert vp.strides != vh.strides
    q = rs.standard_normal((1, Hq, D)).astype(F32)
    idx = np.tile(np.arange(L, dtype=np.int32), (1, Hkv, 1))
    out = oracle.attention(bt, [L], q, kp, vp, Dv, idx, 0.25)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        ref = _sdpa64(q[0, h], rows_k[0, g], rows_v[0, g, :, :Dv], 0.25)
        np.testing.assert_allclose(out[0, h], ref, rtol=1e-12, atol=1e-12)


def test_zero_query_gives_mean_of_selected_values():
    rs = np.random.default_rng(4)
    rows = rs.standard_normal((1, 1, 32, 8)).astype(F32)
    vrows = rs.standard_normal((1, 1, 32, 8)).astype(F32)
    kp, bt = paged(rows, 8)
    vp, _ = paged(vrows, 8)
    sel = np.array([[[3, 9, 10, 31, -1]]], np.int32)
    out = oracle.attention(bt, [32], np.zeros((1, 2, 8), F32), kp, vp, 8, sel, 1.0)
    ref = vrows[0, 0, [3, 9, 10, 31]].astype(np.float64).mean(axis=0)
    np.testing.assert_allclose(out[0, 0], ref, rtol=1e-14, atol=1e-15)


def test_mla_zero_rope_equals_mqa_on_latent():
    # A 576-wide latent row with a zero rope part and a query whose rope part
    # is arbitrary gives the same result as MQA over the 512-wide latent.
    rs = np.random.default_rng(9)
    L, P = 20, 8
    lat = rs.standard_normal((1, 1, L, 576)).astype(F32)
    lat[..., 512:] = 0
    q = rs.standard_normal((1, 4, 576)).astype(F32)
    kp, bt = paged(bf16(lat), P)
    kp512, _ = paged(bf16(lat[..., :512]), P)
    q512 = np.ascontiguousarray(bf16(q)[..., :512])
    sel = np.array([[[0, 4, 7, 11, 19, -1]]], np.int32)
    a = oracle.attention(bt, [L], bf16(q), kp, kp, 512, sel, 0.07)
    b = oracle.attention(bt, [L], q512, kp512, kp512, 512, sel, 0.07)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-13)


def test_empty_selection_gives_zero_output():
    rows = np.ones((1, 1, 8, 4), F32)
    kp, bt = paged(rows, 8)
    out = oracle.attention(bt, [0], np.ones((1, 1, 4), F32), kp, kp, 4,
                           np.full((1, 1, 3), -1, np.int32), 1.0)
    assert np.all(out == 0)


def test_attention_rejects_index_past_kv_len():
    rows = np.ones((1, 1, 8, 4), F32)
    kp, bt = paged(rows, 8)
    with pytest.raises(ValueError):
        oracle.attention(bt, [5], np.ones((1, 1, 4), F32), kp, kp, 4,
                         np.array([[[1, 6]]], np.int32), 1.0)


# ----------------------------------------------------------------- whole path

def _run(w):
    return oracle.sparse_decode(w)


def _repage(w, new_P=None, perm_seed=None):
    """Same logical content with another page size or page placement."""
    P = w.page_size
    B, L = w.batch, int(w.kv_lens.max())

    def logical(pool):
        H, D = pool.shape[1], pool.shape[3]
        out = np.empty((B, H, L, D), pool.dtype)
        for b in range(B):
            for t in range(L):
                out[b, :, t] = pool[w.block_table[b, t // P], :, t % P]
        return out

    nP = new_P or P
    npg = (L + nP - 1) // nP
    perm = np.arange(B * npg)
    if perm_seed is not None:
        perm = np.random.default_rng(perm_seed).permutation(B * npg)
    fill = synth.BF16_NAN if w.k.dtype == np.uint16 else np.nan
    sk, bt = paged(logical(w.score_k), nP, perm=perm, fill=fill)
    k = paged(logical(w.k), nP, perm=perm, fill=fill)[0]
    v = k if w.v is w.k else paged(logical(w.v), nP, perm=perm, fill=fill)[0]
    import dataclasses
    return dataclasses.replace(w, page_size=nP, block_table=bt, score_k=sk, k=k, v=v)


@pytest.mark.parametrize("cfg,kw", [
    (1, dict(kv_len=256, topk=40)),
    (2, dict(batch=2, q_heads=3, kv_heads=3, kv_len=192, topk=70)),
    (3, dict(batch=2, q_heads=8, kv_heads=2, kv_len=320, topk=100)),
    (4, dict(batch=2, idx_heads=8, heads=4, kv_len=256, topk=64)),
])
def test_block_table_permutation_and_page_size_invariance(cfg, kw):
    w = synth.make_workload(cfg, **kw)
    base = _run(w)
    for variant in (_repage(w, perm_seed=99), _repage(w, new_P=w.page_size // 2, perm_seed=5),
                    _repage(w, new_P=w.page_size * 2)):
        r = _run(variant)
        assert np.array_equal(r["scores"], base["scores"])
        assert np.array_equal(r["indices"], base["indices"])
        assert np.array_equal(r["out"], base["out"])


def test_canaries_do_not_leak():
    w = synth.make_workload(5, batch=3, min_len=100, max_len=700, topk=64, idx_heads=8, heads=4)
    assert np.isnan(synth.bf16_bits_to_f32(w.k)).any()          # canaries are present
    r = _run(w)
    assert np.all(np.isfinite(r["out"]))
    for b in range(w.batch):
        L = int(w.kv_lens[b])
        assert np.all(np.isfinite(r["scores"][b, 0, :L]))


def test_dense_equivalent_when_kv_len_at_most_k():
    w = synth.make_workload(4, batch=3, idx_heads=8, heads=4, kv_len=[1, 100, 64], topk=100)
    r = _run(w)
    assert list(r["counts"][:, 0]) == [1, 100, 64]
    assert list(r["indices"][1, 0]) == list(range(100))
    assert list(r["indices"][2, 0, :64]) == list(range(64)) and np.all(r["indices"][2, 0, 64:] == -1)


def test_tiny_config_keeps_heavy_tokens():
    # The tiny workload plants 8 heavy tokens whose keys lean towards the
    # summed query; they must all survive selection.
    w = synth.make_workload(1)
    r = _run(w)
    s = r["scores"][0, 0]
    top8 = np.argsort(-s, kind="stable")[:8]
    assert set(top8).issubset(set(r["indices"][0, 0]))
    assert r["counts"][0, 0] == 128


# ----------------------------------------------------------------- index conversion

def test_local_to_global_by_hand():
    bt = np.array([[5, 2, -1], [0, 9, 3]], np.int32)      # page 9 is outside a 6-page pool
    loc = np.array([[[0, 3, 4, 7, 8, -1]], [[1, 4, 5, 11, 12, 2]]], np.int32)
    got = oracle.local_to_global(bt, 4, 6, loc)
    # request 0: t=0 -> 5*4+0, t=3 -> 23, t=4 -> page 2 -> 8, t=7 -> 11, t=8 -> page -1 -> -1
    # request 1: t=1 -> 1, t=4 -> page 9 (out of pool) -> -1, 5 -> -1, 11 -> page 3 -> 15,
    #            t=12 -> past the table -> -1, t=2 -> 2
    assert got.tolist() == [[[20, 23, 8, 11, -1, -1]], [[1, -1, -1, 15, -1, 2]]]


# ----------------------------------------------------------------- FP8 indexer pools

def _fp8_values(codes):
    """Score one-hot queries against one FP8 row of the given codes with unit
    scale: dot = decode(code) exactly (one nonzero product, exact sums)."""
    codes = np.asarray(codes, dtype=np.uint8)
    D = len(codes)
    pool = codes[None, None, None, :]
    scale = np.ones((1, 1, 1), dtype=F32)
    q = np.eye(D, dtype=F32)[None]                              # [1, D heads, D]
    bt = np.zeros((1, 1), dtype=np.int32)
    # group_sum with G = D heads on one KV head would add them up; score each
    # head alone instead (one query head per call)
    out = []
    for d in range(D):
        s = oracle.score(bt, [1], pool, q[:, d:d + 1, :], None, "group_sum", 1.0, 1, k_scale=scale)
        out.append(s[0, 0, 0])
    return np.array(out, dtype=np.float64)


def test_fp8_e4m3_decode_facts():
    # OCP FP8 E4M3: bias 7, 3 mantissa bits, subnormal step 2^-9, max 448,
    # S.1111.111 is NaN.  Spot values, then the spacing inside every binade.
    spot = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
            0x3F: 1.875, 0x40: 2.0, 0x77: 240.0, 0x7D: 416.0, 0x7E: 448.0,
            0xB8: -1.0, 0xFE: -448.0}
    got = _fp8_values(list(spot))
    assert list(got) == list(spot.values())
    pos = _fp8_values(list(range(0x00, 0x7F)))       # every finite non-negative code
    neg = _fp8_values(list(range(0x80, 0xFF)))
    assert np.array_equal(neg, -pos)                  # sign-magnitude
    steps = np.diff(pos)
    assert np.all(steps[:8] == 2.0 ** -9)             # subnormals and the step into 2^-6
    for e in range(1, 16):                            # binade e: codes 8e .. 8e+7 (8e+7 < 0x7F)
        lo, hi = 8 * e, min(8 * e + 7, 0x7E)
        assert np.all(np.diff(pos[lo:hi + 1]) == 2.0 ** (e - 10)), e
    nan = _fp8_values([0x7F, 0xFF])
    assert np.all(np.isnan(nan))


def test_fp8_pool_scores_as_dequantized_f32_pool():
    # dequantize-then-score: the FP8 row (codes c, scale s) scores exactly as
    # the binary32 row decode(c) * s, one binary32 rounding per element
    w = synth.make_workload(4, batch=2, kv_len=[300, 77], idx_heads=8, heads=4, topk=32,
                            index_dtype="fp8")
    s8 = oracle.score(w.block_table, w.kv_lens, w.score_k, w.score_q, w.head_weights, w.mode,
                      1.0, w.max_kv_len, k_scale=w.score_k_scale)
    # decode table from the one-hot scores (a NaN code in the row would turn
    # every product with it into NaN, so the two NaN codes are left out)
    fin = [c for c in range(256) if c not in (0x7F, 0xFF)]
    table = np.full(256, np.nan, dtype=F32)
    table[fin] = _fp8_values(fin).astype(F32)
    deq = table[w.score_k] * w.score_k_scale[..., None].astype(F32)   # numpy float32 product
    qf = synth.bf16_bits_to_f32(w.score_q)
    s32 = oracle.score(w.block_table, w.kv_lens, deq.astype(F32), qf, w.head_weights, w.mode,
                       1.0, w.max_kv_len)
    assert np.array_equal(s8.view(np.uint32), s32.view(np.uint32))
    # a dropped or misplaced scale would change the scores
    s_unit = oracle.score(w.block_table, w.kv_lens, w.score_k, w.score_q, w.head_weights, w.mode,
                          1.0, w.max_kv_len, k_scale=np.ones_like(w.score_k_scale))
    assert not np.array_equal(s_unit, s8)


def test_fp8_pool_scale_follows_the_page():
    # permuting physical pages (codes and scales together) changes nothing
    w = synth.make_workload(4, batch=2, kv_len=[500, 190], idx_heads=8, heads=4, topk=32,
                            index_dtype="fp8")
    base = oracle.score(w.block_table, w.kv_lens, w.score_k, w.score_q, w.head_weights, w.mode,
                        1.0, w.max_kv_len, k_scale=w.score_k_scale)
    perm = np.random.default_rng(7).permutation(w.score_k.shape[0])
    inv = np.argsort(perm)
    k2, s2 = w.score_k[perm], w.score_k_scale[perm]
    bt2 = np.where(w.block_table >= 0, inv[np.maximum(w.block_table, 0)], -1).astype(np.int32)
    got = oracle.score(bt2, w.kv_lens, k2, w.score_q, w.head_weights, w.mode, 1.0, w.max_kv_len,
                       k_scale=s2)
    assert np.array_equal(got.view(np.uint32), base.view(np.uint32))


# ---------------------------------------------------------------- TriAttention modes

def test_tri_normalize_is_the_population_zscore_of_finite_scores():
    # against numpy's float64 mean / population std over the finite scores
    rs = np.random.default_rng(31)
    s = (rs.standard_normal((1, 2, 3, 5000)) * 7 + 40).astype(F32)
    s[0, 1, 2, 100:140] = -np.inf                      # absent tokens: left out of the statistics
    kv = np.array([5000, 3001], np.int32)
    z = oracle.tri_select(s, kv, "per_layer_perhead", 16)["z"]
    for b in range(2):
        L = int(kv[b])
        for g in range(3):
            row = s[0, b, g, :L].astype(np.float64)
            fin = np.isfinite(row)
            ref = (row - row[fin].mean()) / row[fin].std()   # ddof=0: population
            got = z[0, b, g, :L]
            assert np.allclose(got[fin], ref[fin], rtol=2e-7, atol=2e-7)
            assert np.all(got[~fin] == -np.inf)
            assert np.all(z[0, b, g, L:] == -np.inf)


def test_tri_normalize_bitwise_where_every_order_is_exact():
    # small integers over a power-of-two length: the mean and the squared
    # deviations are exact dyadic sums in any order, so numpy's float64
    # result, rounded once to float32, is the exact definition
    rs = np.random.default_rng(32)
    s = rs.integers(-8, 9, size=(2, 1, 2, 512)).astype(F32)
    kv = np.array([512], np.int32)
    z = oracle.tri_select(s, kv, "per_layer_perhead", 8)["z"]
    x = s.astype(np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    sd = np.sqrt(((x - mu) ** 2).mean(axis=-1, keepdims=True))
    ref = ((x - mu) / sd).astype(F32)
    assert np.array_equal(z.view(np.uint32), ref.view(np.uint32))
    # scaling every score by 4 scales mean and deviation exactly: same z bits
    z4 = oracle.tri_select(s * F32(4), kv, "per_layer_perhead", 8)["z"]
    assert np.array_equal(z4.view(np.uint32), z.view(np.uint32))


def test_exact_sum_is_the_correctly_rounded_real_sum():
    # fractions.Fraction holds the exact real sum; float() of a Fraction is the
    # nearest binary64 (CPython divides the integers with correct rounding)
    from fractions import Fraction
    import math
    rs = np.random.default_rng(34)
    for trial in range(40):
        n = int(rs.integers(1, 400))
        mant = rs.standard_normal(n)
        expo = rs.integers(-60, 61, size=n) if trial % 2 else rs.integers(-1074, 1000, size=n)
        v = np.ldexp(mant, expo)
        v = v[np.isfinite(v)]
        want = float(sum((Fraction(float(x)) for x in v), Fraction(0)))
        got = oracle.exact_sum(v)
        assert got == want, trial
        assert got == math.fsum(v), trial
    # ties go to the even neighbour: 2^53 + 1 and 2^53 + 3 lie halfway
    t = 2.0 ** 53
    assert oracle.exact_sum([t, 1.0]) == t
    assert oracle.exact_sum([t + 2, 1.0]) == t + 4
    assert oracle.exact_sum([t, 1.0, 2.0 ** -1074]) == t + 2      # a sticky bit breaks the tie upward
    # cancellation and intermediate overflow do not enter
    assert oracle.exact_sum([2.0 ** 60, 1.0, -(2.0 ** 60), 3.0]) == 4.0
    assert oracle.exact_sum([1e308, 1e308, -1e308]) == 1e308
    m = np.finfo(np.float64).max
    assert oracle.exact_sum([m, m, -m, -m, 5.0]) == 5.0
    # subnormal steps are kept exactly
    assert oracle.exact_sum([2.0 ** -1074] * 3) == 3 * 2.0 ** -1074
    assert oracle.exact_sum([2.0 ** -1022, -(2.0 ** -1074)]) == 2.0 ** -1022 - 2.0 ** -1074
    assert oracle.exact_sum([]) == 0.0 and oracle.exact_sum([5.0, -5.0]) == 0.0
    with pytest.raises(ValueError):
        oracle.exact_sum([1.0, np.inf])


def test_tri_normalize_follows_exact_sums_not_token_order():
    # The rows' sums depend on the order in which a sequence of binary64 adds
    # would take them; the exactly rounded sum does not.  ulp(2^60) is 256, so
    # in token order 2^60 + 1 rounds back to 2^60:
    #   A = [2^60, 1 (x255), -2^60]: a left-to-right sum gives 0;
    #   B = [1 (x255), 2^60, -2^60]: a left-to-right sum gives 256;
    # the exact sum is 255 for both, so mu = RN(255 / 257) in both rows.  The
    # squared deviations sum to 2^121 exactly rounded (the terms near 1 are far
    # below ulp(2^121)), so sigma = sqrt(2^121 / 257).  Each z is compared
    # with Python's binary64 arithmetic, rounded to binary32.
    import math
    big = F32(2.0 ** 60)
    a = np.concatenate([[big], np.ones(255, F32), [-big]]).astype(F32)
    b = np.concatenate([np.ones(255, F32), [big], [-big]]).astype(F32)
    s = np.stack([a, b]).reshape(1, 1, 2, 257)
    z = oracle.tri_select(s, np.array([257], np.int32), "per_layer_perhead", 4)["z"][0, 0]
    mu = 255.0 / 257.0
    sigma = math.sqrt(2.0 ** 121 / 257)
    for g in (0, 1):
        row = s[0, 0, g].astype(np.float64)
        want = np.array([(x - mu) / sigma for x in row]).astype(F32)
        assert np.array_equal(z[g].view(np.uint32), want.view(np.uint32)), f"row {g}"
    # a token-order mean (0 for row A, 256/257 for row B) moves the z of a one
    for seq_mu in (0.0, 256.0 / 257.0):
        assert F32((1.0 - seq_mu) / sigma) != z[0, 1]


def test_tri_normalize_bitwise_against_rational_statistics():
    # Random rows over a wide dynamic range, every step written out in
    # Python's binary64 arithmetic with Fraction for the exact sums: the
    # oracle's z must agree bit for bit.
    from fractions import Fraction
    import math
    rs = np.random.default_rng(35)
    L = 700
    x = (rs.standard_normal((1, 1, 3, L)) * np.exp2(rs.integers(-20, 21, size=(1, 1, 3, L)))).astype(F32)
    x[0, 0, 1, ::7] = -np.inf
    kv = np.array([L - 33], np.int32)
    z = oracle.tri_select(x, kv, "per_layer_perhead", 8)["z"][0, 0]
    Lr = int(kv[0])
    for g in range(3):
        row = [float(v) for v in x[0, 0, g, :Lr]]
        fin = [v for v in row if math.isfinite(v)]
        n = len(fin)
        mu = float(sum(map(Fraction, fin), Fraction(0))) / n
        sq = [(v - mu) * (v - mu) for v in fin]
        sigma = math.sqrt(float(sum(map(Fraction, sq), Fraction(0))) / n)
        want = np.array([(v - mu) / sigma if math.isfinite(v) else -np.inf for v in row]).astype(F32)
        assert np.array_equal(z[g, :Lr].view(np.uint32), want.view(np.uint32)), g
        assert np.all(z[g, Lr:] == -np.inf)


def test_tri_constant_row_and_empty_row():
    s = np.full((1, 2, 1, 300), 3.25, F32)
    kv = np.array([300, 0], np.int32)
    r = oracle.tri_select(s, kv, "union", 10)
    assert np.all(r["z"][0, 0, 0] == 0.0)
    assert list(r["indices"][0]) == list(range(10))        # all tie: lowest positions
    assert np.all(r["indices"][1] == -1) and r["counts"][1] == 0


def test_tri_per_layer_perhead_matches_raw_topk_on_separated_scores():
    # z is increasing in s, so with well-separated distinct scores the
    # selection on z is the selection on the raw scores
    rs = np.random.default_rng(33)
    L = 4000
    s = np.stack([rs.permutation(L).astype(F32) * F32(0.5) for _ in range(2 * 3 * 2)]).reshape(2, 3, 2, L)
    kv = np.array([4000, 2500, 999], np.int32)
    r = oracle.tri_select(s, kv, "per_layer_perhead", 300)
    raw_i, raw_c = oracle.topk(s.reshape(6, 2, L), np.tile(kv, 2), 300)
    assert np.array_equal(r["indices"], raw_i.reshape(-1, 300))
    assert np.array_equal(r["counts"], raw_c.reshape(-1))


def test_tri_modes_reduce_over_the_right_members():
    rs = np.random.default_rng(34)
    one = rs.standard_normal((1, 2, 1, 3000)).astype(F32)
    kv = np.array([3000, 2000], np.int32)
    base = oracle.tri_select(one, kv, "per_layer_perhead", 128)
    # identical layers and groups reduce to the single row
    same = np.broadcast_to(one, (3, 2, 4, 3000)).copy()
    for mode, rows in (("per_head", 8), ("union", 2)):
        r = oracle.tri_select(same, kv, mode, 128)
        assert r["indices"].shape[0] == rows
        want = base["indices"] if mode == "union" else np.repeat(base["indices"], 4, axis=0)
        assert np.array_equal(r["indices"], want)
    # union's reduced row is the max of per_head's reduced rows over groups,
    # per_head's the max over layers of the per-layer z
    s = rs.standard_normal((3, 2, 4, 3000)).astype(F32)
    ph = oracle.tri_select(s, kv, "per_head", 64)
    un = oracle.tri_select(s, kv, "union", 64)
    assert np.array_equal(un["reduced"], ph["reduced"].reshape(2, 4, 3000).max(axis=1))
    assert np.array_equal(ph["reduced"], ph["z"].max(axis=0).reshape(8, 3000))


def test_tri_union_keeps_a_token_one_head_alone_wants():
    # the reduction is a max: a spike in one head survives the union even when
    # every other head scores the token at the bottom (a mean would drop it)
    rs = np.random.default_rng(35)
    s = rs.standard_normal((1, 1, 8, 2000)).astype(F32)
    s[0, 0, 1:, 777] = -5.0
    s[0, 0, 0, 777] = 40.0
    r = oracle.tri_select(s, np.array([2000], np.int32), "union", 16)
    assert 777 in r["indices"][0]


# ---------------------------------------------------------------- multi-query decode

def test_multi_query_last_row_is_single_query_decode_and_rows_are_causal():
    import dataclasses
    n = 3
    w = synth.make_workload(4, batch=2, kv_len=[300, 130], topk=64, idx_heads=8, heads=4, next_n=n)
    assert w.score_q.shape[0] == 2 * n and w.q.shape[0] == 2 * n
    ref = oracle.sparse_decode(w)
    # the last query token of each request sees the whole cache: it is the
    # single-query decode of that request with its own query
    last = [b * n + n - 1 for b in range(2)]
    w1 = dataclasses.replace(w, score_q=w.score_q[last], head_weights=w.head_weights[last], q=w.q[last],
                             next_n=1)
    one = oracle.sparse_decode(w1)
    assert np.array_equal(ref["indices"][last], one["indices"])
    assert np.array_equal(ref["out"][last], one["out"])
    # query j never selects a token at or past kv_len - (n - 1 - j) (its own
    # later draft positions), and selects every token when that length <= k
    for b, L in enumerate(w.kv_lens):
        for j in range(n):
            lim = int(L) - (n - 1 - j)
            idx = ref["indices"][b * n + j, 0]
            kept = idx[idx >= 0]
            assert kept.max() < lim
            assert ref["counts"][b * n + j, 0] == min(lim, 64)
            if lim <= 64:
                assert list(kept) == list(range(lim))


def test_multi_query_rows_past_the_cache_are_empty():
    n = 4
    w = synth.make_workload(4, batch=2, kv_len=[2, 50], topk=16, idx_heads=8, heads=4, next_n=n)
    ref = oracle.sparse_decode(w)
    # request 0 has 2 tokens: its queries 0 and 1 see -1 and 0 tokens
    for j, lim in enumerate([0, 0, 1, 2]):
        assert ref["counts"][j, 0] == lim
        if lim == 0:
            assert np.all(ref["indices"][j] == -1)
            assert np.all(ref["out"][j] == 0.0)


# ---------------------------------------------------------------- block-granular indices

def test_block_expansion_by_hand():
    # block size 4, kv_len 10: entry 2 -> tokens 8, 9 (10, 11 lie past the
    # cache), -1 -> nothing, entry 0 -> 0..3, entry 3 -> nothing (12..15)
    tok = oracle.expand_blocks(np.array([[[2, -1, 0, 3]]]), np.array([10]), 4)
    assert tok.tolist() == [[[8, 9, -1, -1, -1, -1, -1, -1, 0, 1, 2, 3, -1, -1, -1, -1]]]
    # block size 1 is the token list itself, with the past-L entries dropped
    one = oracle.expand_blocks(np.array([[[5, 0, 12, -3]]]), np.array([10]), 1)
    assert one.tolist() == [[[5, 0, -1, -1]]]


def test_block_attention_of_one_covering_block_is_dense_attention():
    w = synth.make_workload(3, batch=2, kv_len=[70, 33], topk=16)
    G = w.k.shape[1]
    full = np.tile(np.arange(70, dtype=np.int32), (2, G, 1))
    full[1, :, 33:] = -1
    dense = oracle.attention(w.block_table, w.kv_lens, w.q, w.k, w.v, w.v_dim, full, w.softmax_scale)
    blk = oracle.expand_blocks(np.zeros((2, G, 1), np.int32), w.kv_lens, 128)   # one block of 128
    got = oracle.attention(w.block_table, w.kv_lens, w.q, w.k, w.v, w.v_dim, blk, w.softmax_scale)
    assert np.array_equal(got, dense)


# ---------------------------------------------------------------- threads

def test_oracle_results_do_not_depend_on_thread_count():
    # the row loops run on several threads; each row's arithmetic is the
    # same, so every output is bit-identical to the one-thread run
    w = synth.make_workload(5, batch=6, min_len=300, max_len=5000, topk=256, idx_heads=16, heads=32)
    s = np.random.default_rng(36).standard_normal((2, 3, 2, 3000)).astype(F32)
    kv = np.array([3000, 1700, 5], np.int32)
    runs = []
    for n in (1, 4):
        oracle.set_threads(n)
        runs.append((oracle.sparse_decode(w), oracle.tri_select(s, kv, "union", 64)))
    oracle.set_threads(os.cpu_count() or 1)
    (a, ta), (b, tb) = runs
    for key in ("scores", "indices", "counts"):
        assert np.array_equal(np.asarray(a[key]).view(np.uint8), np.asarray(b[key]).view(np.uint8)), key
    assert np.array_equal(a["out"].view(np.uint64), b["out"].view(np.uint64))
    for key in ("z", "reduced", "indices", "counts"):
        assert np.array_equal(np.asarray(ta[key]).view(np.uint8), np.asarray(tb[key]).view(np.uint8)), key
