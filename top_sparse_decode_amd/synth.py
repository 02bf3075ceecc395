"""Seeded synthetic inputs for top-k sparse decode attention.

This module only draws random tensors and lays them out in paged pools; it
holds none of the method's arithmetic (no scoring, selection or softmax), so
both the HIP path and the CPU oracle can be fed from it.

Random numbers come from NumPy's Philox4x32 counter-based generator (Salmon et
al., "Parallel random numbers: as easy as 1, 2, 3", SC'11), keyed by
(seed, tensor id), so every tensor is reproducible on its own.  Float tensors
are drawn in float32 and, for bfloat16 workloads, rounded once to bfloat16
(round to nearest even) here on the host; both sides then read identical bits.
bfloat16 tensors are carried as uint16 arrays of the raw bits.

Pool layout is HND: [num_pages, num_kv_heads, page_size, head_dim], so one
(page, KV head) is one contiguous run.  Unassigned pages and the slots past a
request's last token are filled with NaN canaries.

The five workload families (sizes are the defaults; every size can be
overridden to make a smaller case with the same structure):

1. ``tiny_f32``      fp32, B1, 4 query heads on 1 KV head, D64, L1024, page 16,
                     top-k 128, 8 heavy tokens with K shifted by 3*qbar/|qbar|.
2. ``mha_bf16``      bf16 distilgpt2-shaped MHA: B6, 12 heads, D64, L1024,
                     page 32, per-head top-k 408, rank-8 low-rank K/Q mixture.
3. ``gqa_bf16``      bf16 Qwen3-8B-shaped GQA: B32, 32 q / 8 KV heads, D128,
                     L8192, page 64, top-k 2048 per KV head, mean over the 4
                     heads; K/V channels scaled by exp(U(ln .5, ln 4)).
4. ``dsa_mla``       DSA sparse MLA: B16, 64x128 bf16 indexer, w ~ U(0,1),
                     L65536, page 64, top-k 2048; 128 heads over a 576-wide
                     latent row (V = first 512), scale 1/sqrt(192).
5. ``dsa_mla_mixed`` as 4 with B64, L ~ U{4096..131072}, one shared pool with
                     fragmented random page assignment, 1% of tokens with
                     k_I += 4.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

BF16_NAN = np.uint16(0x7FC0)

# tensor ids (part of the Philox key)
_T_PERM, _T_Q, _T_K, _T_V, _T_W, _T_QI, _T_KI, _T_LAT, _T_HEAVY, _T_BASIS, _T_MIX, _T_SCALE, \
    _T_LEN, _T_BIAS = range(1, 15)


def rng(seed: int, tensor: int, sub: int = 0) -> np.random.Generator:
    """Philox generator for (seed, tensor id, sub-stream)."""
    key = (int(seed) & 0xFFFFFFFF) << 64 | (int(tensor) & 0xFFFFFFFF) << 32 | (int(sub) & 0xFFFFFFFF)
    return np.random.Generator(np.random.Philox(key=key))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bits, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


FP8_NAN = np.uint8(0x7F)
FP8_MAX = 448.0


def to_fp8_e4m3(x: np.ndarray) -> np.ndarray:
    """float32 -> OCP FP8 E4M3 codes (sign, 4 exponent bits with bias 7, 3
    mantissa bits; subnormals m * 2^-9), round to nearest even, magnitudes
    above 448 saturated to 448.  Finite inputs.  Normals round the binary32
    mantissa to 3 bits on the bit pattern (a carry moves into the exponent);
    below 2^-6 the code is rne(|x| * 2^9) itself (8 is the smallest normal)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint8)
    xf, of = x.reshape(-1), out.reshape(-1)
    step = 1 << 22
    for s in range(0, xf.size, step):
        u = xf[s:s + step].view(np.uint32)
        a = u & np.uint32(0x7FFFFFFF)
        r = (a + np.uint32(0x7FFFF) + ((a >> np.uint32(20)) & np.uint32(1))) >> np.uint32(20)
        code_n = r.astype(np.int32) - (120 << 3)          # binary32 bias 127 -> E4M3 bias 7
        code_s = np.rint(a.view(np.float32) * np.float32(512.0)).astype(np.int32)
        code = np.minimum(np.where(a >= np.uint32(0x3C800000), code_n, code_s), 0x7E)  # 2^-6
        of[s:s + step] = ((u >> np.uint32(24)) & np.uint32(0x80)).astype(np.uint8) | code.astype(np.uint8)
    return out


def quantize_rows_fp8(rows_f32: np.ndarray):
    """Per-row block scaling: scale = max|row| / 448 (1 for an all-zero row),
    codes = E4M3(row / scale).  rows [..., D] -> (codes uint8 [..., D],
    scales float32 [...]).  Rows holding a NaN get code 0x7F and scale NaN."""
    rows = np.asarray(rows_f32, dtype=np.float32)
    D = rows.shape[-1]
    flat = rows.reshape(-1, D)
    codes = np.empty(flat.shape, np.uint8)
    scale = np.empty(flat.shape[0], np.float32)
    step = max(1, (1 << 22) // D)
    for s in range(0, flat.shape[0], step):
        r = flat[s:s + step]
        nan = np.isnan(r).any(axis=-1)
        r = np.where(nan[:, None], np.float32(0.0), r)
        amax = np.max(np.abs(r), axis=-1)
        sc = np.where(amax > 0, amax / np.float32(FP8_MAX), np.float32(1.0)).astype(np.float32)
        c = to_fp8_e4m3(r / sc[:, None])
        c[nan] = FP8_NAN
        sc[nan] = np.float32(np.nan)
        codes[s:s + step] = c
        scale[s:s + step] = sc
    return codes.reshape(rows.shape), scale.reshape(rows.shape[:-1])


@dataclass
class Workload:
    """One decode step's inputs.  Arrays are host numpy; bfloat16 as uint16 bits."""

    name: str
    seed: int
    page_size: int
    block_table: np.ndarray          # int32 [B, max_pages]; -1 past the last page
    kv_lens: np.ndarray              # int32 [B]
    max_kv_len: int                  # row length of score buffers
    # scoring side
    score_k: np.ndarray              # pool [pages, Hs_kv, P, Ds]
    score_q: np.ndarray              # [B, Hs, Ds]
    head_weights: Optional[np.ndarray]  # float32 [B, Hs] or None
    mode: str                        # "group_sum" | "group_mean" | "relu_weighted"
    head_scale: float
    topk: int
    # attention side
    q: np.ndarray                    # [B, Hq, Dqk]
    k: np.ndarray                    # pool [pages, Hkv, P, Dqk]
    v: np.ndarray                    # pool [pages, Hkv, P, Drow] (may be k itself)
    v_dim: int
    softmax_scale: float
    out_dtype: str                   # "f32" | "bf16"
    meta: dict = field(default_factory=dict)
    # FP8 indexer pools: score_k holds E4M3 codes (uint8) and this the row
    # scales [pages, Hs_kv, P] float32
    score_k_scale: Optional[np.ndarray] = None
    # multi-query decode: next_n query tokens per request; score_q,
    # head_weights and q then hold batch * next_n rows (request-major)
    next_n: int = 1

    @property
    def batch(self) -> int:
        return int(self.kv_lens.shape[0])

    @property
    def num_pages(self) -> int:
        return int(self.k.shape[0])

    @property
    def groups(self) -> int:
        return int(self.score_k.shape[1])

    @property
    def v_aliases_k(self) -> bool:
        return self.v is self.k


# ----------------------------------------------------------------- page tables

def _assign_pages(seed: int, kv_lens: np.ndarray, page_size: int, num_pages: int,
                  max_pages: int) -> np.ndarray:
    """Disjoint random page sets: a random permutation of the pool handed out
    request by request, so each request's pages are scattered over the pool."""
    need = [(int(L) + page_size - 1) // page_size for L in kv_lens]
    if sum(need) > num_pages:
        raise ValueError("pool too small for the requested lengths")
    perm = rng(seed, _T_PERM).permutation(num_pages).astype(np.int32)
    bt = np.full((len(kv_lens), max_pages), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(need):
        bt[b, :n] = perm[pos:pos + n]
        pos += n
    return bt


def _canary_mask(block_table: np.ndarray, kv_lens: np.ndarray, page_size: int, num_pages: int):
    """(assigned page flags [pages], list of (page, first dead slot) tail pages)."""
    used = np.zeros(num_pages, dtype=bool)
    tails = []
    for b in range(block_table.shape[0]):
        L = int(kv_lens[b])
        n = (L + page_size - 1) // page_size
        pages = block_table[b, :n]
        used[pages] = True
        if n and L % page_size:
            tails.append((int(pages[n - 1]), L % page_size))
    return used, tails


def _apply_canaries(pool: np.ndarray, used: np.ndarray, tails) -> None:
    nan = BF16_NAN if pool.dtype == np.uint16 else np.float32(np.nan)
    pool[~used] = nan
    for page, slot in tails:
        pool[page, :, slot:, :] = nan


# ----------------------------------------------------------------- pool fill

def _torch_gen(seed: int, tensor: int, sub: int):
    import torch

    key = ((int(seed) & 0xFFFF) << 40) | ((int(tensor) & 0xFF) << 32) | (int(sub) & 0xFFFFFFFF)
    return torch.Generator(device="cpu").manual_seed(key)


def _normal_pool(seed: int, tensor: int, shape, bf16: bool, used: np.ndarray,
                 chunk_pages: int = 256, channel_scale: Optional[np.ndarray] = None) -> np.ndarray:
    """N(0,1) pool (optionally times a per-(KV head, channel) scale), drawn
    page-chunk by page-chunk, each chunk from its own seeded generator
    (PyTorch's CPU generator, seeded from (seed, tensor id, chunk)), into
    preallocated buffers.  bfloat16 rounding is round to nearest even.
    Unassigned pages are left for the caller to fill with canaries."""
    import torch

    pages = int(shape[0])
    inner = tuple(int(s) for s in shape[1:])
    out = torch.empty((pages,) + inner, dtype=torch.bfloat16 if bf16 else torch.float32)
    buf = torch.empty((min(chunk_pages, max(pages, 1)),) + inner, dtype=torch.float32)
    cs = None if channel_scale is None else torch.from_numpy(
        np.ascontiguousarray(channel_scale, dtype=np.float32))[None, :, None, :]
    for c0 in range(0, pages, chunk_pages):
        c1 = min(pages, c0 + chunk_pages)
        if not used[c0:c1].any():
            continue
        b = buf[: c1 - c0]
        torch.randn(b.shape, generator=_torch_gen(seed, tensor, c0 // chunk_pages), out=b)
        if cs is not None:
            b.mul_(cs)
        out[c0:c1].copy_(b)
    if bf16:
        return out.view(torch.int16).numpy().view(np.uint16)
    return out.numpy()


# ----------------------------------------------------------------- configs

DEFAULTS = {
    1: dict(batch=1, q_heads=4, kv_heads=1, head_dim=64, kv_len=1024, page_size=16, topk=128,
            heavy=8, num_pages=None),
    2: dict(batch=6, q_heads=12, kv_heads=12, head_dim=64, kv_len=1024, page_size=32, topk=408,
            rank=8, num_pages=None),
    3: dict(batch=32, q_heads=32, kv_heads=8, head_dim=128, kv_len=8192, page_size=64, topk=2048,
            num_pages=None),
    4: dict(batch=16, idx_heads=64, idx_dim=128, kv_len=65536, page_size=64, topk=2048,
            heads=128, latent=576, v_dim=512, num_pages=None, index_dtype="bf16", next_n=1),
    5: dict(batch=64, idx_heads=64, idx_dim=128, min_len=4096, max_len=131072, page_size=64,
            topk=2048, heads=128, latent=576, v_dim=512, bias_frac=0.01, bias=4.0,
            slack=1.25, kv_lens=None, index_dtype="bf16", next_n=1),
}

NAMES = {1: "tiny_f32", 2: "mha_bf16", 3: "gqa_bf16", 4: "dsa_mla", 5: "dsa_mla_mixed"}


def _lens_arg(kv_len, batch):
    if np.ndim(kv_len) == 0:
        return np.full(batch, int(kv_len), dtype=np.int32)
    a = np.asarray(kv_len, dtype=np.int32)
    assert a.shape == (batch,)
    return a


def make_workload(config: int, seed: Optional[int] = None, **kw) -> Workload:
    """Build workload ``config`` (1..5).  Seed defaults to the config number.
    Keyword overrides replace the defaults above; ``kv_len`` may be an int or
    a per-request list."""
    if config not in DEFAULTS:
        raise ValueError(f"unknown config {config}")
    p = dict(DEFAULTS[config])
    unknown = set(kw) - set(p)
    if unknown:
        raise TypeError(f"unknown overrides {sorted(unknown)} for config {config}")
    p.update(kw)
    seed = config if seed is None else int(seed)
    return _BUILDERS[config](seed, p)


def _paged_common(seed, p, kv_lens, max_len=None):
    P = p["page_size"]
    B = len(kv_lens)
    max_len = int(max(kv_lens.max(initial=0), 1)) if max_len is None else int(max_len)
    max_pages = max(1, (max_len + P - 1) // P)
    need = int(sum((int(L) + P - 1) // P for L in kv_lens))
    num_pages = p.get("num_pages") or max(need, 1)
    bt = _assign_pages(seed, kv_lens, P, num_pages, max_pages)
    used, tails = _canary_mask(bt, kv_lens, P, num_pages)
    return P, B, max_len, max_pages, num_pages, bt, used, tails


def _build_tiny(seed, p):
    B, Hq, Hkv, D = p["batch"], p["q_heads"], p["kv_heads"], p["head_dim"]
    kv_lens = _lens_arg(p["kv_len"], B)
    P, B, max_len, max_pages, num_pages, bt, used, tails = _paged_common(seed, p, kv_lens)
    q = rng(seed, _T_Q).standard_normal((B, Hq, D), dtype=np.float32)
    k = rng(seed, _T_K).standard_normal((num_pages, Hkv, P, D), dtype=np.float32)
    v = rng(seed, _T_V).standard_normal((num_pages, Hkv, P, D), dtype=np.float32)
    # heavy tokens: K shifted by 3 * qbar / |qbar|, qbar the sum of the group's query heads
    G = Hq // Hkv
    hr = rng(seed, _T_HEAVY)
    for b in range(B):
        L = int(kv_lens[b])
        n = min(p["heavy"], L)
        pos = hr.choice(L, size=n, replace=False) if n else []
        for g in range(Hkv):
            qbar = q[b, g * G:(g + 1) * G].astype(np.float64).sum(axis=0)
            shift = (3.0 * qbar / np.linalg.norm(qbar)).astype(np.float32)
            for t in pos:
                k[bt[b, t // P], g, t % P] += shift
    _apply_canaries(k, used, tails)
    _apply_canaries(v, used, tails)
    return Workload(NAMES[1], seed, P, bt, kv_lens, max_len, k, q, None, "group_sum",
                    1.0 / math.sqrt(D), p["topk"], q, k, v, D, 1.0 / math.sqrt(D), "f32",
                    meta=dict(p))


def _build_mha(seed, p):
    B, H, D, r = p["batch"], p["q_heads"], p["head_dim"], p["rank"]
    assert p["kv_heads"] == H
    kv_lens = _lens_arg(p["kv_len"], B)
    P, B, max_len, max_pages, num_pages, bt, used, tails = _paged_common(seed, p, kv_lens)
    basis = rng(seed, _T_BASIS).standard_normal((B, H, r, D), dtype=np.float32) / np.float32(
        math.sqrt(r))
    # Q = z_q + a_q U
    zq = rng(seed, _T_Q).standard_normal((B, H, D), dtype=np.float32)
    aq = rng(seed, _T_MIX, 0).standard_normal((B, H, r), dtype=np.float32)
    q = zq + np.einsum("bhr,bhrd->bhd", aq, basis)
    # K_t = z_t + a_t U, per request through its own pages
    kf = rng(seed, _T_K).standard_normal((num_pages, H, P, D), dtype=np.float32)
    ak = rng(seed, _T_MIX, 1).standard_normal((num_pages, H, P, r), dtype=np.float32)
    owner = np.full(num_pages, -1, dtype=np.int64)
    for b in range(B):
        n = (int(kv_lens[b]) + P - 1) // P
        owner[bt[b, :n]] = b
    for pg in np.nonzero(owner >= 0)[0]:
        kf[pg] += np.einsum("hpr,hrd->hpd", ak[pg], basis[owner[pg]])
    v = rng(seed, _T_V).standard_normal((num_pages, H, P, D), dtype=np.float32)
    qb, kb, vb = to_bf16_bits(q), to_bf16_bits(kf), to_bf16_bits(v)
    _apply_canaries(kb, used, tails)
    _apply_canaries(vb, used, tails)
    return Workload(NAMES[2], seed, P, bt, kv_lens, max_len, kb, qb, None, "group_sum", 1.0,
                    p["topk"], qb, kb, vb, D, 1.0 / math.sqrt(D), "bf16", meta=dict(p))


def _build_gqa(seed, p):
    B, Hq, Hkv, D = p["batch"], p["q_heads"], p["kv_heads"], p["head_dim"]
    kv_lens = _lens_arg(p["kv_len"], B)
    P, B, max_len, max_pages, num_pages, bt, used, tails = _paged_common(seed, p, kv_lens)
    lo, hi = math.log(0.5), math.log(4.0)
    sr = rng(seed, _T_SCALE)
    ck = np.exp(sr.uniform(lo, hi, size=(Hkv, D))).astype(np.float32)
    cv = np.exp(sr.uniform(lo, hi, size=(Hkv, D))).astype(np.float32)
    q = to_bf16_bits(rng(seed, _T_Q).standard_normal((B, Hq, D), dtype=np.float32))
    kb = _normal_pool(seed, _T_K, (num_pages, Hkv, P, D), True, used, channel_scale=ck)
    vb = _normal_pool(seed, _T_V, (num_pages, Hkv, P, D), True, used, channel_scale=cv)
    _apply_canaries(kb, used, tails)
    _apply_canaries(vb, used, tails)
    return Workload(NAMES[3], seed, P, bt, kv_lens, max_len, kb, q, None, "group_mean", 1.0,
                    p["topk"], q, kb, vb, D, 1.0 / math.sqrt(D), "bf16", meta=dict(p))


def _build_dsa(seed, p, kv_lens, name, max_len=None, num_pages=None):
    Hi, Di, H, Dl = p["idx_heads"], p["idx_dim"], p["heads"], p["latent"]
    p = dict(p)
    if num_pages is not None:
        p["num_pages"] = num_pages
    P, B, max_len, max_pages, num_pages, bt, used, tails = _paged_common(seed, p, kv_lens, max_len)
    n = int(p.get("next_n", 1))
    qi = to_bf16_bits(rng(seed, _T_QI).standard_normal((B * n, Hi, Di), dtype=np.float32))
    w = rng(seed, _T_W).random((B * n, Hi), dtype=np.float32)
    ki = _normal_pool(seed, _T_KI, (num_pages, 1, P, Di), True, used)
    if p.get("bias_frac"):
        # +bias on every indexer-key channel for a Bernoulli(bias_frac) subset of tokens
        br = rng(seed, _T_BIAS)
        for b in range(B):
            L = int(kv_lens[b])
            hit = np.nonzero(br.random(L) < p["bias_frac"])[0]
            if hit.size == 0:
                continue
            pg, sl = bt[b, hit // P], hit % P
            rows = bf16_bits_to_f32(ki[pg, 0, sl, :]) + np.float32(p["bias"])
            ki[pg, 0, sl, :] = to_bf16_bits(rows)
    q = to_bf16_bits(rng(seed, _T_Q).standard_normal((B * n, H, Dl), dtype=np.float32))
    lat = _normal_pool(seed, _T_LAT, (num_pages, 1, P, Dl), True, used)
    _apply_canaries(ki, used, tails)
    _apply_canaries(lat, used, tails)
    ki_scale = None
    if p.get("index_dtype", "bf16") == "fp8":
        # the same keys, block-scaled to FP8 E4M3 with one scale per token row
        # (canary rows stay NaN: code 0x7F, scale NaN)
        ki, ki_scale = quantize_rows_fp8(bf16_bits_to_f32(ki))
    elif p.get("index_dtype", "bf16") != "bf16":
        raise ValueError(f"index_dtype must be bf16 or fp8, got {p['index_dtype']}")
    return Workload(name, seed, P, bt, kv_lens, max_len, ki, qi, w, "relu_weighted", 1.0,
                    p["topk"], q, lat, lat, p["v_dim"], 1.0 / math.sqrt(192.0), "bf16",
                    meta=dict(p), score_k_scale=ki_scale, next_n=n)


def _build_dsa4(seed, p):
    kv_lens = _lens_arg(p["kv_len"], p["batch"])
    return _build_dsa(seed, p, kv_lens, NAMES[4])


def _build_dsa5(seed, p):
    B, P = p["batch"], p["page_size"]
    if p.get("kv_lens") is not None:
        kv_lens = _lens_arg(p["kv_lens"], B)
    else:
        kv_lens = rng(seed, _T_LEN).integers(p["min_len"], p["max_len"], size=B,
                                               endpoint=True).astype(np.int32)
    need = int(sum((int(L) + P - 1) // P for L in kv_lens))
    num_pages = int(math.ceil(p["slack"] * need))
    max_len = int(max(p["max_len"], kv_lens.max(initial=1)))
    q = dict(p)
    q.pop("kv_lens", None)
    return _build_dsa(seed, q, kv_lens, NAMES[5], max_len=max_len, num_pages=num_pages)


_BUILDERS = {1: _build_tiny, 2: _build_mha, 3: _build_gqa, 4: _build_dsa4, 5: _build_dsa5}
