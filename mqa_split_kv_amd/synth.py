"""Seeded synthetic inputs for paged decode attention.

This module draws random numbers, rounds them to the stored formats and packs
pages.  It holds none of the attention arithmetic: both the HIP path and the CPU
oracle consume what it produces, and nothing here imports either of them.

Recipe (numpy PCG64; one generator per case, seeded by the caller):
  1. seq_lens (ragged case only): L = clip(rint(exp(U(ln lo, ln hi))), lo, hi)
  2. page permutation of the pool; request b takes the next ceil(L_b / P) pages
     of the permutation, in order; unused block-table entries are 0
  3. q ~ N(0, 1) rounded to bf16 (round to nearest even), shape [B, Hq, D]
  4. K pool, then V pool ~ N(0, 1) (every slot, also padding slots and unused
     pages), drawn in chunks of consecutive pages; chunk c of pool w (0 = K or the
     MLA pool, 1 = V) has its own PCG64 stream seeded with SeedSequence((seed, w, c)),
     so that chunks are drawn in parallel and the values do not depend on the thread
     count
  5. bf16 pools: rounded to bf16.
     fp8 page-head pools: per (page, KV head) scale = max|x| / 448 over the page's
     P*D values (1 if the max is 0), code = e4m3(RNE(x / scale)) saturated to +-448;
     K and V get separate scales.
     MLA 656-byte pool: per token, the 576-dim latent ~ N(0, 1); dims 0..511 are
     quantized in 4 tiles of 128 with scale = max|x| / 448 each; dims 512..575 are
     kept as bf16.  Bytes: [512 e4m3][4 fp32 scales][64 bf16].  V aliases K.
"""
from __future__ import annotations

import math
import os
from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

KV_BF16, KV_FP8_PAGE_HEAD, KV_MLA656 = 0, 1, 2
E4M3_MAX = 448.0
MLA_TOKEN_BYTES = 656


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + r) >> 16).astype(np.uint16)


def f32_to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    """Round float32 to OCP e4m3 (nearest even, saturating at +-448); uint8 codes."""
    import torch

    y = np.clip(np.asarray(x, dtype=np.float32), -E4M3_MAX, E4M3_MAX)
    t = torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


@dataclass
class CaseSpec:
    """Shape and format of one decode-attention instance."""

    B: int
    Hq: int
    Hkv: int
    D: int
    Dv: int
    page_size: int
    seq_lens: Sequence[int] = ()
    kv_format: int = KV_BF16
    pool_pages: Optional[int] = None     # None: exactly the pages used
    layout: str = "HND"                  # HND [page][head][tok][D] or NHD [page][tok][head][D]
    loguniform: Optional[tuple] = None   # (lo, hi): draw seq_lens log-uniformly
    num_splits: int = 0
    name: str = ""
    q_len: int = 1                       # query tokens per request (draft length)
    extra: dict = field(default_factory=dict)


# The five workloads of the decode-attention scope table, by index.
WORKLOADS = {
    0: CaseSpec(B=2, Hq=8, Hkv=1, D=64, Dv=64, page_size=16, seq_lens=(100, 257),
                pool_pages=40, num_splits=1, name="tiny GQA paged decode"),
    1: CaseSpec(B=32, Hq=64, Hkv=8, D=128, Dv=128, page_size=64, seq_lens=(4096,) * 32,
                pool_pages=2048, num_splits=0, name="GQA decode, Llama-70B-like"),
    2: CaseSpec(B=8, Hq=32, Hkv=4, D=64, Dv=64, page_size=256, seq_lens=(1536,) * 8,
                num_splits=8, name="HD64 GQA decode"),
    3: CaseSpec(B=64, Hq=32, Hkv=8, D=128, Dv=128, page_size=16, loguniform=(256, 131072),
                kv_format=KV_FP8_PAGE_HEAD, num_splits=0, name="ragged long-context FP8 KV"),
    4: CaseSpec(B=64, Hq=128, Hkv=1, D=576, Dv=512, page_size=64, seq_lens=(8192,) * 64,
                kv_format=KV_MLA656, pool_pages=8192, num_splits=0, name="MLA-style MQA decode"),
}
SEED_BASE = 1000


def draw_loguniform_lens(rng: np.random.Generator, B: int, lo: int, hi: int) -> np.ndarray:
    u = rng.uniform(math.log(lo), math.log(hi), size=B)
    return np.clip(np.rint(np.exp(u)), lo, hi).astype(np.int32)


def _normal_f32(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


# values per pool chunk (one independent stream each)
CHUNK_VALUES = 1 << 24


def _chunk_rng(seed: int, which: int, chunk: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence((seed, which, chunk))))


def _fill_chunks(num_pages: int, values_per_page: int, seed: int, which: int, fill) -> None:
    """Call fill(rng, p0, p1) for every chunk [p0, p1) of pages, in parallel."""
    from concurrent.futures import ThreadPoolExecutor

    per = max(1, CHUNK_VALUES // values_per_page)
    chunks = [(c, p0, min(num_pages, p0 + per)) for c, p0 in enumerate(range(0, num_pages, per))]
    workers = max(1, min(len(chunks), 16, os.cpu_count() or 1))
    if workers == 1:
        for c, p0, p1 in chunks:
            fill(_chunk_rng(seed, which, c), p0, p1)
        return
    with ThreadPoolExecutor(max_workers=workers) as ex:
        for f in [ex.submit(fill, _chunk_rng(seed, which, c), p0, p1) for c, p0, p1 in chunks]:
            f.result()


def make_case(spec: CaseSpec, seed: int, scale: Optional[float] = None) -> dict:
    """Draw one instance.  Returns a dict of numpy arrays plus shape fields.

    Keys: B, Hkv, G, D, Dv, page_size, num_pages, max_pages, s_page, s_head, s_tok
    (pool strides in storage units: bf16 elements, or bytes for fp8 / MLA),
    kv_format, layout, q [B,Hq,D] uint16 (bf16 bits; [B,q_len,Hq,D] when q_len > 1),
    q_len, k_pool, v_pool (None for MLA),
    k_scale, v_scale ([num_pages, Hkv] float32 or None), block_table [B, max_pages]
    int32, seq_lens [B] int32, scale (float), num_splits.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    B, Hq, Hkv, D, Dv, P = spec.B, spec.Hq, spec.Hkv, spec.D, spec.Dv, spec.page_size
    assert Hq % Hkv == 0
    G = Hq // Hkv
    if spec.loguniform is not None:
        seq_lens = draw_loguniform_lens(rng, B, *spec.loguniform)
    else:
        seq_lens = np.asarray(spec.seq_lens, dtype=np.int32)
        assert seq_lens.shape == (B,)
    pages_needed = [-(-int(L) // P) for L in seq_lens]
    used = int(sum(pages_needed))
    num_pages = spec.pool_pages if spec.pool_pages is not None else max(used, 1)
    assert num_pages >= used
    max_pages = max(max(pages_needed) if pages_needed else 1, 1)
    perm = rng.permutation(num_pages).astype(np.int32)
    block_table = np.zeros((B, max_pages), np.int32)
    pos = 0
    for b in range(B):
        n = pages_needed[b]
        block_table[b, :n] = perm[pos:pos + n]
        pos += n

    nq = spec.q_len
    q = f32_to_bf16_bits(_normal_f32(rng, (B, Hq, D) if nq == 1 else (B, nq, Hq, D)))

    case = dict(B=B, Hkv=Hkv, G=G, D=D, Dv=Dv, page_size=P, num_pages=num_pages, q_len=nq,
                max_pages=max_pages, kv_format=spec.kv_format, layout=spec.layout,
                q=q, block_table=block_table, seq_lens=seq_lens.astype(np.int32),
                scale=float(scale if scale is not None else 1.0 / math.sqrt(D)),
                num_splits=spec.num_splits, name=spec.name, k_scale=None, v_scale=None)

    if spec.kv_format == KV_MLA656:
        assert Hkv == 1 and D == 576 and Dv == 512
        pool = np.empty((num_pages, P, MLA_TOKEN_BYTES), np.uint8)

        def fill_mla(crng, p0, p1):
            x = _normal_f32(crng, (p1 - p0, P, 576))
            nope = x[..., :512].reshape(p1 - p0, P, 4, 128)
            amax = np.abs(nope).max(axis=-1)
            sc = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
            codes = f32_to_e4m3_codes(nope / sc[..., None]).reshape(p1 - p0, P, 512)
            rope = f32_to_bf16_bits(x[..., 512:])
            pool[p0:p1, :, 0:512] = codes
            pool[p0:p1, :, 512:528] = sc.view(np.uint8).reshape(p1 - p0, P, 16)
            pool[p0:p1, :, 528:656] = rope.view(np.uint8).reshape(p1 - p0, P, 128)

        _fill_chunks(num_pages, P * 576, seed, 0, fill_mla)
        case.update(k_pool=pool, v_pool=None, s_page=P * MLA_TOKEN_BYTES, s_head=0,
                    s_tok=MLA_TOKEN_BYTES)
        return case

    assert D == Dv
    fp8 = spec.kv_format == KV_FP8_PAGE_HEAD
    pools, scales = [], []
    for which in (0, 1):
        pool = np.empty((num_pages, Hkv, P, D), np.uint8 if fp8 else np.uint16)
        sc_all = np.empty((num_pages, Hkv), np.float32) if fp8 else None

        def fill_kv(crng, p0, p1, pool=pool, sc_all=sc_all):
            x = _normal_f32(crng, (p1 - p0, Hkv, P, D))
            if fp8:
                amax = np.abs(x).max(axis=(2, 3))
                sc = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
                pool[p0:p1] = f32_to_e4m3_codes(x / sc[:, :, None, None])
                sc_all[p0:p1] = sc
            else:
                pool[p0:p1] = f32_to_bf16_bits(x)

        _fill_chunks(num_pages, Hkv * P * D, seed, which, fill_kv)
        pools.append(pool)
        scales.append(sc_all)
    case.update(k_pool=pools[0], v_pool=pools[1], k_scale=scales[0], v_scale=scales[1])
    set_layout(case, spec.layout)
    return case


def set_layout(case: dict, layout: str) -> dict:
    """Store the pools as HND [page][head][tok][D] or NHD [page][tok][head][D] and set
    the strides.  The values of every (page, head, token) stay the same."""
    cur = case.get("_stored", "HND")
    k, v = case["k_pool"], case["v_pool"]
    if cur != layout:
        k = np.ascontiguousarray(k.transpose(0, 2, 1, 3))
        v = np.ascontiguousarray(v.transpose(0, 2, 1, 3))
    Hkv, P, D = case["Hkv"], case["page_size"], case["D"]
    if layout == "HND":
        s_page, s_head, s_tok = Hkv * P * D, P * D, D
    elif layout == "NHD":
        s_page, s_head, s_tok = P * Hkv * D, D, Hkv * D
    else:
        raise ValueError(layout)
    case.update(k_pool=k, v_pool=v, s_page=s_page, s_head=s_head, s_tok=s_tok,
                layout=layout, _stored=layout)
    return case


def config_case(index: int, B: Optional[int] = None, seed: Optional[int] = None,
                **overrides) -> dict:
    """Instance of workload ``index`` (seed 1000 + index unless given); ``B`` picks the
    batch of the two-batch HD64 workload (its pool is 6 pages per request)."""
    import dataclasses

    spec = WORKLOADS[index]
    if index == 2:
        B = 8 if B is None else B
        spec = dataclasses.replace(spec, B=B, seq_lens=(1536,) * B, pool_pages=6 * B)
    if overrides:
        spec = dataclasses.replace(spec, **overrides)
    return make_case(spec, SEED_BASE + index if seed is None else seed)


def sparse_indices(case: dict, topk: int, seed: int) -> np.ndarray:
    """[B, topk] int32 key positions for sparse decode: distinct positions drawn uniformly
    from each request's [0, L), ascending (a request shorter than topk lists all of its
    positions, then -1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = np.full((case["B"], topk), -1, np.int32)
    for b, L in enumerate(int(x) for x in case["seq_lens"]):
        n = min(L, topk)
        out[b, :n] = np.sort(rng.choice(L, size=n, replace=False))
    return out


def kv_bytes(case: dict) -> int:
    """Algorithmic KV bytes of one decode step: every valid token's K and V read once
    per KV head (fp8: plus one K and one V scale per (page, head) touched); for sparse
    decode, every listed valid position once."""
    if case.get("topk"):
        idx = np.asarray(case["indices"])
        L = np.asarray(case["seq_lens"], np.int64)[:, None]
        return int(((idx >= 0) & (idx < L)).sum() * MLA_TOKEN_BYTES)
    L = np.asarray(case["seq_lens"], np.int64)
    Hkv, D, Dv, P = case["Hkv"], case["D"], case["Dv"], case["page_size"]
    fmt = case["kv_format"]
    if fmt == KV_BF16:
        return int(L.sum() * Hkv * (D + Dv) * 2)
    if fmt == KV_FP8_PAGE_HEAD:
        pages = (-(-L // P)).sum()
        return int(L.sum() * Hkv * (D + Dv) + pages * Hkv * 8)
    return int(L.sum() * MLA_TOKEN_BYTES)


def io_bytes(case: dict) -> int:
    """q, out (bf16), lse (fp32), block table and seq_lens bytes of one step."""
    B, Hkv, G, D, Dv = case["B"], case["Hkv"], case["G"], case["D"], case["Dv"]
    R = Hkv * G * case.get("q_len", 1)          # query rows per request
    P = case["page_size"]
    pages = int((-(-np.asarray(case["seq_lens"], np.int64) // P)).sum())
    return B * R * D * 2 + B * R * Dv * 2 + B * R * 4 + pages * 4 + B * 4
