"""Test helper: the same logical KV cache stored with another page size.

Token t of request b (every KV head) keeps its bytes; only the page that holds it
changes: new page block_table'[b][t // P'] at slot t % P'.  The new pool's pages
are a random permutation, and every slot no valid token occupies holds random
bytes (finite values), so a result that depends on the page size, on a page's
position in the pool or on padding would show.  bf16 (HND or NHD strides) and
MLA-656 pools only: a page-head FP8 pool quantises with one scale per (page, head),
so its stored values themselves depend on the page size.
"""
from __future__ import annotations

import numpy as np

from mqa_split_kv_amd import synth


def _garbage(rng, shape, dtype):
    if dtype == np.uint16:                          # finite bf16 of moderate size
        x = rng.standard_normal(size=shape).astype(np.float32)
        return synth.f32_to_bf16_bits(x)
    return rng.integers(0, 256, size=shape).astype(np.uint8)


def repack(case: dict, P_new: int, seed: int = 0, extra_pages: int = 3) -> dict:
    fmt = case["kv_format"]
    assert fmt in (synth.KV_BF16, synth.KV_MLA656)
    rng = np.random.default_rng(seed)
    B, P = case["B"], case["page_size"]
    L = [int(x) for x in case["seq_lens"]]
    need = [-(-x // P_new) for x in L]
    n_pages = sum(need) + extra_pages
    max_pages = max(max(need), 1)
    perm = rng.permutation(n_pages).astype(np.int32)
    bt = np.zeros((B, max_pages), np.int32)
    pos = 0
    for b in range(B):
        bt[b, :need[b]] = perm[pos:pos + need[b]]
        pos += need[b]
    out = dict(case)
    out.update(page_size=P_new, num_pages=n_pages, max_pages=max_pages, block_table=bt)
    if fmt == synth.KV_MLA656:
        pool = case["k_pool"]                                   # [pages][P][656]
        new = _garbage(rng, (n_pages, P_new, pool.shape[2]), np.uint8)
        new[:, :, 512:528] = np.ones((n_pages, P_new, 4), np.float32).view(np.uint8)
        for b in range(B):
            t = np.arange(L[b])
            new[bt[b, t // P_new], t % P_new] = pool[case["block_table"][b, t // P], t % P]
        out.update(k_pool=new, s_page=P_new * pool.shape[2])
        return out
    Hkv, D = case["Hkv"], case["D"]
    layout = case["layout"]
    for key in ("k_pool", "v_pool"):
        pool = case[key]
        if layout == "HND":                                     # [pages][Hkv][P][D]
            new = _garbage(rng, (n_pages, Hkv, P_new, D), pool.dtype)
        else:                                                   # [pages][P][Hkv][D]
            new = _garbage(rng, (n_pages, P_new, Hkv, D), pool.dtype)
        for b in range(B):
            t = np.arange(L[b])
            src_p, src_s = case["block_table"][b, t // P], t % P
            dst_p, dst_s = bt[b, t // P_new], t % P_new
            if layout == "HND":
                new[dst_p, :, dst_s] = pool[src_p, :, src_s]
            else:
                new[dst_p, dst_s] = pool[src_p, src_s]
        out[key] = new
    if layout == "HND":
        out.update(s_page=Hkv * P_new * D, s_head=P_new * D, s_tok=D)
    else:
        out.update(s_page=P_new * Hkv * D, s_head=D, s_tok=Hkv * D)
    return out
