"""Pins of the byte and FLOP accounting behind every roofline fraction the benchmark
reports (CPU only).

* the MLA token is 656 bytes: 512 e4m3 codes, 4 fp32 scales, 64 bf16 rope values
  (FlashMLA walk-through, section 数据加载, byte-layout table), against a token that
  the generator packs (offsets of the scales and the rope values);
* the MLA FLOPs per token: the walk-through's matrix-core ledger for 64 query heads is
  64 x (576 + 512) x 2 FLOP, 34 cycles at 4096 FLOP per cycle (section 计算环节一);
  the benchmark counts 128 heads, twice that;
* its BF16 comparison: a 128K-token request's BF16 latent cache over 62 layers is
  576 x 2 x 62 x 128 x 1024 bytes = 8.72 GiB (section 数据加载), i.e. 1152 bytes per
  token and layer, which the 656-byte format nearly halves;
* KV bytes of a step, counted independently: every (valid token, KV head) read once
  by brute force over the block tables (and every (page, head) scale pair touched),
  against synth.kv_bytes, and the hand-computed totals of the workloads;
* the q / out / lse / table bytes of the Llama-70B-like workload, by hand.
"""
import os
import sys

import numpy as np
import pytest

from mqa_split_kv_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_mla_token_bytes_match_the_pages_layout():
    assert synth.MLA_TOKEN_BYTES == 512 * 1 + 4 * 4 + 64 * 2 == 656
    spec = synth.CaseSpec(B=1, Hq=16, Hkv=1, D=576, Dv=512, page_size=16, seq_lens=(16,),
                          kv_format=synth.KV_MLA656)
    case = synth.make_case(spec, 3)
    tok = case["k_pool"][case["block_table"][0, 0], 0]
    assert tok.shape == (656,)
    sc = tok[512:528].view(np.float32)              # 4 fp32 scales right after the codes
    assert np.all(sc > 0) and np.all(np.isfinite(sc))
    codes = tok[:512].reshape(4, 128)
    # scale = max|x| / 448 per 128 values: each tile's largest code is +-448 (0x7E / 0xFE)
    assert all(((c & 0x7F) == 0x7E).any() for c in codes)
    rope = tok[528:656].view(np.uint16)             # 64 bf16 values at the end
    assert rope.shape == (64,)


def test_mla_flops_per_token_match_the_pages_ledger():
    per_64_heads = 64 * (576 + 512) * 2
    assert round(per_64_heads / 4096) == 34          # the walk-through's 34 cycles
    assert bench.MLA_FLOP_PER_TOKEN == 2 * per_64_heads == 278528


def test_bf16_latent_cache_size_of_the_pages():
    per_token_layer = 576 * 2
    total = per_token_layer * 62 * 128 * 1024
    assert round(total / 2 ** 30, 2) == 8.72
    assert synth.MLA_TOKEN_BYTES / per_token_layer < 0.6    # "nearly halved"


def _brute_kv_bytes(case):
    """Bytes a step must read once: per valid token and KV head, its K row and its V row
    (element size of the format); for page-head FP8 also one K and one V scale per
    (page, KV head) that holds a valid token.  MLA: one 656-byte token per valid token."""
    L = case["seq_lens"]
    P = case["page_size"]
    fmt = case["kv_format"]
    total = 0
    for b in range(case["B"]):
        toks = np.arange(int(L[b]))
        if fmt == synth.KV_MLA656:
            total += toks.size * 656
            continue
        eb = 2 if fmt == synth.KV_BF16 else 1
        for _h in range(case["Hkv"]):
            total += toks.size * (case["D"] + case["Dv"]) * eb
            if fmt == synth.KV_FP8_PAGE_HEAD:
                total += np.unique(case["block_table"][b, toks // P]).size * 8
    return total


@pytest.mark.parametrize("fmt,kw", [
    (synth.KV_BF16, dict(Hq=8, Hkv=2, D=64, lens=(37, 64, 129))),
    (synth.KV_FP8_PAGE_HEAD, dict(Hq=8, Hkv=2, D=128, lens=(1, 16, 17, 300))),
    (synth.KV_MLA656, dict(Hq=16, Hkv=1, D=576, lens=(5, 70))),
])
def test_kv_bytes_against_brute_force(fmt, kw):
    lens = kw.pop("lens")
    Dv = 512 if fmt == synth.KV_MLA656 else kw["D"]
    spec = synth.CaseSpec(B=len(lens), Dv=Dv, page_size=16, seq_lens=lens, kv_format=fmt, **kw)
    case = synth.make_case(spec, 1)
    assert synth.kv_bytes(case) == _brute_kv_bytes(case)


def test_workload_byte_totals_by_hand():
    # Llama-70B-like: 32 requests x 4096 tokens x 8 KV heads x (128 + 128) bf16 values
    c1 = synth.WORKLOADS[1]
    n1 = c1.B * 4096 * c1.Hkv * (c1.D + c1.Dv) * 2
    assert n1 == 536870912
    # MLA: 64 requests x 8192 tokens x 656 bytes
    c4 = synth.WORKLOADS[4]
    assert c4.B * 8192 * 656 == 343932928
    # HD64, B = 8: 8 x 1536 tokens x 4 heads x (64 + 64) x 2 bytes
    c2 = synth.WORKLOADS[2]
    assert 8 * 1536 * c2.Hkv * (c2.D + c2.Dv) * 2 == 12582912


def test_io_bytes_of_the_llama_workload_by_hand():
    B, Hq, D = 32, 64, 128
    q = B * Hq * D * 2
    out = B * Hq * D * 2
    lse = B * Hq * 4
    table = B * 64 * 4                               # 64 pages of 64 tokens per request
    lens = B * 4
    case = dict(B=B, Hkv=8, G=8, D=D, Dv=D, page_size=64, seq_lens=np.full(B, 4096, np.int32))
    assert synth.io_bytes(case) == q + out + lse + table + lens == 1065088
    full = dict(case, kv_format=synth.KV_BF16)
    assert synth.kv_bytes(full) == 536870912
