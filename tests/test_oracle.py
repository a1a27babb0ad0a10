"""Pins of the CPU oracle against things other than itself (no GPU needed).

* dense attention from library routines (torch SDPA in float64 and scipy's
  logsumexp) on contiguous K/V gathered with numpy fancy indexing;
* element codecs against torch's own bf16 / float8_e4m3fn conversions;
* closed forms (one token, identical keys, zero query, one dominant logit);
* invariances (page relocation, page-size repacking, HND vs NHD, garbage in unused
  slots, other heads' data, GQA vs expanded MHA, split + merge vs whole);
* the worked rescale example of the pipelining page (tests/golden).
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from mqa_split_kv_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------------------
# Independent dense path: numpy gather + torch dequantisation + library attention
# --------------------------------------------------------------------------------------

def _bf16_to_f64(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).double().numpy()


def _e4m3_to_f64(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()


def dense_kv(case, b, h):
    """Contiguous dequantised K [L, D] and V [L, Dv] of (request b, KV head h)."""
    L, P = int(case["seq_lens"][b]), case["page_size"]
    t = np.arange(L)
    pages = case["block_table"][b, t // P]
    slots = t % P
    fmt = case["kv_format"]
    if fmt == synth.KV_MLA656:
        tok = case["k_pool"][pages, slots]                     # [L, 656]
        nope = _e4m3_to_f64(tok[:, :512])
        sc = np.ascontiguousarray(tok[:, 512:528]).view(np.float32).astype(np.float64)  # [L, 4]
        nope = nope * np.repeat(sc, 128, axis=1)
        rope = _bf16_to_f64(np.ascontiguousarray(tok[:, 528:656]).view(np.uint16))
        K = np.concatenate([nope, rope], axis=1)
        return K, K[:, :512].copy()
    out = []
    for pool, scl in ((case["k_pool"], case["k_scale"]), (case["v_pool"], case["v_scale"])):
        if case["layout"] == "HND":
            raw = pool[pages, h, slots]
        else:
            raw = pool[pages, slots, h]
        if fmt == synth.KV_BF16:
            x = _bf16_to_f64(raw)
        else:
            x = _e4m3_to_f64(raw) * scl[pages, h].astype(np.float64)[:, None]
        out.append(x)
    return out[0], out[1]


def library_attention(case, scale=None):
    """(out, lse) from torch SDPA (float64, CPU) and scipy logsumexp."""
    B, Hkv, G, Dv = case["B"], case["Hkv"], case["G"], case["Dv"]
    sc = case["scale"] if scale is None else scale
    q = _bf16_to_f64(case["q"])                                 # [B, Hq, D]
    out = np.zeros((B, Hkv * G, Dv))
    lse = np.full((B, Hkv * G), -np.inf)
    for b in range(B):
        for h in range(Hkv):
            K, V = dense_kv(case, b, h)
            if K.shape[0] == 0:
                continue
            qg = q[b, h * G:(h + 1) * G]                        # [G, D]
            o = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(qg)[None, :, None, :],
                torch.from_numpy(K)[None, None].expand(1, G, -1, -1),
                torch.from_numpy(V)[None, None].expand(1, G, -1, -1), scale=sc)
            out[b, h * G:(h + 1) * G] = o[0, :, 0].numpy()
            lse[b, h * G:(h + 1) * G] = scipy.special.logsumexp(sc * (qg @ K.T), axis=1)
    return out, lse


def small_case(fmt=synth.KV_BF16, B=3, Hq=8, Hkv=2, D=64, P=16, lens=(37, 64, 129),
               layout="HND", pool_extra=5, seed=7):
    Dv = 512 if fmt == synth.KV_MLA656 else D
    if fmt == synth.KV_MLA656:
        Hkv, D = 1, 576
    used = sum(-(-L // P) for L in lens)
    spec = synth.CaseSpec(B=B, Hq=Hq, Hkv=Hkv, D=D, Dv=Dv, page_size=P, seq_lens=lens,
                          kv_format=fmt, pool_pages=used + pool_extra, layout=layout)
    return synth.make_case(spec, seed)


CASES = [
    dict(),
    dict(Hq=4, Hkv=4, D=128, P=32, lens=(1, 33, 200)),          # MHA-like, G = 1
    dict(Hq=16, Hkv=1, D=64, P=64, lens=(300, 5, 64)),            # MQA, G = 16
    dict(layout="NHD"),
    dict(fmt=synth.KV_FP8_PAGE_HEAD, Hq=8, Hkv=2, D=128, lens=(17, 90, 250)),
    dict(fmt=synth.KV_MLA656, Hq=8, P=16, lens=(20, 47, 3)),
]


@pytest.mark.parametrize("kw", CASES)
def test_oracle_matches_library_attention(kw):
    case = small_case(**kw)
    out, lse = oracle.decode(case)
    ref_out, ref_lse = library_attention(case)
    np.testing.assert_allclose(out, ref_out, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_oracle_zero_length_request():
    case = small_case(lens=(0, 40, 0))
    out, lse = oracle.decode(case)
    assert np.all(out[0] == 0) and np.all(out[2] == 0)
    assert np.all(np.isneginf(lse[0])) and np.all(np.isneginf(lse[2]))
    ref_out, ref_lse = library_attention(case)
    np.testing.assert_allclose(out[1], ref_out[1], rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------------------
# Codecs
# --------------------------------------------------------------------------------------

def test_e4m3_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(mine[~nan], ref[~nan])
    assert mine[0x7E] == 448.0 and mine[0xFE] == -448.0       # largest finite magnitude
    assert mine[0x01] == 2.0 ** -9                            # smallest subnormal


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 1 << 16, size=100000, dtype=np.uint16)
    mine = oracle.bf16_decode(bits)
    ref = _bf16_to_f64(bits)
    same = (mine == ref) | (np.isnan(mine) & np.isnan(ref))
    assert same.all()


def test_mla656_roundtrip():
    rng = np.random.Generator(np.random.PCG64(11))
    x = rng.standard_normal((50, 576), dtype=np.float32)
    nope = x[:, :512].reshape(50, 4, 128)
    sc = (np.abs(nope).max(-1) / np.float32(448.0)).astype(np.float32)
    codes = synth.f32_to_e4m3_codes(nope / sc[..., None]).reshape(50, 512)
    tok = np.zeros((50, 656), np.uint8)
    tok[:, :512] = codes
    tok[:, 512:528] = sc.view(np.uint8).reshape(50, 16)
    tok[:, 528:] = synth.f32_to_bf16_bits(x[:, 512:]).view(np.uint8).reshape(50, 128)
    k = oracle.mla656_unpack(tok)
    # exact against torch's own decoders
    ref_nope = _e4m3_to_f64(codes) * np.repeat(sc.astype(np.float64), 128, axis=1)
    assert np.array_equal(k[:, :512], ref_nope)
    assert np.array_equal(k[:, 512:], _bf16_to_f64(synth.f32_to_bf16_bits(x[:, 512:])))
    # and close to the values before quantisation (e4m3 keeps 3 mantissa bits)
    err = np.abs(k[:, :512] - x[:, :512]).reshape(50, 4, 128)
    assert np.all(err <= (np.abs(x[:, :512]).reshape(50, 4, 128) * 2.0 ** -4 + sc[..., None] * 2.0 ** -9 + 1e-12))
    assert np.all(np.abs(k[:, 512:] - x[:, 512:]) <= np.abs(x[:, 512:]) * 2.0 ** -8 + 1e-30)


# --------------------------------------------------------------------------------------
# Closed forms
# --------------------------------------------------------------------------------------

def test_single_token_gives_its_value_row():
    case = small_case(lens=(1, 1, 1), D=64)
    out, lse = oracle.decode(case)
    q = _bf16_to_f64(case["q"])
    for b in range(case["B"]):
        for h in range(case["Hkv"]):
            K, V = dense_kv(case, b, h)
            for g in range(case["G"]):
                assert np.array_equal(out[b, h * case["G"] + g], V[0])
                s0 = case["scale"] * float(q[b, h * case["G"] + g] @ K[0])
                assert abs(lse[b, h * case["G"] + g] - s0) <= 1e-12 * max(1.0, abs(s0))


def test_identical_keys_give_mean_value_and_log_count():
    case = small_case(lens=(50, 77, 16), D=64)
    P = case["page_size"]
    # every slot of every page holds the same key row (per head)
    row = case["k_pool"][0, :, 0, :].copy()                    # [Hkv, D]
    case["k_pool"][:] = row[None, :, None, :]
    out, lse = oracle.decode(case)
    q = _bf16_to_f64(case["q"])
    for b in range(case["B"]):
        L = int(case["seq_lens"][b])
        for h in range(case["Hkv"]):
            K, V = dense_kv(case, b, h)
            for g in range(case["G"]):
                hq = h * case["G"] + g
                np.testing.assert_allclose(out[b, hq], V.mean(axis=0), rtol=1e-12, atol=1e-13)
                s = case["scale"] * float(q[b, hq] @ K[0])
                assert abs(lse[b, hq] - (s + math.log(L))) < 1e-11
    assert P == 16


def test_zero_query_gives_mean_value_and_log_length():
    case = small_case(lens=(9, 100, 33))
    case["q"][:] = 0
    out, lse = oracle.decode(case)
    for b in range(case["B"]):
        L = int(case["seq_lens"][b])
        for h in range(case["Hkv"]):
            _K, V = dense_kv(case, b, h)
            G = case["G"]
            np.testing.assert_allclose(out[b, h * G:(h + 1) * G], np.broadcast_to(V.mean(0), (G, V.shape[1])),
                                       rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(lse[b, h * G:(h + 1) * G], math.log(L), rtol=0, atol=1e-12)


def test_dominant_logit_selects_its_value():
    case = small_case(lens=(64, 64, 64), D=64)
    out, _ = oracle.decode(case, scale=case["scale"] * 40.0)
    q = _bf16_to_f64(case["q"])
    for b in range(case["B"]):
        for h in range(case["Hkv"]):
            K, V = dense_kv(case, b, h)
            for g in range(case["G"]):
                hq = h * case["G"] + g
                s = K @ q[b, hq]
                top2 = np.sort(s)[-2:]
                if (top2[1] - top2[0]) * case["scale"] * 40.0 > 40:  # clear winner
                    np.testing.assert_allclose(out[b, hq], V[np.argmax(s)], atol=1e-12)


# --------------------------------------------------------------------------------------
# Invariances
# --------------------------------------------------------------------------------------

def test_page_relocation_invariance():
    case = small_case(lens=(40, 100, 7), pool_extra=9)
    out0, lse0 = oracle.decode(case)
    rng = np.random.default_rng(5)
    perm = rng.permutation(case["num_pages"])                  # new physical slot of page p
    moved = dict(case)
    kp = np.empty_like(case["k_pool"])
    vp = np.empty_like(case["v_pool"])
    kp[perm] = case["k_pool"]
    vp[perm] = case["v_pool"]
    moved.update(k_pool=kp, v_pool=vp, block_table=perm[case["block_table"]].astype(np.int32))
    out1, lse1 = oracle.decode(moved)
    assert np.array_equal(out0, out1) and np.array_equal(lse0, lse1)


def test_hnd_nhd_invariance():
    case = small_case(lens=(40, 100, 7))
    out0, lse0 = oracle.decode(case)
    synth.set_layout(case, "NHD")
    out1, lse1 = oracle.decode(case)
    assert np.array_equal(out0, out1) and np.array_equal(lse0, lse1)


@pytest.mark.parametrize("fmt", [synth.KV_BF16, synth.KV_FP8_PAGE_HEAD])
def test_garbage_in_unused_slots_is_ignored(fmt):
    case = small_case(fmt=fmt, lens=(40, 100, 7), pool_extra=6, D=128)
    out0, lse0 = oracle.decode(case)
    P = case["page_size"]
    rng = np.random.default_rng(9)
    used = np.zeros((case["num_pages"], P), bool)
    for b, L in enumerate(case["seq_lens"]):
        for t in range(int(L)):
            used[case["block_table"][b, t // P], t % P] = True
    for pool in (case["k_pool"], case["v_pool"]):
        junk = rng.integers(0, 256 if fmt else 65536, size=pool.shape).astype(pool.dtype)
        if fmt == synth.KV_FP8_PAGE_HEAD:
            junk[(junk & 0x7F) == 0x7F] = 0                   # no NaN codes
        else:
            junk[(junk & 0x7F80) == 0x7F80] = 0                # no inf/NaN bf16
        mask = ~used[:, None, :, None]
        np.copyto(pool, junk, where=np.broadcast_to(mask, pool.shape))
    out1, lse1 = oracle.decode(case)
    assert np.array_equal(out0, out1) and np.array_equal(lse0, lse1)


@pytest.mark.parametrize("fmt,layout,P,P_new", [(synth.KV_BF16, "HND", 16, 64),
                                                 (synth.KV_BF16, "NHD", 64, 16),
                                                 (synth.KV_BF16, "HND", 32, 256),
                                                 (synth.KV_MLA656, "HND", 64, 16),
                                                 (synth.KV_MLA656, "HND", 16, 256)])
def test_page_size_repacking_invariance(fmt, layout, P, P_new):
    """The same tokens stored with another page size (and other physical pages, and
    garbage elsewhere) give bit-identical results: the definition sums over token
    positions, pages only say where a token's bytes are."""
    from repack import repack
    case = small_case(fmt=fmt, layout=layout, P=P, lens=(40, 300, 7, 1), B=4, D=128)
    out0, lse0 = oracle.decode(case)
    moved = repack(case, P_new, seed=P_new)
    out1, lse1 = oracle.decode(moved)
    assert np.array_equal(out0, out1) and np.array_equal(lse0, lse1)
    # and the result is not vacuous: the library path agrees on the repacked cache
    ref_out, ref_lse = library_attention(moved)
    np.testing.assert_allclose(out1, ref_out, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse1, ref_lse, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("fmt", [synth.KV_BF16, synth.KV_FP8_PAGE_HEAD])
def test_other_heads_data_leaves_this_head_unchanged(fmt):
    """Changing the K/V of every other KV head and the queries of their groups leaves
    the rows of KV head h bit-identical, and changes the rows of the others."""
    case = small_case(fmt=fmt, Hq=16, Hkv=4, D=64, lens=(40, 100, 7))
    out0, lse0 = oracle.decode(case)
    G, Hkv, h = case["G"], case["Hkv"], 2
    other = [x for x in range(Hkv) if x != h]
    rng = np.random.default_rng(3)
    mod = dict(case)
    for key in ("k_pool", "v_pool"):
        a = case[key].copy()
        sel = a[:, other]                                     # HND: [page][head][P][D]
        a[:, other] = np.roll(sel, 1, axis=2)                 # other tokens' bytes
        mod[key] = a
    if fmt == synth.KV_FP8_PAGE_HEAD:
        for key in ("k_scale", "v_scale"):
            a = case[key].copy()
            a[:, other] *= np.float32(1.5)
            mod[key] = a
    q = case["q"].copy()
    rows = np.concatenate([np.arange(o * G, (o + 1) * G) for o in other])
    q[:, rows] = synth.f32_to_bf16_bits(rng.standard_normal(q[:, rows].shape).astype(np.float32))
    mod["q"] = q
    out1, lse1 = oracle.decode(mod)
    mine = slice(h * G, (h + 1) * G)
    assert np.array_equal(out0[:, mine], out1[:, mine]) and np.array_equal(lse0[:, mine], lse1[:, mine])
    assert not np.array_equal(lse0[:, rows], lse1[:, rows])


def test_mla_other_query_heads_leave_this_head_unchanged():
    """MQA: each query head's row depends on its own query only."""
    case = small_case(fmt=synth.KV_MLA656, Hq=32, P=16, lens=(20, 47, 3))
    out0, lse0 = oracle.decode(case)
    q = case["q"].copy()
    rng = np.random.default_rng(4)
    q[:, 1:] = synth.f32_to_bf16_bits(rng.standard_normal(q[:, 1:].shape).astype(np.float32))
    mod = dict(case, q=q)
    out1, lse1 = oracle.decode(mod)
    assert np.array_equal(out0[:, 0], out1[:, 0]) and np.array_equal(lse0[:, 0], lse1[:, 0])
    assert not np.array_equal(lse0[:, 1:], lse1[:, 1:])


def test_grouped_heads_equal_independent_mha():
    case = small_case(Hq=8, Hkv=2, lens=(30, 64, 90))
    out0, lse0 = oracle.decode(case)
    G, Hkv = case["G"], case["Hkv"]
    mha = dict(case)
    mha.update(Hkv=Hkv * G, G=1,
               k_pool=np.ascontiguousarray(np.repeat(case["k_pool"], G, axis=1)),
               v_pool=np.ascontiguousarray(np.repeat(case["v_pool"], G, axis=1)))
    P, D = case["page_size"], case["D"]
    mha.update(s_page=Hkv * G * P * D, s_head=P * D, s_tok=D)
    out1, lse1 = oracle.decode(mha)
    assert np.array_equal(out0, out1) and np.array_equal(lse0, lse1)


@pytest.mark.parametrize("splits", [1, 2, 3, 8])
def test_split_merge_equals_whole(splits):
    from oracle import plan
    case = small_case(lens=(1, 130, 257), D=64)
    items = plan.fixed_items(case["seq_lens"], splits)
    out1, lse1, _ = oracle.split_decode(case, items)
    out0, lse0 = oracle.decode(case)
    np.testing.assert_allclose(out1, out0, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse1, lse0, rtol=1e-13, atol=1e-12)


def test_merge_rescale_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "rescale_example.json")))
    m_old, m_new = g["old_max"], g["new_max"]
    l_old, l_new = 3.0, 5.0
    o_old = np.array([[1.0, -2.0]])
    o_new = np.array([[0.5, 4.0]])
    O, lse = oracle.merge(np.array([[m_old], [m_new]]), np.array([[l_old], [l_new]]),
                          np.stack([o_old, o_new]))
    f = math.exp(-2.0)
    assert abs(math.exp(m_old - m_new) - f) < 1e-15
    ell = l_old * f + l_new
    np.testing.assert_allclose(O[0], (o_old[0] * f + o_new[0]) / ell, rtol=1e-15)
    assert abs(lse[0] - (m_new + math.log(ell))) < 1e-14


def test_merge_skips_empty_partials():
    O, lse = oracle.merge(np.array([[-np.inf], [1.0]]), np.array([[0.0], [2.0]]),
                          np.array([[[0.0, 0.0]], [[2.0, 4.0]]]))
    np.testing.assert_array_equal(O[0], [1.0, 2.0])
    assert abs(lse[0] - (1.0 + math.log(2.0))) < 1e-15
    O, lse = oracle.merge(np.array([[-np.inf], [-np.inf]]), np.zeros((2, 1)), np.zeros((2, 1, 3)))
    assert np.all(O == 0) and np.isneginf(lse[0])


# --------------------------------------------------------------------------------------
# Several query tokens per request (linear draft, causal within the draft)
# --------------------------------------------------------------------------------------

def spec_case(q_len, fmt=synth.KV_BF16, B=3, Hq=8, Hkv=2, D=64, P=16, lens=(37, 64, 129),
              seed=9):
    used = sum(-(-L // P) for L in lens)
    spec = synth.CaseSpec(B=B, Hq=Hq, Hkv=Hkv, D=D, Dv=D, page_size=P, seq_lens=lens,
                          kv_format=fmt, pool_pages=used + 3, q_len=q_len)
    return synth.make_case(spec, seed)


def library_attention_multi(case):
    """Library path with an explicit boolean mask: query token i of a request of length L
    may see key t iff t <= L - q_len + i.  torch SDPA (float64) + scipy logsumexp."""
    B, Hkv, G, Dv, nq = case["B"], case["Hkv"], case["G"], case["Dv"], case["q_len"]
    sc = case["scale"]
    q = _bf16_to_f64(case["q"])                                 # [B, nq, Hq, D]
    out = np.zeros((B, nq, Hkv * G, Dv))
    lse = np.full((B, nq, Hkv * G), -np.inf)
    for b in range(B):
        L = int(case["seq_lens"][b])
        allowed = np.arange(L)[None, :] <= (L - nq + np.arange(nq))[:, None]     # [nq, L]
        for h in range(Hkv):
            K, V = dense_kv(case, b, h)
            for g in range(G):
                hq = h * G + g
                qq = q[b, :, hq]                                # [nq, D]
                rows = allowed.any(axis=1)
                o = torch.nn.functional.scaled_dot_product_attention(
                    torch.from_numpy(qq[rows])[None], torch.from_numpy(K)[None],
                    torch.from_numpy(V)[None], attn_mask=torch.from_numpy(allowed[rows])[None],
                    scale=sc)
                out[b, rows, hq] = o[0].numpy()
                logits = np.where(allowed, sc * (qq @ K.T), -np.inf)
                lse[b, rows, hq] = scipy.special.logsumexp(logits[rows], axis=1)
    return out, lse


@pytest.mark.parametrize("q_len,kw", [(2, {}), (4, dict(Hq=16, Hkv=4, D=128, P=32)),
                                      (3, dict(fmt=synth.KV_FP8_PAGE_HEAD, D=128)),
                                      (5, dict(lens=(5, 6, 40))), (2, dict(lens=(1, 2, 17)))])
def test_multi_token_matches_library_masked_attention(q_len, kw):
    case = spec_case(q_len, **kw)
    out, lse = oracle.decode(case)
    ref_out, ref_lse = library_attention_multi(case)
    assert out.shape == ref_out.shape
    np.testing.assert_allclose(out, ref_out, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(ref_lse))
    fin = np.isfinite(ref_lse)
    np.testing.assert_allclose(lse[fin], ref_lse[fin], rtol=1e-12, atol=1e-12)


def test_multi_token_first_draft_token_of_a_draft_only_request():
    """L = q_len: draft token 0 sees only key 0, so its output is v_0 and its lse s_0;
    a request shorter than the draft leaves its first tokens with nothing to see."""
    case = spec_case(3, lens=(3, 2, 20))
    out, lse = oracle.decode(case)
    G = case["G"]
    q = _bf16_to_f64(case["q"])
    for h in range(case["Hkv"]):
        K, V = dense_kv(case, 0, h)
        for g in range(G):
            np.testing.assert_allclose(out[0, 0, h * G + g], V[0], rtol=0, atol=1e-15)
            s0 = case["scale"] * float(q[0, 0, h * G + g] @ K[0])
            assert abs(lse[0, 0, h * G + g] - s0) < 1e-13
    assert np.all(out[1, 0] == 0) and np.all(np.isneginf(lse[1, 0]))
    assert np.all(np.isfinite(lse[1, 1:]))


def test_multi_token_last_draft_token_is_plain_decode():
    """The last draft token sees the whole request: it equals one-token decode of that q."""
    case = spec_case(4, Hq=8, Hkv=2, D=128, P=16, lens=(100, 33, 7))
    out, lse = oracle.decode(case)
    one = dict(case, q=np.ascontiguousarray(case["q"][:, -1]), q_len=1)
    out1, lse1 = oracle.decode(one)
    np.testing.assert_array_equal(out[:, -1], out1)
    np.testing.assert_array_equal(lse[:, -1], lse1)


@pytest.mark.parametrize("splits", [1, 2, 5])
def test_multi_token_split_merge_equals_whole(splits):
    from oracle import plan
    case = spec_case(3, lens=(3, 130, 257))
    items = plan.fixed_items(case["seq_lens"], splits)
    out1, lse1, _ = oracle.split_decode(case, items)
    out0, lse0 = oracle.decode(case)
    np.testing.assert_allclose(out1, out0, rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(np.isneginf(lse1), np.isneginf(lse0))
    fin = np.isfinite(lse0)
    np.testing.assert_allclose(lse1[fin], lse0[fin], rtol=1e-13, atol=1e-12)
