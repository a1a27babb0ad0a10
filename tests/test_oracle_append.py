"""Pins of the oracle's e4m3 encoder and KV append (no GPU needed).

* the encoder against the format itself (decode/encode round trip of every finite
  code, ties to even at midpoints, saturation) and against torch's float8_e4m3fn cast
  (a library routine);
* bf16 append: the new tokens land exactly at positions L - n_new + j, nothing else
  changes;
* fp8 page-head append: the page scale is the running max|x| / 448 of everything the
  page received (equal to the static max|x| / 448 of the page), codes written without
  a scale change equal the library cast of fp32(x / scale), and every value stays
  within one e4m3 rounding per write and per later scale growth of its page;
* MLA-656 append: per-tile scales max|x| / 448, codes equal the library cast, rope bits
  copied.
"""
import numpy as np
import pytest
import torch

import oracle
from mqa_split_kv_amd import synth


def torch_e4m3(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


# ------------------------------------------------------------------------------ encoder

def test_encode_roundtrip_every_finite_code():
    c = np.arange(256, dtype=np.uint8)
    v = oracle.e4m3_decode(c)
    fin = ~np.isnan(v)
    assert fin.sum() == 254
    np.testing.assert_array_equal(oracle.e4m3_encode(v[fin].astype(np.float32)), c[fin])


def test_encode_ties_to_even_and_saturation():
    pos = np.arange(0, 0x7E, dtype=np.uint8)          # consecutive positive finite codes
    lo, hi = oracle.e4m3_decode(pos), oracle.e4m3_decode(pos + 1)
    mid = ((lo + hi) / 2).astype(np.float32)          # exact in fp32 (few mantissa bits)
    assert np.all(mid.astype(np.float64) == (lo + hi) / 2)
    enc = oracle.e4m3_encode(mid)
    even = np.where(pos % 2 == 0, pos, pos + 1)       # the code whose mantissa LSB is 0
    np.testing.assert_array_equal(enc, even)
    np.testing.assert_array_equal(oracle.e4m3_encode(np.array([448, 460, 1e6, -500], np.float32)),
                                  [0x7E, 0x7E, 0x7E, 0xFE])
    assert oracle.e4m3_encode(np.array([np.nan], np.float32))[0] == 0x7F


def test_encode_matches_library_cast():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(300000) * np.exp(rng.uniform(-16, 7, 300000))).astype(np.float32)
    x = np.clip(x, -448, 448)
    np.testing.assert_array_equal(oracle.e4m3_encode(x), torch_e4m3(x))


# ------------------------------------------------------------------------------ append

def _case(fmt, lens, Hq=8, Hkv=2, D=64, P=16, layout="HND", seed=3, extra=4):
    Dv = 512 if fmt == synth.KV_MLA656 else D
    if fmt == synth.KV_MLA656:
        Hkv, D = 1, 576
    used = sum(-(-L // P) for L in lens)
    spec = synth.CaseSpec(B=len(lens), Hq=Hq, Hkv=Hkv, D=D, Dv=Dv, page_size=P,
                          seq_lens=tuple(lens), kv_format=fmt, pool_pages=used + extra,
                          layout=layout)
    return synth.make_case(spec, seed)


def _new_tokens(case, n_new, seed=5, spread=1.0):
    rng = np.random.default_rng(seed)
    B = case["B"]
    if case["kv_format"] == synth.KV_MLA656:
        x = rng.standard_normal((B, n_new, 576)).astype(np.float32) * spread
        return synth.f32_to_bf16_bits(x), None
    shape = (B, n_new, case["Hkv"], case["D"])
    k = synth.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * spread)
    v = synth.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * spread)
    return k, v


def _bits_to_f32(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32)


def _slot_view(case, pool, page, h, slot):
    if case["layout"] == "HND":
        return pool[page, h, slot]
    return pool[page, slot, h]


@pytest.mark.parametrize("layout", ["HND", "NHD"])
def test_append_bf16_is_an_exact_scatter(layout):
    lens = (20, 16, 47, 5)
    n_new = 5
    case = _case(synth.KV_BF16, lens, layout=layout)
    k_new, v_new = _new_tokens(case, n_new)
    out = oracle.kv_append(case, n_new, k_new, v_new)
    P = case["page_size"]
    touched = np.zeros(case["k_pool"].shape[:-1], bool)
    for b, L in enumerate(lens):
        for j in range(n_new):
            pos = L - n_new + j
            page, slot = case["block_table"][b, pos // P], pos % P
            for h in range(case["Hkv"]):
                np.testing.assert_array_equal(_slot_view(case, out["k_pool"], page, h, slot), k_new[b, j, h])
                np.testing.assert_array_equal(_slot_view(case, out["v_pool"], page, h, slot), v_new[b, j, h])
                if layout == "HND":
                    touched[page, h, slot] = True
                else:
                    touched[page, slot, h] = True
    np.testing.assert_array_equal(out["k_pool"][~touched], case["k_pool"][~touched])
    np.testing.assert_array_equal(out["v_pool"][~touched], case["v_pool"][~touched])


def _grow(fmt, steps, B=3, P=16, Hkv=2, D=64, seed=11, spread_of=None):
    """Requests grow from empty by steps[i] tokens per call.  Returns the final case, the
    original fp32 values of every position per request ([L, Hkv, D] for K and V), and
    how often each (pool, page, head) scale grew while the page already held tokens."""
    total = sum(steps)
    case = _case(fmt, (total,) * B, Hkv=Hkv, D=D, P=P, seed=seed)
    orig_k = [[] for _ in range(B)]
    orig_v = [[] for _ in range(B)]
    growths = {}
    L = 0
    for i, n in enumerate(steps):
        before = {k: np.array(case[k], copy=True) for k in ("k_scale", "v_scale") if case.get(k) is not None}
        L0, L = L, L + n
        case["seq_lens"] = np.full(B, L, np.int32)
        spread = 1.0 if spread_of is None else spread_of(i)
        k_new, v_new = _new_tokens(case, n, seed=100 + i, spread=spread)
        case = oracle.kv_append(case, n, k_new, v_new)
        for b in range(B):
            orig_k[b].append(_bits_to_f32(k_new[b]))
            if v_new is not None:
                orig_v[b].append(_bits_to_f32(v_new[b]))
            if L0 % P and before:                     # the first touched page held tokens
                page = case["block_table"][b, L0 // P]
                for key in before:
                    for h in range(Hkv):
                        if case[key][page, h] != before[key][page, h]:
                            growths[(key, page, h)] = growths.get((key, page, h), 0) + 1
    ok = [np.concatenate(o) for o in orig_k]
    ov = [np.concatenate(o) for o in orig_v] if orig_v[0] else None
    return case, ok, ov, growths


@pytest.mark.parametrize("steps", [(16, 16, 16), (1,) * 40, (3, 5, 1, 7, 16, 2, 9), (37, 1, 1)])
def test_append_fp8_scale_is_the_running_max(steps):
    # growing magnitudes force rescaling of partly filled pages
    case, ok, ov, _ = _grow(synth.KV_FP8_PAGE_HEAD, steps, spread_of=lambda i: 1.0 + 0.7 * i)
    P = case["page_size"]
    L = sum(steps)
    for b in range(case["B"]):
        for lp in range(-(-L // P)):
            page = case["block_table"][b, lp]
            for h in range(case["Hkv"]):
                for orig, sc in ((ok, case["k_scale"]), (ov, case["v_scale"])):
                    amax = np.float32(np.abs(orig[b][lp * P:(lp + 1) * P, h]).max())
                    assert sc[page, h] == np.float32(amax / np.float32(448.0))


@pytest.mark.parametrize("steps,growing", [((1,) * 40, False), ((1,) * 40, True),
                                           ((3, 5, 1, 7, 16, 2, 9), True)])
def test_append_fp8_values_within_the_roundings_taken(steps, growing):
    """A value is rounded once when written and once more each time its page's scale
    grows afterwards: |dequantised - x| <= (1 + growths) * (2^-4 |x| + 2^-10 scale)."""
    case, ok, ov, growths = _grow(synth.KV_FP8_PAGE_HEAD, steps,
                                  spread_of=(lambda i: 1.0 + 0.7 * i) if growing else None)
    P = case["page_size"]
    L = sum(steps)
    worst = 0
    for b in range(case["B"]):
        for pos in range(L):
            page, slot = case["block_table"][b, pos // P], pos % P
            for h in range(case["Hkv"]):
                for key, orig, pool in (("k_scale", ok, case["k_pool"]), ("v_scale", ov, case["v_pool"])):
                    x = orig[b][pos, h].astype(np.float64)
                    s = float(case[key][page, h])
                    k = growths.get((key, page, h), 0)
                    worst = max(worst, k)
                    got = oracle.e4m3_decode(_slot_view(case, pool, page, h, slot)) * s
                    bound = (1 + k) * (2.0 ** -4 * np.abs(x) + 2.0 ** -10 * s) * 1.01
                    assert np.all(np.abs(got - x) <= bound)
    if growing:
        assert worst >= 3            # the case does exercise repeated requantisation


def test_append_fp8_codes_without_scale_change_equal_library_cast():
    """A fresh page filled in one call: codes are the library cast of fp32(x / scale)."""
    P = 16
    case = _case(synth.KV_FP8_PAGE_HEAD, (2 * P, P), P=P)
    n_new = P
    k_new, v_new = _new_tokens(case, n_new, seed=9)
    out = oracle.kv_append(case, n_new, k_new, v_new)
    for b in range(case["B"]):
        L = int(case["seq_lens"][b])
        page = case["block_table"][b, (L - 1) // P]
        for h in range(case["Hkv"]):
            for new, pool, sc in ((k_new, out["k_pool"], out["k_scale"]),
                                  (v_new, out["v_pool"], out["v_scale"])):
                x = _bits_to_f32(new[b, :, h])                     # [P, D]
                s = sc[page, h]
                assert s == np.float32(np.abs(x).max() / np.float32(448.0))
                want = torch_e4m3((x / s).astype(np.float32))
                got = np.stack([_slot_view(case, pool, page, h, t) for t in range(P)])
                np.testing.assert_array_equal(got, want)


def test_append_fp8_untouched_pages_and_heads_unchanged():
    case = _case(synth.KV_FP8_PAGE_HEAD, (40, 7, 33))
    n_new = 3
    k_new, v_new = _new_tokens(case, n_new)
    out = oracle.kv_append(case, n_new, k_new, v_new)
    P = case["page_size"]
    pages = {int(case["block_table"][b, (int(L) - 1 - j) // P])
             for b, L in enumerate(case["seq_lens"]) for j in range(n_new)}
    other = np.array([p for p in range(case["num_pages"]) if p not in pages])
    np.testing.assert_array_equal(out["k_pool"][other], case["k_pool"][other])
    np.testing.assert_array_equal(out["k_scale"][other], case["k_scale"][other])
    np.testing.assert_array_equal(out["v_scale"][other], case["v_scale"][other])


def test_append_mla_token():
    case = _case(synth.KV_MLA656, (9, 64, 65), P=64)
    n_new = 2
    k_new, _ = _new_tokens(case, n_new, spread=3.0)
    out = oracle.kv_append(case, n_new, k_new)
    P = case["page_size"]
    for b, L in enumerate(case["seq_lens"]):
        for j in range(n_new):
            pos = int(L) - n_new + j
            tok = out["k_pool"][case["block_table"][b, pos // P], pos % P]
            x = _bits_to_f32(k_new[b, j])
            sc = np.ascontiguousarray(tok[512:528]).view(np.float32)
            amax = np.abs(x[:512].reshape(4, 128)).max(-1)
            np.testing.assert_array_equal(sc, (amax / np.float32(448.0)).astype(np.float32))
            want = torch_e4m3((x[:512].reshape(4, 128) / sc[:, None]).astype(np.float32)).reshape(512)
            np.testing.assert_array_equal(tok[:512], want)
            np.testing.assert_array_equal(np.ascontiguousarray(tok[528:]).view(np.uint16), k_new[b, j, 512:])


def test_append_rejects_requests_shorter_than_the_draft():
    case = _case(synth.KV_BF16, (2, 9))
    k_new, v_new = _new_tokens(case, 3)
    with pytest.raises(ValueError):
        oracle.kv_append(case, 3, k_new, v_new)
