"""GPU parity for several query tokens per request (speculative decoding with a linear
draft: query token i of a request of length L sees keys [0, L - q_len + i + 1); XQA
article, section "投机解码: XQA 的第二个工作负载").  The G * q_len query rows of a KV
head share each K/V read; more than 16 rows take several column tiles."""
import numpy as np
import pytest

import oracle
from mqa_split_kv_amd import synth

from gpu_util import DecodeRun, assert_parity

pytestmark = pytest.mark.gpu


def _spec(q_len, fmt=synth.KV_BF16, Hq=8, Hkv=1, D=64, P=16, lens=(37, 64, 129),
          layout="HND", splits=0, seed=21):
    used = sum(-(-L // P) for L in lens)
    spec = synth.CaseSpec(B=len(lens), Hq=Hq, Hkv=Hkv, D=D, Dv=D, page_size=P, seq_lens=lens,
                          kv_format=fmt, pool_pages=used + 3, layout=layout,
                          num_splits=splits, q_len=q_len)
    return synth.make_case(spec, seed)


SPEC_CASES = [
    dict(q_len=2),                                                     # 16 rows, one tile
    dict(q_len=2, splits=1),
    dict(q_len=2, splits=3, lens=(1, 2, 65, 200)),                     # L < q_len, L = q_len
    dict(q_len=4, Hq=32, Hkv=8, D=128, P=16, lens=(2000, 33, 4097)),   # G = 4: 16 rows
    dict(q_len=3, Hq=16, Hkv=2, D=128, P=32, lens=(700, 5, 1300)),     # 24 rows: 2 tiles
    dict(q_len=8, Hq=8, Hkv=1, D=128, P=64, lens=(3000, 9), splits=2),  # 64 rows: 4 tiles
    dict(q_len=16, Hq=1, Hkv=1, D=64, P=16, lens=(16, 300, 40)),       # G = 1, 16 rows
    dict(q_len=5, layout="NHD", Hq=16, Hkv=2, D=128, P=16, lens=(129, 7, 640)),
    dict(q_len=2, fmt=synth.KV_FP8_PAGE_HEAD, Hq=32, Hkv=8, D=128, P=16, lens=(300, 17, 1025)),
    dict(q_len=3, fmt=synth.KV_FP8_PAGE_HEAD, Hq=8, Hkv=2, D=64, P=32, lens=(64, 65, 2),
         splits=2),
    dict(q_len=2, lens=(0, 50, 0)),
]


@pytest.mark.parametrize("kw", SPEC_CASES)
def test_spec_parity(kw):
    case = _spec(**kw)
    out, lse = DecodeRun(case)()
    ref_out, ref_lse = oracle.decode(case)
    assert out.shape == ref_out.shape
    assert_parity(case, out, lse, ref_out, ref_lse)


@pytest.mark.parametrize("kw", [dict(q_len=3, Hq=16, Hkv=2, D=128, P=32, lens=(700, 5, 1300)),
                                dict(q_len=2, splits=3, lens=(1, 2, 65, 200))])
def test_spec_fused_equals_separate(kw):
    case = _spec(**kw)
    o1, l1 = DecodeRun(case)()
    o2, l2 = DecodeRun(case, fused=True)()
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_spec_draft_token_sees_exactly_its_prefix():
    """Plant a dominant key at the position of draft token 1 (t = L - q_len + 1): draft
    token 0 must not see it (its causal limit ends just before), tokens 1.. must."""
    q_len, L, D, P = 3, 130, 128, 16
    case = _spec(q_len, Hq=8, Hkv=1, D=D, P=P, lens=(L,))
    rng = np.random.default_rng(3)
    u = rng.standard_normal(D).astype(np.float32)
    u /= np.linalg.norm(u)
    case["q"][0] = synth.f32_to_bf16_bits(np.tile(u * 4.0, (q_len, 8, 1)))
    t = L - q_len + 1
    page = case["block_table"][0, t // P]
    case["k_pool"][page, 0, t % P] = synth.f32_to_bf16_bits(u * 12.0)
    scale = 4.0 / np.sqrt(D)
    out, lse = DecodeRun(case)(scale=scale)
    ref_out, ref_lse = oracle.decode(case, scale=scale)
    assert_parity(case, out, lse, ref_out, ref_lse)
    from test_oracle import dense_kv
    _K, V = dense_kv(case, 0, 0)
    assert np.abs(out[0, 0] - V[t]).max() > 0.3            # token 0 cannot see key t
    for qi in (1, 2):
        np.testing.assert_allclose(out[0, qi], np.tile(V[t], (8, 1)), atol=0.05)


def test_spec_llama70b_shape_sampled():
    """The Llama-70B-like workload with two draft tokens per request (16 query rows per
    KV head: the MFMA columns are all used), balanced plan, sampled pairs."""
    case = synth.config_case(1, q_len=2)
    out, lse = DecodeRun(case)()
    B, Hkv, G = case["B"], case["Hkv"], case["G"]
    pairs = np.zeros((B, Hkv), bool)
    pairs[[0, 13, 31], [0, 5, 7]] = True
    ref_out, ref_lse = oracle.decode(case, pairs=pairs)
    rows = np.repeat(pairs, G, axis=1)[:, None, :].repeat(2, axis=1)
    assert_parity(case, out, lse, ref_out, ref_lse, rows=rows)


def _mla_spec(q_len, lens, G=64, P=64, splits=0, seed=41):
    used = sum(-(-L // P) for L in lens)
    spec = synth.CaseSpec(B=len(lens), Hq=G, Hkv=1, D=576, Dv=512, page_size=P, seq_lens=lens,
                          kv_format=synth.KV_MLA656, pool_pages=used + 2, num_splits=splits,
                          q_len=q_len)
    return synth.make_case(spec, seed)


@pytest.mark.parametrize("kw", [dict(q_len=2, lens=(300, 2, 1000)),
                                dict(q_len=2, lens=(300, 2, 1000), G=128, splits=3),
                                dict(q_len=3, lens=(65, 700), G=16, P=32, splits=1),
                                dict(q_len=4, lens=(5000, 3), G=32)])
def test_spec_mla_parity(kw):
    case = _mla_spec(**kw)
    out, lse = DecodeRun(case)()
    ref_out, ref_lse = oracle.decode(case)
    assert out.shape == ref_out.shape
    assert_parity(case, out, lse, ref_out, ref_lse)


def test_spec_mla_with_window_and_sinks():
    case = _mla_spec(2, (700, 40, 1300), G=64)
    rng = np.random.default_rng(12)
    case["window"] = 200
    case["sinks"] = (rng.standard_normal(64) + 1.0).astype(np.float32)
    out, lse = DecodeRun(case)()
    ref_out, ref_lse = oracle.decode(case)
    assert_parity(case, out, lse, ref_out, ref_lse)
