"""GPU parity at the largest sizes the library accepts (one step below each limit that
pa_decode_run rejects; the rejections themselves are host tests in test_abi.py):

* 4096 requests, the plan kernel's limit (it keeps every request's tile prefix in LDS);
* 256 fixed splits, the most chunks per request, most of them empty for short requests;
* 256 query rows per KV head for the bf16 / fp8 kernel (16 column tiles of 16 rows), as
  G = 4 heads x 64 draft tokens (the most draft tokens) and G = 16 x 16;
* 1024 query rows for the MLA kernel (G = 128 heads x 8 draft tokens: 16 head groups of 64),
  and the MLA kernel with 256 fixed splits;
* the smallest and largest page sizes (16 and 256 tokens) in one case each;
* logits in the thousands (query x 20, softmax scale 1): the running maximum moves by far
  more than the exponent range between tiles, which the rescale and the MLA kernel's lazily
  moved reference must absorb.

Each result is compared element by element with the oracle at the parity bar of the
other GPU tests (|out diff| <= 1e-2 max|V|, |lse diff| <= 1e-3); the plan words of the
4096-request plan are compared word for word.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import plan as oplan
from mqa_split_kv_amd import binding as pb
from mqa_split_kv_amd import synth

from gpu_util import DecodeRun, assert_parity

pytestmark = pytest.mark.gpu

MAX_BATCH = 4096


def _case(lens, Hq=4, Hkv=1, D=64, P=16, q_len=1, fmt=synth.KV_BF16, splits=0, seed=5):
    used = sum(-(-L // P) for L in lens)
    spec = synth.CaseSpec(B=len(lens), Hq=Hq, Hkv=Hkv, D=D, Dv=D, page_size=P, seq_lens=lens,
                          kv_format=fmt, pool_pages=used + 3, num_splits=splits, q_len=q_len)
    return synth.make_case(spec, seed)


def _mla_case(lens, G=128, P=64, q_len=1, splits=0, seed=13):
    used = sum(-(-L // P) for L in lens)
    spec = synth.CaseSpec(B=len(lens), Hq=G, Hkv=1, D=576, Dv=512, page_size=P, seq_lens=lens,
                          kv_format=synth.KV_MLA656, pool_pages=used + 2, num_splits=splits,
                          q_len=q_len)
    return synth.make_case(spec, seed)


def _max_batch_lens(seed=17):
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, 48, size=MAX_BATCH)
    lens[rng.choice(MAX_BATCH, 64, replace=False)] = 0     # empty requests among them
    lens[7] = 600                                          # one long request
    return tuple(int(x) for x in lens)


@pytest.mark.parametrize("splits", [0, 3])
def test_max_batch_plan_words(splits):
    lens = _max_batch_lens()
    desc = pb.make_desc(MAX_BATCH, 1, 4, 64, 64, 16, 1 << 16, 64, 16 * 64, 16 * 64, 64,
                        splits, pb.PA_KV_BF16)
    ref = oplan.plan_words(list(lens), splits, pb.pa_decode_num_parts(desc), n_rowgroups=1)
    pbytes, _ = pb.pa_decode_plan(desc)
    assert pbytes == ref.size * 4
    plan_t = torch.full(((pbytes + 3) // 4,), -7, dtype=torch.int32, device="cuda")
    pb.pa_decode_plan(desc, torch.tensor(lens, dtype=torch.int32, device="cuda"), plan_t)
    torch.cuda.synchronize()
    got = plan_t.cpu().numpy()
    n = oplan.valid_words(ref)
    assert np.array_equal(got[:n], ref[:n])


@pytest.mark.parametrize("splits", [0, 2])
def test_max_batch_parity(splits):
    case = _case(_max_batch_lens(), splits=splits)
    out, lse = DecodeRun(case)()
    ref_out, ref_lse = oracle.decode(case)
    assert_parity(case, out, lse, ref_out, ref_lse)


@pytest.mark.parametrize("fmt", [synth.KV_BF16, synth.KV_FP8_PAGE_HEAD])
def test_max_splits_parity(fmt):
    # 20000 tokens: 313 tiles of 64 in 157 chunks of 2 (99 empty); 70 tokens: 2 chunks of 1
    case = _case((20000, 70, 0), Hq=8, Hkv=2, D=128, P=64, fmt=fmt, splits=256)
    out, lse = DecodeRun(case)()
    ref_out, ref_lse = oracle.decode(case)
    assert_parity(case, out, lse, ref_out, ref_lse)


@pytest.mark.parametrize("kw", [dict(q_len=64, Hq=4, Hkv=1, lens=(70, 64, 300)),
                                dict(q_len=16, Hq=32, Hkv=2, D=128, P=32, lens=(500, 16, 33)),
                                dict(q_len=16, Hq=32, Hkv=2, D=128, P=32, lens=(500, 16, 33),
                                     fmt=synth.KV_FP8_PAGE_HEAD, splits=3)])
def test_max_query_rows_parity(kw):
    case = _case(**kw)
    out, lse = DecodeRun(case)()
    ref_out, ref_lse = oracle.decode(case)
    assert_parity(case, out, lse, ref_out, ref_lse)


def test_mla_max_query_rows_parity():
    case = _mla_case((150, 9, 70), q_len=8)
    out, lse = DecodeRun(case)()
    ref_out, ref_lse = oracle.decode(case)
    assert_parity(case, out, lse, ref_out, ref_lse)


def test_mla_max_splits_parity():
    case = _mla_case((5000, 3), G=16, splits=256)
    out, lse = DecodeRun(case)()
    ref_out, ref_lse = oracle.decode(case)
    assert_parity(case, out, lse, ref_out, ref_lse)


@pytest.mark.parametrize("P", [16, 256])
def test_page_size_extremes_parity(P):
    case = _case((1, P - 1, P, P + 1, 5 * P + 3), Hq=16, Hkv=2, D=128, P=P)
    out, lse = DecodeRun(case)()
    ref_out, ref_lse = oracle.decode(case)
    assert_parity(case, out, lse, ref_out, ref_lse)


def _scale_q(case, k):
    q = (case["q"].astype(np.uint32) << 16).view(np.float32) * np.float32(k)
    case["q"] = synth.f32_to_bf16_bits(q)


@pytest.mark.parametrize("fmt", [synth.KV_BF16, synth.KV_FP8_PAGE_HEAD])
def test_extreme_logits_parity(fmt):
    case = _case((900, 5, 2100), Hq=16, Hkv=2, D=128, P=16, fmt=fmt, splits=0)
    _scale_q(case, 20.0)
    out, lse = DecodeRun(case)(scale=1.0)
    ref_out, ref_lse = oracle.decode(case, scale=1.0)
    assert np.max(np.abs(ref_lse)) > 500.0
    assert_parity(case, out, lse, ref_out, ref_lse)


def test_mla_extreme_logits_parity():
    """Logits in the thousands (query x 20, scale 1) on the MLA-656 path, at the plain bar:
    the scores run on bf16 MFMAs (exact products, fp32 sums) with the per-token tile scales
    applied in fp32, so their error stays a few fp32 roundings of the score."""
    case = _mla_case((900, 5, 2100), G=32, splits=0)
    _scale_q(case, 20.0)
    out, lse = DecodeRun(case)(scale=1.0)
    ref_out, ref_lse = oracle.decode(case, scale=1.0)
    assert np.max(np.abs(ref_lse)) > 500.0
    assert_parity(case, out, lse, ref_out, ref_lse)
