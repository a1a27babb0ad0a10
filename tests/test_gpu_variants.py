"""GPU parity for the variants: sliding window, attention sinks, sparse top-k positions
(MLA), against the oracle on the same seeded inputs, and the plan words of windowed and
sparse plans against the oracle's partition twin."""
import numpy as np
import pytest
import torch

import oracle
from oracle import plan as oplan
from mqa_split_kv_amd import binding as pb
from mqa_split_kv_amd import synth

from gpu_util import DecodeRun, assert_parity
from test_gpu_decode import _case, _mla_case
from test_oracle_variants import _indices

pytestmark = pytest.mark.gpu


def _sinks(case, seed=3, loc=1.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(case["Hkv"] * case["G"]) * 2.0 + loc).astype(np.float32)


def _check(case, fused=False):
    out, lse = DecodeRun(case, fused=fused)()
    ref_out, ref_lse = oracle.decode(case)
    assert out.shape == ref_out.shape
    assert_parity(case, out, lse, ref_out, ref_lse)
    return out, lse


# ------------------------------------------------------------------------------ window

WINDOW = [
    dict(window=100, lens=(37, 640, 1290), splits=0),
    dict(window=1, lens=(37, 64, 129), splits=1),
    dict(window=64, Hq=32, Hkv=8, D=128, P=16, lens=(2000, 33, 4097), splits=3),
    dict(window=200, fmt=synth.KV_FP8_PAGE_HEAD, Hq=32, Hkv=8, D=128, P=16, lens=(300, 17, 1025)),
    dict(window=77, layout="NHD", Hq=16, Hkv=2, D=128, P=16, lens=(129, 7, 640)),
]


@pytest.mark.parametrize("kw", WINDOW)
def test_window_parity(kw):
    w = kw.pop("window")
    case = _case(**kw)
    case["window"] = w
    _check(case)


def test_window_with_draft_tokens():
    spec = synth.CaseSpec(B=3, Hq=16, Hkv=2, D=128, Dv=128, page_size=32, seq_lens=(700, 5, 1300),
                          pool_pages=70, q_len=3)
    case = synth.make_case(spec, 31)
    case["window"] = 90
    _check(case)


def test_window_mla():
    case = _mla_case((1000, 33, 300), G=64, P=64)
    case["window"] = 150
    _check(case)


@pytest.mark.parametrize("splits", [0, 2])
def test_window_plan_words(splits):
    lens = (0, 1, 63, 64, 65, 4000, 17, 9000)
    desc = pb.make_desc(len(lens), 8, 4, 128, 128, 16, 1 << 20, 1 << 14, 8 * 16 * 128, 16 * 128,
                        128, splits, pb.PA_KV_BF16, q_len=2, window=300)
    np_ = pb.pa_decode_num_parts(desc)
    ref = oplan.plan_words(list(lens), splits, np_, n_rowgroups=8, q_len=2, window=300)
    pbytes, _ = pb.pa_decode_plan(desc)
    assert pbytes == ref.size * 4
    plan_t = torch.full(((pbytes + 3) // 4,), -7, dtype=torch.int32, device="cuda")
    pb.pa_decode_plan(desc, torch.tensor(lens, dtype=torch.int32, device="cuda"), plan_t)
    torch.cuda.synchronize()
    got = plan_t.cpu().numpy()
    n = oplan.valid_words(ref)
    assert np.array_equal(got[:n], ref[:n])


# ------------------------------------------------------------------------------ sinks

SINKS = [
    dict(lens=(37, 640, 1290), splits=0),
    dict(lens=(37, 64, 129), splits=1),
    dict(lens=(0, 50, 0), splits=0),
    dict(lens=(0, 50, 0), splits=4),
    dict(fmt=synth.KV_FP8_PAGE_HEAD, Hq=32, Hkv=8, D=128, P=16, lens=(300, 17, 1025)),
]


@pytest.mark.parametrize("kw", SINKS)
def test_sinks_parity(kw):
    case = _case(**kw)
    case["sinks"] = _sinks(case)
    _check(case)


@pytest.mark.parametrize("kw", [dict(lens=(37, 640, 1290), splits=0), dict(lens=(0, 50, 0), splits=0)])
def test_sinks_fused_equals_separate(kw):
    case = _case(**kw)
    case["sinks"] = _sinks(case)
    o1, l1 = DecodeRun(case)()
    o2, l2 = DecodeRun(case, fused=True)()
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_sinks_dominant():
    """A sink far above every logit takes almost all the weight: out -> 0, lse -> sink."""
    case = _case(lens=(37, 640, 1290), splits=0)
    case["sinks"] = np.full(case["Hkv"] * case["G"], 40.0, np.float32)
    out, lse = _check(case)
    assert np.abs(out).max() < 1e-6
    np.testing.assert_allclose(lse, 40.0, atol=1e-5)


def test_sinks_with_draft_tokens():
    spec = synth.CaseSpec(B=3, Hq=16, Hkv=2, D=128, Dv=128, page_size=32, seq_lens=(700, 5, 1300),
                          pool_pages=70, q_len=2)
    case = synth.make_case(spec, 32)
    case["sinks"] = _sinks(case)
    _check(case)


@pytest.mark.parametrize("splits", [0, 1])
def test_sinks_mla(splits):
    case = _mla_case((1000, 33, 0, 300), G=64, P=64, splits=splits)
    case["sinks"] = _sinks(case)
    _check(case)


@pytest.mark.parametrize("splits", [0, 3])
def test_sinks_mla_fused_equals_separate(splits):
    case = _mla_case((1000, 33, 0, 300), G=64, P=64, splits=splits)
    case["sinks"] = _sinks(case)
    o1, l1 = DecodeRun(case)()
    o2, l2 = _check(case, fused=True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_window_mla_fused_equals_separate():
    case = _mla_case((1000, 33, 300), G=32, P=64)
    case["window"] = 200
    o1, l1 = DecodeRun(case)()
    o2, l2 = _check(case, fused=True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_sparse_mla_fused_is_unsupported():
    case = _mla_case((1000, 33, 300), G=16)
    case["topk"] = 64
    case["indices"] = _indices(case, 64)
    with pytest.raises(pb.PaDecodeError) as e:
        DecodeRun(case, fused=True)()
    assert e.value.status == pb.PA_ERR_UNSUPPORTED


# ------------------------------------------------------------------------------ sparse

SPARSE = [
    dict(lens=(1000, 33, 300), topk=64, splits=0),
    dict(lens=(1000, 33, 300), topk=100, splits=1),
    dict(lens=(5000, 2100), topk=2048, splits=0, G=128),
    dict(lens=(0, 700, 90), topk=37, splits=3, G=16, P=16),
]


@pytest.mark.parametrize("kw", SPARSE)
def test_sparse_mla_parity(kw):
    topk = kw.pop("topk")
    case = _mla_case(**kw)
    case.update(topk=topk, indices=_indices(case, topk))
    _check(case)


def test_sparse_mla_with_sinks():
    case = _mla_case((1000, 33, 300), G=64, P=64)
    case.update(topk=64, indices=_indices(case, 64), sinks=_sinks(case))
    _check(case)


def test_sparse_mla_needle():
    """One listed position holds a key aligned with the query: the output is its value
    row; any other listed position or an unlisted one would move it by O(1)."""
    import math
    case = _mla_case((600,), G=16, P=64)
    topk = 48
    idx = _indices(case, topk, dup=False, bad=True)
    t = int(idx[0, 10])
    rng = np.random.default_rng(5)
    u = rng.standard_normal(576).astype(np.float32)
    u /= np.linalg.norm(u)
    case["q"][0] = synth.f32_to_bf16_bits(np.tile(u * 4.0, (16, 1)))
    page = case["block_table"][0, t // 64]
    x = (u * 12.0).astype(np.float32)
    nope = x[:512].reshape(4, 128)
    sc = (np.abs(nope).max(-1) / np.float32(448.0)).astype(np.float32)
    tok = case["k_pool"][page, t % 64]
    tok[:512] = synth.f32_to_e4m3_codes(nope / sc[:, None]).reshape(512)
    tok[512:528] = sc.view(np.uint8)
    tok[528:] = synth.f32_to_bf16_bits(x[512:]).view(np.uint8)
    case.update(topk=topk, indices=idx)
    scale = 8.0 / math.sqrt(576)
    out, lse = DecodeRun(case)(scale=scale)
    ref_out, ref_lse = oracle.decode(case, scale=scale)
    assert_parity(case, out, lse, ref_out, ref_lse)
    v = oracle.mla656_unpack(tok)[:512]
    np.testing.assert_allclose(out[0], np.tile(v, (16, 1)), atol=0.05)


@pytest.mark.parametrize("splits", [0, 3])
def test_sparse_plan_words(splits):
    lens = (0, 700, 90, 5000)
    desc = pb.make_desc(len(lens), 1, 64, 576, 512, 64, 4096, 128, 64 * 656, 0, 656, splits,
                        pb.PA_KV_MLA656, topk=200)
    np_ = pb.pa_decode_num_parts(desc)
    ref = oplan.plan_words(list(lens), splits, np_, n_rowgroups=1, topk=200)
    pbytes, _ = pb.pa_decode_plan(desc)
    assert pbytes == ref.size * 4
    plan_t = torch.full(((pbytes + 3) // 4,), -7, dtype=torch.int32, device="cuda")
    pb.pa_decode_plan(desc, torch.tensor(lens, dtype=torch.int32, device="cuda"), plan_t)
    torch.cuda.synchronize()
    got = plan_t.cpu().numpy()
    n = oplan.valid_words(ref)
    assert np.array_equal(got[:n], ref[:n])


# ------------------------------------------------------------------------------ padding

@pytest.mark.parametrize("which", ["mla", "mla_splits", "bf16", "fp8"])
def test_nan_bytes_in_padding_slots_are_never_used(which):
    """Slots past each request's last token in its last page hold all-ones bytes (NaN
    codes, NaN scales, NaN bf16): the outputs stay finite and equal the oracle's."""
    if which.startswith("mla"):
        case = _mla_case((100, 33, 300, 64), G=64, P=64, splits=3 if which == "mla_splits" else 0)
    elif which == "bf16":
        case = _case(Hq=16, Hkv=2, D=128, P=64, lens=(100, 33, 300, 64))
    else:
        case = _case(fmt=synth.KV_FP8_PAGE_HEAD, Hq=16, Hkv=2, D=128, P=64, lens=(100, 33, 300, 64))
    P = case["page_size"]
    for b, L in enumerate(case["seq_lens"]):
        if L % P == 0:
            continue
        page = case["block_table"][b, (L - 1) // P]
        if which.startswith("mla"):
            case["k_pool"][page, L % P:] = 0xFF
        else:
            for pool in (case["k_pool"], case["v_pool"]):
                pool[page, :, L % P:] = 0xFFFF if pool.dtype == np.uint16 else 0xFF
    _check(case)
