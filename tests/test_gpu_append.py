"""GPU KV append (pa_kv_append) against the oracle's append, bit for bit: pools (codes
and bf16 bits) and fp8 scale tables must be identical, since every quantisation
decision is taken in fp32 on both sides.  Then attention over the appended cache."""
import numpy as np
import pytest
import torch

import oracle
from mqa_split_kv_amd import binding as pb
from mqa_split_kv_amd import synth

from gpu_util import DecodeRun, assert_parity, to_device
from test_oracle_append import _case, _new_tokens

pytestmark = pytest.mark.gpu


def _t(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def _gpu_append(case, n_new, k_new, v_new):
    """Run pa_kv_append on device copies of the case; returns host copies of the pools
    and scales afterwards."""
    dev = to_device(case)
    desc = pb.desc_from_case(case)
    kn, vn = _t(k_new), (None if v_new is None else _t(v_new))
    pb.pa_kv_append(desc, n_new, kn, vn, dev["block_table"], dev["seq_lens"], dev["k_pool"],
                    dev["v_pool"], dev["k_scale"], dev["v_scale"])
    torch.cuda.synchronize()
    out = dict(case)

    def back(t, like):
        x = t.cpu().numpy()
        return x.view(np.uint16) if like.dtype == np.uint16 else x

    out["k_pool"] = back(dev["k_pool"], case["k_pool"])
    out["v_pool"] = None if dev["v_pool"] is None else back(dev["v_pool"], case["v_pool"])
    for key in ("k_scale", "v_scale"):
        out[key] = None if dev[key] is None else dev[key].cpu().numpy()
    return out


def _assert_same(got, ref):
    np.testing.assert_array_equal(got["k_pool"], ref["k_pool"])
    if ref.get("v_pool") is not None:
        np.testing.assert_array_equal(got["v_pool"], ref["v_pool"])
    for key in ("k_scale", "v_scale"):
        if ref.get(key) is not None:
            np.testing.assert_array_equal(got[key].view(np.uint32), ref[key].view(np.uint32))


APPEND = [
    (synth.KV_BF16, "HND", (20, 16, 47, 5), 5, 1.0),
    (synth.KV_BF16, "NHD", (20, 16, 47, 5), 1, 1.0),
    (synth.KV_FP8_PAGE_HEAD, "HND", (20, 16, 47, 5), 1, 1.0),
    (synth.KV_FP8_PAGE_HEAD, "HND", (20, 16, 47, 37), 3, 4.0),     # scale growth
    (synth.KV_FP8_PAGE_HEAD, "NHD", (40, 37, 64, 70), 37, 2.0),    # spans pages
    (synth.KV_FP8_PAGE_HEAD, "HND", (40, 33, 64, 70), 16, 1e-3),   # tiny values
    (synth.KV_MLA656, "HND", (9, 64, 65), 2, 3.0),
    (synth.KV_MLA656, "HND", (130, 64, 1), 1, 1e-4),
]


@pytest.mark.parametrize("fmt,layout,lens,n_new,spread", APPEND)
def test_append_matches_oracle_bitwise(fmt, layout, lens, n_new, spread):
    D = 128 if fmt == synth.KV_FP8_PAGE_HEAD else 64
    P = 64 if fmt == synth.KV_MLA656 else 16
    Hq = 16 if fmt == synth.KV_MLA656 else 8          # MLA descriptors take G in 16s
    case = _case(fmt, lens, Hq=Hq, D=D, P=P, layout=layout)
    k_new, v_new = _new_tokens(case, n_new, spread=spread)
    ref = oracle.kv_append(case, n_new, k_new, v_new)
    got = _gpu_append(case, n_new, k_new, v_new)
    _assert_same(got, ref)


def test_append_token_by_token_growth_matches_oracle():
    """20 appends of one token with growing magnitudes: the pages' scales grow and their
    older codes are re-encoded again and again; GPU and oracle stay identical."""
    case = _case(synth.KV_FP8_PAGE_HEAD, (20, 20, 20), D=64, P=16)
    ref = dict(case)
    for i in range(20):
        L = i + 1
        ref["seq_lens"] = np.full(3, L, np.int32)
        k_new, v_new = _new_tokens(ref, 1, seed=50 + i, spread=1.0 + 0.5 * i)
        got = _gpu_append(ref, 1, k_new, v_new)
        ref = oracle.kv_append(ref, 1, k_new, v_new)
        _assert_same(got, ref)


@pytest.mark.parametrize("fmt", [synth.KV_BF16, synth.KV_FP8_PAGE_HEAD])
def test_append_then_speculative_decode(fmt):
    """Append a 3-token draft, then attend with q_len = 3 over the appended cache: the
    result matches the oracle over the oracle's appended cache."""
    lens = (100, 35, 260)
    n_new = 3
    case = _case(fmt, lens, Hq=16, Hkv=2, D=128, P=16)
    k_new, v_new = _new_tokens(case, n_new, seed=77)
    ref = oracle.kv_append(case, n_new, k_new, v_new)
    got = _gpu_append(case, n_new, k_new, v_new)
    _assert_same(got, ref)
    rng = np.random.default_rng(8)
    q = synth.f32_to_bf16_bits(rng.standard_normal((len(lens), n_new, 16, 128)).astype(np.float32))
    spec_case = dict(ref, q=q, q_len=n_new)
    out, lse = DecodeRun(spec_case)()
    ref_out, ref_lse = oracle.decode(spec_case)
    assert_parity(spec_case, out, lse, ref_out, ref_lse)
