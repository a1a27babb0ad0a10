"""Pins of the oracle's variants (no GPU needed): sliding window, attention sinks and
sparse top-k positions, each against a library path that shares nothing with it:

* window: torch SDPA (float64) with the explicit boolean window-and-causal mask;
* sinks: SDPA over keys augmented with one extra "sink" key whose logit is the sink
  and whose value is zero (an extra dimension carries the logit);
* sparse: SDPA over the listed rows gathered with numpy fancy indexing;
plus closed forms (window 1 gives the newest value row; an empty request with a sink
gives lse = sink) and invariances (a window covering the request, indices listing every
position, split + merge)."""
import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import plan
from mqa_split_kv_amd import synth

from test_oracle import _bf16_to_f64, dense_kv


def _case(fmt=synth.KV_BF16, lens=(37, 64, 129), Hq=8, Hkv=2, D=64, P=16, q_len=1, seed=13,
          **extra):
    used = sum(-(-L // P) for L in lens)
    spec = synth.CaseSpec(B=len(lens), Hq=Hq, Hkv=Hkv, D=D, Dv=D, page_size=P,
                          seq_lens=tuple(lens), kv_format=fmt, pool_pages=used + 3, q_len=q_len)
    case = synth.make_case(spec, seed)
    case.update(extra)
    return case


def _q(case):
    q = _bf16_to_f64(case["q"])
    return q if case.get("q_len", 1) > 1 else q[:, None]          # [B, nq, Hq, D]


def library(case, allowed_fn=None, rows_fn=None, sinks=None):
    """SDPA per (b, h, g) over keys chosen by allowed_fn(b, L) -> bool [nq, L] or by
    rows_fn(b, L) -> gathered key rows; optional sink logits [Hq]."""
    B, Hkv, G, Dv = case["B"], case["Hkv"], case["G"], case["Dv"]
    nq = case.get("q_len", 1)
    sc = case["scale"]
    q = _q(case)
    out = np.zeros((B, nq, Hkv * G, Dv))
    lse = np.full((B, nq, Hkv * G), -np.inf)
    for b in range(B):
        L = int(case["seq_lens"][b])
        for h in range(Hkv):
            K, V = dense_kv(case, b, h)
            if rows_fn is not None:
                r = rows_fn(b, L)
                K, V = K[r], V[r]
                allowed = np.ones((nq, K.shape[0]), bool)
            else:
                allowed = allowed_fn(b, L)
            for g in range(G):
                hq = h * G + g
                qq = q[b, :, hq]
                Ka, Va, qa, al = K, V, qq, allowed
                if sinks is not None:      # augmented sink key: logit = sink, value = 0
                    Ka = np.concatenate([np.concatenate([K, np.zeros((K.shape[0], 1))], 1),
                                         np.concatenate([np.zeros((1, K.shape[1])),
                                                         [[sinks[hq] / sc]]], 1)])
                    Va = np.concatenate([V, np.zeros((1, Dv))])
                    qa = np.concatenate([qq, np.ones((nq, 1))], 1)
                    al = np.concatenate([allowed, np.ones((nq, 1), bool)], 1)
                rows = al.any(axis=1)
                if not rows.any():
                    continue
                o = torch.nn.functional.scaled_dot_product_attention(
                    torch.from_numpy(qa[rows])[None], torch.from_numpy(Ka)[None],
                    torch.from_numpy(Va)[None], attn_mask=torch.from_numpy(al[rows])[None],
                    scale=sc)
                out[b, rows, hq] = o[0].numpy()
                logits = np.where(al, sc * (qa @ Ka.T), -np.inf)
                lse[b, rows, hq] = scipy.special.logsumexp(logits[rows], axis=1)
    if nq == 1:
        return out[:, 0], lse[:, 0]
    return out, lse


def _close(case, got, ref):
    out, lse = got
    ref_out, ref_lse = ref
    np.testing.assert_allclose(out, ref_out, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(ref_lse))
    fin = np.isfinite(ref_lse)
    np.testing.assert_allclose(lse[fin], ref_lse[fin], rtol=1e-12, atol=1e-12)


def _window_mask(W, nq):
    def f(b, L):
        p = L - nq + np.arange(nq)
        t = np.arange(L)
        return (t[None] <= p[:, None]) & (t[None] >= p[:, None] - W + 1)
    return f


# ------------------------------------------------------------------------------ window

@pytest.mark.parametrize("W,q_len,kw", [(5, 1, {}), (64, 1, {}), (1, 1, {}), (17, 3, {}),
                                        (40, 2, dict(fmt=synth.KV_FP8_PAGE_HEAD, D=128)),
                                        (3, 4, dict(lens=(2, 9, 300)))])
def test_window_matches_library_masked_attention(W, q_len, kw):
    case = _case(q_len=q_len, window=W, **kw)
    _close(case, oracle.decode(case), library(case, allowed_fn=_window_mask(W, q_len)))


def test_window_covering_the_request_is_no_window():
    case = _case(lens=(37, 64, 129))
    a = oracle.decode(case)
    b = oracle.decode(dict(case, window=129))
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_window_of_one_gives_the_newest_value_row():
    case = _case(window=1)
    out, lse = oracle.decode(case)
    G = case["G"]
    q = _q(case)
    for b, L in enumerate(case["seq_lens"]):
        for h in range(case["Hkv"]):
            K, V = dense_kv(case, b, h)
            for g in range(G):
                np.testing.assert_allclose(out[b, h * G + g], V[L - 1], rtol=0, atol=1e-15)
                assert abs(lse[b, h * G + g] - case["scale"] * q[b, 0, h * G + g] @ K[L - 1]) < 1e-12


# ------------------------------------------------------------------------------ sinks

@pytest.mark.parametrize("q_len,kw", [(1, {}), (1, dict(fmt=synth.KV_FP8_PAGE_HEAD, D=128)),
                                      (3, {}), (1, dict(lens=(0, 5, 300)))])
def test_sinks_match_library_with_a_sink_key(q_len, kw):
    rng = np.random.default_rng(4)
    case = _case(q_len=q_len, **kw)
    sinks = (rng.standard_normal(case["Hkv"] * case["G"]) * 2.0 + 1.0).astype(np.float32)
    case["sinks"] = sinks
    nq = q_len

    def causal(b, L):
        p = L - nq + np.arange(nq)
        return np.arange(L)[None] <= p[:, None]
    _close(case, oracle.decode(case), library(case, allowed_fn=causal, sinks=sinks.astype(np.float64)))


def test_sink_closed_forms():
    case = _case(lens=(0, 40))
    sinks = np.linspace(-1, 2, case["Hkv"] * case["G"]).astype(np.float32)
    out, lse = oracle.decode(dict(case, sinks=sinks))
    assert np.all(out[0] == 0)
    np.testing.assert_array_equal(lse[0], sinks.astype(np.float64))   # empty request: lse = sink
    out0, lse0 = oracle.decode(case)
    # a sink scales the output by l / (l + e^sink) and adds e^sink to the denominator
    f = np.exp(lse0[1]) / (np.exp(lse0[1]) + np.exp(sinks.astype(np.float64)))
    np.testing.assert_allclose(out[1], out0[1] * f[:, None], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse[1], np.logaddexp(lse0[1], sinks.astype(np.float64)), rtol=1e-13)


# ------------------------------------------------------------------------------ sparse

def _indices(case, topk, seed=6, dup=True, bad=True):
    rng = np.random.default_rng(seed)
    idx = np.zeros((case["B"], topk), np.int32)
    for b, L in enumerate(case["seq_lens"]):
        if L == 0:
            idx[b] = -1
            continue
        idx[b] = rng.integers(0, L, topk)
        if dup:
            idx[b, 1] = idx[b, 0]
        if bad:
            idx[b, 2] = -1
            idx[b, 3] = L + 5
    return idx


@pytest.mark.parametrize("topk,kw", [(16, {}), (100, {}), (7, dict(fmt=synth.KV_FP8_PAGE_HEAD, D=128)),
                                     (33, dict(lens=(0, 8, 200)))])
def test_sparse_matches_library_on_gathered_rows(topk, kw):
    case = _case(**kw)
    idx = _indices(case, topk)
    case.update(topk=topk, indices=idx)

    def rows(b, L):
        r = idx[b]
        return r[(r >= 0) & (r < L)]
    _close(case, oracle.decode(case), library(case, rows_fn=rows))


def test_sparse_listing_every_position_is_dense():
    case = _case(lens=(37, 64, 129))
    L = case["seq_lens"]
    topk = int(L.max())
    idx = np.full((case["B"], topk), -1, np.int32)
    for b in range(case["B"]):
        idx[b, :L[b]] = np.arange(L[b])
    a = oracle.decode(case)
    s = oracle.decode(dict(case, topk=topk, indices=idx))
    np.testing.assert_allclose(s[0], a[0], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(s[1], a[1], rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------------------------ splits

@pytest.mark.parametrize("variant", ["window", "sparse", "sinks"])
def test_variants_split_merge_equals_whole(variant):
    case = _case(lens=(3, 130, 257))
    if variant == "window":
        case["window"] = 50
        items = plan.fixed_items(case["seq_lens"], 3)
    elif variant == "sparse":
        topk = 90
        case.update(topk=topk, indices=_indices(case, topk))
        items = plan.fixed_items([topk] * case["B"], 4)
    else:
        case["sinks"] = np.linspace(-2, 3, case["Hkv"] * case["G"]).astype(np.float32)
        items = plan.fixed_items(case["seq_lens"], 3)
    out1, lse1, _ = oracle.split_decode(case, items)
    out0, lse0 = oracle.decode(case)
    np.testing.assert_allclose(out1, out0, rtol=1e-12, atol=1e-13)
    fin = np.isfinite(lse0)
    np.testing.assert_allclose(lse1[fin], lse0[fin], rtol=1e-13, atol=1e-12)
