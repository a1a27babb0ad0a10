"""Helpers for the GPU parity tests: move a synthetic instance to the device, run the
HIP path through the C ABI, and the tolerance of the parity bar."""
from __future__ import annotations

import numpy as np
import torch

from mqa_split_kv_amd import binding as pb
from mqa_split_kv_amd import synth

# Parity bar: |out_gpu - out_oracle| <= OUT_TOL * max|V| (valid tokens), |lse diff| <= LSE_TOL
OUT_TOL = 1e-2
LSE_TOL = 1e-3


_WORKLOADS: dict = {}
_WORKLOAD_REFS: dict = {}


def workload(index: int, B=None) -> dict:
    """The seeded instance of a named workload, drawn once per test session (the large
    ones take seconds to draw).  Callers must not modify it."""
    key = (index, B)
    if key not in _WORKLOADS:
        _WORKLOADS[key] = synth.config_case(index, B=B)
    return _WORKLOADS[key]


def workload_ref(index: int, B=None):
    """The oracle's (out, lse) for every row of workload(index, B), computed once."""
    key = (index, B)
    if key not in _WORKLOAD_REFS:
        import oracle
        _WORKLOAD_REFS[key] = oracle.decode(workload(index, B))
    return _WORKLOAD_REFS[key]


def to_device(case: dict, device="cuda") -> dict:
    def t(a, dt=None):
        if a is None:
            return None
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to(device)

    return dict(q=t(case["q"]), k_pool=t(case["k_pool"]),
                v_pool=t(case["v_pool"]) if case.get("v_pool") is not None else None,
                k_scale=t(case.get("k_scale")), v_scale=t(case.get("v_scale")),
                block_table=t(case["block_table"]), seq_lens=t(case["seq_lens"]),
                indices=t(case.get("indices")), sinks=t(case.get("sinks")))


def bf16_bits_to_f64(t: torch.Tensor) -> np.ndarray:
    x = t.detach().view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32) << 16
    return x.view(np.float32).astype(np.float64)


class DecodeRun:
    """Plan + decode + combine for one instance and split setting."""

    def __init__(self, case: dict, num_splits=None, dev=None, poison=True, fused=False):
        self.case = case
        self.desc = pb.desc_from_case(case, num_splits, fused=fused)
        self.dev = dev if dev is not None else to_device(case)
        B, Hq, Dv, nq = case["B"], case["Hkv"] * case["G"], case["Dv"], case.get("q_len", 1)
        lead = (B, Hq) if nq == 1 else (B, nq, Hq)
        self.runner = pb.PagedDecode(self.desc)
        self.out = torch.empty(lead + (Dv,), dtype=torch.bfloat16, device="cuda")
        self.lse = torch.empty(lead, dtype=torch.float32, device="cuda")
        if poison:
            self.out.fill_(float("nan"))
            self.lse.fill_(float("nan"))
            self.runner.ws.fill_(float("nan"))
            self.runner.plan_t.fill_(-7)

    def plan(self):
        self.runner.plan(self.dev["seq_lens"])

    def step(self, scale: float = 0.0):
        d = self.dev
        self.runner.run(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["seq_lens"],
                        self.out, self.lse, k_scale=d["k_scale"], v_scale=d["v_scale"],
                        scale=scale, indices=d.get("indices"), sinks=d.get("sinks"))
        self.runner.combine(self.out, self.lse, sinks=d.get("sinks"))

    def __call__(self, scale: float = 0.0):
        self.plan()
        self.step(scale)
        torch.cuda.synchronize()
        return bf16_bits_to_f64(self.out), self.lse.cpu().numpy().astype(np.float64)

    def plan_words(self) -> np.ndarray:
        torch.cuda.synchronize()
        return self.runner.plan_t.cpu().numpy()


def v_absmax(case: dict) -> float:
    """max |V| over the dequantised values of every valid token of the instance."""
    L = np.asarray(case["seq_lens"])
    P = case["page_size"]
    fmt = case["kv_format"]
    best = 0.0
    for b in range(case["B"]):
        n = -(-int(L[b]) // P)
        if n == 0:
            continue
        pages = case["block_table"][b, :n]
        valid = np.arange(n * P) < L[b]
        if fmt == synth.KV_MLA656:
            tok = case["k_pool"][pages].reshape(n * P, -1)[valid]
            codes = np.ascontiguousarray(tok[:, :512])
            sc = np.ascontiguousarray(tok[:, 512:528]).view(np.float32)
            x = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
            x = np.abs(x.reshape(-1, 4, 128)) * sc[:, :, None]
            best = max(best, float(x.max()))
            continue
        vp = case["v_pool"]
        if case["layout"] == "HND":
            x = vp[pages]                              # [n, Hkv, P, D]
            x = x.transpose(0, 2, 1, 3).reshape(n * P, case["Hkv"], -1)[valid]
        else:
            x = vp[pages].reshape(n * P, case["Hkv"], -1)[valid]
        if fmt == synth.KV_BF16:
            f = (x.astype(np.uint32) << 16).view(np.float32)
            best = max(best, float(np.abs(f).max()))
        else:
            f = torch.from_numpy(np.ascontiguousarray(x)).view(torch.float8_e4m3fn).float().numpy()
            sc = case["v_scale"][pages]                # [n, Hkv]
            sc = np.repeat(sc, P, axis=0)[valid]       # [tokens, Hkv]
            best = max(best, float((np.abs(f) * sc[:, :, None]).max()))
    return best


_VMAX: dict = {}


def _vmax(case: dict) -> float:
    # the session's workload instances are never modified: their max|V| is kept
    if any(case is w for w in _WORKLOADS.values()):
        if id(case) not in _VMAX:
            _VMAX[id(case)] = v_absmax(case)
        return _VMAX[id(case)]
    return v_absmax(case)


def assert_parity(case, out, lse, ref_out, ref_lse, rows=None, vmax=None):
    """Element-wise parity at the tolerance above; rows: boolean mask [B, Hq] to compare."""
    vmax = _vmax(case) if vmax is None else vmax
    if rows is None:
        rows = np.ones(lse.shape, bool)
    o, r = out[rows], ref_out[rows]
    le, lr = lse[rows], ref_lse[rows]
    assert np.all(np.isfinite(o)), "non-finite output"
    err = np.abs(o - r).max() if o.size else 0.0
    assert err <= OUT_TOL * vmax, f"out max err {err} > {OUT_TOL} * {vmax}"
    fin = np.isfinite(lr)
    assert np.array_equal(np.isneginf(le), np.isneginf(lr)), "lse -inf pattern differs"
    lerr = np.abs(le[fin] - lr[fin]).max() if fin.any() else 0.0
    assert lerr <= LSE_TOL, f"lse max err {lerr}"
    return err / max(vmax, 1e-30), lerr
