"""GPU tests of pa_decode_noalloc, the entry point for callers that cannot allocate
(graph capture, serving loops): plan + decode + combine with the plan and partials in
the library's own per-device buffer.  Its results must be the bits of the three-call
sequence with caller buffers (same kernels), and within the parity bar of the oracle,
on two calls in a row where the second has a smaller input (the buffer keeps the first
call's contents), and under graph capture."""
import numpy as np
import pytest
import torch

import oracle
from mqa_split_kv_amd import binding as pb
from mqa_split_kv_amd import synth

from gpu_util import DecodeRun, assert_parity, bf16_bits_to_f64, to_device
from test_gpu_decode import _case, _mla_case

pytestmark = pytest.mark.gpu


def _noalloc(case, fused=False, scale=0.0):
    d = to_device(case)
    desc = pb.desc_from_case(case, fused=fused)
    B, Hq, Dv, nq = case["B"], case["Hkv"] * case["G"], case["Dv"], case.get("q_len", 1)
    lead = (B, Hq) if nq == 1 else (B, nq, Hq)
    out = torch.full(lead + (Dv,), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full(lead, float("nan"), dtype=torch.float32, device="cuda")

    def call():
        pb.pa_decode_noalloc(desc, d["q"], d["k_pool"], d["v_pool"], d["k_scale"], d["v_scale"],
                             d["block_table"], d["seq_lens"], scale, out, lse,
                             indices=d.get("indices"), sinks=d.get("sinks"))
    return call, out, lse


def _result(out, lse):
    torch.cuda.synchronize()
    return bf16_bits_to_f64(out), lse.cpu().numpy().astype(np.float64)


PAIRS = [
    ("bf16 balanced",
     lambda: _case(Hq=32, Hkv=8, D=128, P=16, lens=(2000, 33, 4097), splits=0),
     lambda: _case(Hq=32, Hkv=8, D=128, P=16, lens=(100, 7), splits=0, seed=2), False),
    ("fp8 fixed splits",
     lambda: _case(fmt=synth.KV_FP8_PAGE_HEAD, Hq=32, Hkv=8, D=128, P=16, lens=(3000, 17, 1025), splits=3),
     lambda: _case(fmt=synth.KV_FP8_PAGE_HEAD, Hq=32, Hkv=8, D=128, P=16, lens=(65,), splits=3, seed=3), False),
    ("hd64 fused",
     lambda: synth.config_case(2, B=8),
     lambda: synth.config_case(2, B=1), True),
    ("mla balanced",
     lambda: _mla_case((1000, 33, 300), G=64, P=64),
     lambda: _mla_case((64,), G=64, P=64, seed=12), False),
]


@pytest.mark.parametrize("name,big,small,fused", PAIRS, ids=[p[0] for p in PAIRS])
def test_noalloc_matches_three_calls_twice(name, big, small, fused):
    for make in (big, small):                 # second call: a smaller input
        case = make()
        print(f"[noalloc] {name}: B={case['B']} lens={list(case['seq_lens'])}", flush=True)
        ref_o, ref_l = DecodeRun(case, fused=fused)()
        call, out, lse = _noalloc(case, fused=fused)
        call()
        o, l = _result(out, lse)
        assert np.array_equal(o, ref_o) and np.array_equal(l, ref_l)
        want_o, want_l = oracle.decode(case)
        assert_parity(case, o, l, want_o, want_l)


def test_noalloc_graph_capture():
    """The no-allocation call captured in a graph: every replay (eager work and a
    synchronisation in between) reproduces the eager result."""
    case = _case(Hq=32, Hkv=8, D=128, P=16, lens=(3000, 17, 900, 4096, 0, 65), splits=0)
    call, out, lse = _noalloc(case)
    call()
    o_ref, l_ref = _result(out, lse)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for k in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        o, l = _result(out, lse)
        assert np.array_equal(o, o_ref) and np.array_equal(l, l_ref), f"replay {k} differs"
    want_o, want_l = oracle.decode(case)
    assert_parity(case, o_ref, l_ref, want_o, want_l)
