"""GPU tests of the fused combine (PA_FLAG_FUSED_COMBINE) and of graph replay.

With the flag, pa_decode_run merges the chunks itself (the last workgroup to finish a
request's chunks merges them, XQA article, section "归约怎么记"), and
pa_decode_combine does nothing (bf16 and fp8 page-head formats; the MLA format with one
query token and no sparse indices).  The merge arithmetic is the combine kernel's, so the
fused result must be bit-identical to run + separate combine, and within the parity bar
of the oracle.  The counters the fused path uses live in the plan and must be back at
zero after every run, so that one plan serves any number of runs.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import plan as oplan
from mqa_split_kv_amd import binding as pb
from mqa_split_kv_amd import synth

from gpu_util import DecodeRun, assert_parity, bf16_bits_to_f64, to_device, workload, workload_ref
from test_gpu_decode import _case, _mla_case

pytestmark = pytest.mark.gpu

FUSED_CASES = [
    dict(splits=2),
    dict(splits=3, lens=(1, 15, 16, 17)),
    dict(splits=8, lens=(31, 32, 33, 300)),
    dict(Hq=32, Hkv=8, D=128, P=16, lens=(2000, 33, 4097), splits=0),
    dict(Hq=16, Hkv=1, D=128, P=32, lens=(5111, 512, 13), splits=0),
    dict(layout="NHD", Hq=16, Hkv=2, D=128, P=16, lens=(1290, 7, 640), splits=0),
    dict(fmt=synth.KV_FP8_PAGE_HEAD, Hq=32, Hkv=8, D=128, P=16, lens=(3000, 17, 1025)),
    dict(fmt=synth.KV_FP8_PAGE_HEAD, Hq=8, Hkv=2, D=64, P=32, lens=(64, 65, 2), splits=2),
    dict(lens=(0, 50, 0), splits=0),
    dict(lens=(0, 5000, 0, 0), splits=0),
    dict(lens=(0, 50, 0), splits=4),
]


def _rowgroups(case):
    return -(-case["G"] // 64) if case["kv_format"] == synth.KV_MLA656 else case["Hkv"]


def _check_counters_zero(run):
    words = run.plan_words()
    cs = oplan.counters_slice(words, _rowgroups(run.case))
    assert cs.stop == words.size
    assert np.all(words[cs] == 0), "fused-combine counters not returned to zero"


@pytest.mark.parametrize("kw", FUSED_CASES)
def test_fused_equals_separate_and_oracle(kw):
    case = _case(**kw)
    o_sep, l_sep = DecodeRun(case)()
    run = DecodeRun(case, fused=True)
    o_fu, l_fu = run()
    assert np.array_equal(o_fu, o_sep) and np.array_equal(l_fu, l_sep)
    ref_out, ref_lse = oracle.decode(case)
    assert_parity(case, o_fu, l_fu, ref_out, ref_lse)
    _check_counters_zero(run)


def test_fused_repeated_runs_one_plan():
    case = _case(Hq=32, Hkv=8, D=128, P=16, lens=(3000, 17, 900, 4096, 0, 65))
    run = DecodeRun(case, fused=True)
    o1, l1 = run()
    for _ in range(3):
        run.step()
        torch.cuda.synchronize()
        o2, l2 = bf16_bits_to_f64(run.out), run.lse.cpu().numpy().astype(np.float64)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
        _check_counters_zero(run)


@pytest.mark.parametrize("kw", [dict(Hq=32, Hkv=8, D=128, P=16, lens=(3000, 17, 900, 4096, 0, 65)),
                                dict(Hq=32, Hkv=4, D=64, P=256, lens=(1536,) * 8, splits=8)])
def test_fused_changing_inputs_one_workspace(kw):
    """Runs on one plan and workspace with different q and KV each time: the merging
    workgroup must see this launch's partials, never an earlier launch's."""
    cases = [_case(seed=s, **kw) for s in (21, 22, 23)]
    run = DecodeRun(cases[0], fused=True)
    run.plan()
    for c in cases + cases[:1]:
        run.dev = to_device(c)
        run.step()
        torch.cuda.synchronize()
        o, l = bf16_bits_to_f64(run.out), run.lse.cpu().numpy().astype(np.float64)
        ref_out, ref_lse = oracle.decode(c)
        assert_parity(c, o, l, ref_out, ref_lse)
        _check_counters_zero(run)


@pytest.mark.parametrize("kw", [dict(lens=(300, 1, 64)),
                                dict(lens=(1000, 33), splits=3),
                                dict(lens=(129, 2000), G=64, P=16),
                                dict(lens=(0, 700, 0), G=32, P=128),
                                dict(lens=(0, 700, 0), G=32, P=128, splits=4),
                                dict(lens=(5000, 3), G=16, splits=256)])
def test_fused_mla_equals_separate_and_oracle(kw):
    case = _mla_case(**kw)
    o_sep, l_sep = DecodeRun(case)()
    run = DecodeRun(case, fused=True)
    o_fu, l_fu = run()
    assert np.array_equal(o_fu, o_sep) and np.array_equal(l_fu, l_sep)
    ref_out, ref_lse = oracle.decode(case)
    assert_parity(case, o_fu, l_fu, ref_out, ref_lse)
    _check_counters_zero(run)


def test_fused_mla_config():
    case = workload(4)
    o_sep, l_sep = DecodeRun(case)()
    run = DecodeRun(case, fused=True)
    o_fu, l_fu = run()
    assert np.array_equal(o_fu, o_sep) and np.array_equal(l_fu, l_sep)
    ref_out, ref_lse = workload_ref(4)
    assert_parity(case, o_fu, l_fu, ref_out, ref_lse)
    _check_counters_zero(run)


def test_fused_ragged_fp8_config():
    case = workload(3)
    run = DecodeRun(case, fused=True)
    out, lse = run()
    ref_out, ref_lse = workload_ref(3)
    assert_parity(case, out, lse, ref_out, ref_lse)
    _check_counters_zero(run)


@pytest.mark.parametrize("B", [1, 8])
def test_fused_hd64_config(B):
    case = workload(2, B=B)
    out, lse = DecodeRun(case, fused=True)()
    ref_out, ref_lse = workload_ref(2, B=B)
    assert_parity(case, out, lse, ref_out, ref_lse)


# ---------------------------------------------------------------------------- graph replay

@pytest.mark.parametrize("fused,which", [(False, "hd64"), (True, "hd64"), (False, "ragged"),
                                         (True, "ragged"), (False, "mla"), (True, "mla")])
def test_graph_replay_matches_eager(fused, which):
    """Capture one step (run + combine) in a graph; every replay, with eager work and
    synchronisation in between, must reproduce the eager result bit for bit."""
    if which == "hd64":
        case = synth.config_case(2, B=8)
    elif which == "mla":
        case = _mla_case(lens=(1000, 0, 33, 2100), splits=0)
    else:
        case = _case(Hq=32, Hkv=8, D=128, P=16, lens=(3000, 17, 900, 4096, 0, 65))
    run = DecodeRun(case, fused=fused)
    o_ref, l_ref = run()                     # eager: plan + step
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run.step()                           # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run.step()
    for k in range(4):
        run.out.fill_(float("nan"))          # eager work between replays
        run.lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o, l = bf16_bits_to_f64(run.out), run.lse.cpu().numpy().astype(np.float64)
        assert np.array_equal(o, o_ref) and np.array_equal(l, l_ref), f"replay {k} differs"
    if fused:
        _check_counters_zero(run)
