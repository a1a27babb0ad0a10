"""GPU invariance tests (the decode reads pages only through the block table, so where a
page sits in the pool cannot change a single bit of the result; XQA article, section
"分页 KV: 页号怎么变成地址"), and a long graph replay.

* page-table permutation: the same logical KV moved to other physical pages (pool rows
  and per-page scales permuted, block table remapped) gives bit-identical out and lse,
  for bf16 (HND and NHD strides), fp8 page-head and MLA-656, dense and sparse;
* page-size repacking: the same tokens stored with another page size (other pages,
  garbage elsewhere) give bit-identical out and lse (bf16 HND / NHD, HD64, MLA-656);
* graph replay x100: one captured step (run + combine) replayed 100 times, with eager
  work between replays, reproduces the eager result bit for bit every time.
"""
import numpy as np
import pytest
import torch

from mqa_split_kv_amd import synth

from gpu_util import DecodeRun, bf16_bits_to_f64
from test_gpu_decode import _case, _mla_case
from test_oracle_variants import _indices

pytestmark = pytest.mark.gpu


def _permute_pages(case, seed=99):
    """The same logical cache at other physical pages: page p moves to perm[p]."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(case["num_pages"]).astype(np.int32)
    out = dict(case)
    for key in ("k_pool", "v_pool", "k_scale", "v_scale"):
        a = case[key]
        if a is None:
            continue
        moved = np.empty_like(a)
        moved[perm] = a
        out[key] = moved
    out["block_table"] = perm[case["block_table"]]
    return out


PERM_CASES = [
    ("bf16", dict(Hq=32, Hkv=8, D=128, P=16, lens=(2000, 33, 4097), splits=0)),
    ("bf16 NHD", dict(layout="NHD", Hq=16, Hkv=2, D=128, P=16, lens=(129, 7, 640), splits=3)),
    ("fp8", dict(fmt=synth.KV_FP8_PAGE_HEAD, Hq=32, Hkv=8, D=128, P=16, lens=(300, 17, 1025))),
    ("hd64", dict(Hq=32, Hkv=4, D=64, P=256, lens=(1536, 700), splits=8)),
]


@pytest.mark.parametrize("name,kw", PERM_CASES, ids=[c[0] for c in PERM_CASES])
def test_page_permutation_bit_identical(name, kw):
    case = _case(pool_extra=9, **kw)
    o1, l1 = DecodeRun(case)()
    o2, l2 = DecodeRun(_permute_pages(case))()
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("sparse", [False, True])
def test_mla_page_permutation_bit_identical(sparse):
    case = _mla_case((1000, 33, 300), G=64, P=64, pool_extra=7)
    if sparse:
        case.update(topk=100, indices=_indices(case, 100))
    o1, l1 = DecodeRun(case)()
    o2, l2 = DecodeRun(_permute_pages(case))()
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


REPACK_CASES = [
    ("bf16 16->64", dict(Hq=32, Hkv=8, D=128, P=16, lens=(2000, 33, 4097), splits=0), 64),
    ("bf16 NHD 64->16", dict(layout="NHD", Hq=16, Hkv=2, D=64, P=64, lens=(129, 7, 640), splits=3), 16),
    ("hd64 256->32", dict(Hq=32, Hkv=4, D=64, P=256, lens=(1536, 700), splits=8), 32),
]


@pytest.mark.parametrize("name,kw,P_new", REPACK_CASES, ids=[c[0] for c in REPACK_CASES])
def test_page_size_repacking_bit_identical(name, kw, P_new):
    """The same tokens stored with another page size give bit-identical out and lse: the
    kernels' arithmetic follows token positions, pages only locate the bytes."""
    from repack import repack
    case = _case(**kw)
    o1, l1 = DecodeRun(case)()
    o2, l2 = DecodeRun(repack(case, P_new, seed=3))()
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("P,P_new", [(64, 16), (16, 256)])
def test_mla_page_size_repacking_bit_identical(P, P_new):
    from repack import repack
    case = _mla_case((1000, 33, 300), G=64, P=P)
    o1, l1 = DecodeRun(case)()
    o2, l2 = DecodeRun(repack(case, P_new, seed=4))()
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("fused", [False, True])
def test_graph_replay_100(fused):
    case = synth.config_case(2, B=8)
    run = DecodeRun(case, fused=fused)
    o_ref, l_ref = run()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run.step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run.step()
    for k in range(100):
        if k % 10 == 0:
            run.out.fill_(float("nan"))      # eager work between replays
            run.lse.fill_(float("nan"))
            torch.cuda.synchronize()
        g.replay()
        if k % 10 == 9:
            torch.cuda.synchronize()
            o, l = bf16_bits_to_f64(run.out), run.lse.cpu().numpy().astype(np.float64)
            assert np.array_equal(o, o_ref) and np.array_equal(l, l_ref), f"replay {k} differs"
