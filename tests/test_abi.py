"""C-ABI checks that need no GPU: the library loads, exports every entry point its
header declares, and rejects bad arguments with the documented status before any
HIP call (so these run on a machine without a GPU)."""
import ctypes
import re

import pytest

from mqa_split_kv_amd import binding as pb


def _declared():
    src = open(pb.HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:pa_status|const char \*)\s*(pa_\w+)\s*\(", src, re.M)))


def test_header_declares_the_documented_entry_points():
    assert set(_declared()) == set(pb.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = pb.lib()
    for name in _declared():
        assert hasattr(L, name), name


def test_status_strings():
    for s in range(5):
        assert pb.status_string(s)
    assert pb.status_string(99) == "unknown status"


def _desc(**kw):
    base = dict(B=2, Hkv=1, G=8, D=64, Dv=64, page_size=16, num_pages=40, max_pages_per_seq=17,
                s_page=16 * 64, s_head=16 * 64, s_tok=64, num_splits=1, kv_format=pb.PA_KV_BF16)
    base.update(kw)
    return pb.make_desc(**base)


def _plan_status(desc):
    pbytes = ctypes.c_size_t(0)
    wbytes = ctypes.c_size_t(0)
    return pb.lib().pa_decode_plan(ctypes.byref(desc), None, None, ctypes.byref(pbytes),
                                   ctypes.byref(wbytes), None), pbytes.value, wbytes.value


BAD = [
    (dict(B=0), pb.PA_ERR_INVALID),
    (dict(G=0), pb.PA_ERR_INVALID),
    (dict(Hkv=-1), pb.PA_ERR_INVALID),
    (dict(page_size=0), pb.PA_ERR_INVALID),
    (dict(s_tok=4), pb.PA_ERR_INVALID),          # 8-byte stride: not 16-byte aligned
    (dict(s_tok=56), pb.PA_ERR_INVALID),         # not a multiple of 16 bytes... 112 B
    (dict(num_splits=-1), pb.PA_ERR_INVALID),
    (dict(window=-1), pb.PA_ERR_INVALID),
    (dict(topk=-1), pb.PA_ERR_INVALID),
    (dict(topk=64), pb.PA_ERR_UNSUPPORTED),      # sparse decode: MLA tokens only
    (dict(kv_format=pb.PA_KV_MLA656, Hkv=1, G=16, D=576, Dv=512, s_tok=656, s_page=656 * 16,
          topk=64, window=8), pb.PA_ERR_UNSUPPORTED),
    (dict(flags=2), pb.PA_ERR_INVALID),           # undefined flag bit
    (dict(flags=-1), pb.PA_ERR_INVALID),
    (dict(kv_format=7), pb.PA_ERR_INVALID),
    (dict(D=96, Dv=96, s_tok=96, s_head=16 * 96, s_page=16 * 96), pb.PA_ERR_UNSUPPORTED),
    (dict(D=128, Dv=64), pb.PA_ERR_UNSUPPORTED),
    (dict(page_size=8), pb.PA_ERR_UNSUPPORTED),
    (dict(page_size=48), pb.PA_ERR_UNSUPPORTED),
    (dict(G=17), pb.PA_ERR_UNSUPPORTED),
    (dict(q_len=0), pb.PA_ERR_INVALID),
    (dict(q_len=65), pb.PA_ERR_UNSUPPORTED),
    (dict(G=8, q_len=33), pb.PA_ERR_UNSUPPORTED),   # more than 256 query rows per KV head
    (dict(kv_format=pb.PA_KV_MLA656, Hkv=1, G=128, D=576, Dv=512, s_tok=656, s_page=656 * 16,
          q_len=9), pb.PA_ERR_UNSUPPORTED),     # more than 1024 query rows
    (dict(B=5000), pb.PA_ERR_UNSUPPORTED),
    (dict(Hkv=512, G=16, q_len=16, num_splits=0, flags=1), pb.PA_ERR_UNSUPPORTED),  # fused: partials >= 2 GiB
    (dict(kv_format=pb.PA_KV_MLA656, Hkv=1, G=16, D=576, Dv=512, s_tok=(1 << 20) + 16,
          s_page=((1 << 20) + 16) * 16), pb.PA_ERR_UNSUPPORTED),   # MLA token stride over 2^20 B
    (dict(kv_format=pb.PA_KV_MLA656, Hkv=2, D=576, Dv=512, s_tok=656, s_page=656 * 16),
     pb.PA_ERR_UNSUPPORTED),
    (dict(kv_format=pb.PA_KV_MLA656, Hkv=1, G=16, D=576, Dv=512, s_tok=656, s_page=656 * 16,
          flags=1, q_len=2), pb.PA_ERR_UNSUPPORTED),   # MLA fused merge: one query token
    (dict(kv_format=pb.PA_KV_MLA656, Hkv=1, G=16, D=576, Dv=512, s_tok=656, s_page=656 * 16,
          flags=1, topk=64), pb.PA_ERR_UNSUPPORTED),   # ... and no sparse indices
]


@pytest.mark.parametrize("kw,status", BAD)
def test_invalid_descriptors_rejected_on_host(kw, status):
    st, _, _ = _plan_status(_desc(**kw))
    assert st == status


def test_size_query_fixed_splits_needs_no_device():
    # fixed split counts do not depend on the device, so the size query is pure host logic
    st, pbytes, wbytes = _plan_status(_desc(num_splits=2))
    assert st == pb.PA_OK
    B, s = 2, 2
    # header | part_begin | chunk_off | items | fused-combine counters (B x Hkv)
    assert pbytes == 4 * (8 + (B * s + 1) + (B + 1) + 4 * B * s + B * 1)
    o = (B * s * 1 * 8 * 64 * 4 + 255) // 256 * 256
    assert wbytes == o + B * s * 1 * 8 * 4


def test_size_query_scales_with_query_tokens():
    # partials are kept per query token: the workspace grows q_len times, the plan not
    st1, p1, w1 = _plan_status(_desc(num_splits=2))
    st3, p3, w3 = _plan_status(_desc(num_splits=2, q_len=3))
    assert st1 == st3 == pb.PA_OK and p1 == p3
    B, s, rows = 2, 2, 3 * 8
    assert w3 == (B * s * rows * 64 * 4 + 255) // 256 * 256 + B * s * rows * 4


def test_fused_flag_accepted_and_combine_is_launch_free():
    st, pbytes, _ = _plan_status(_desc(num_splits=2, flags=pb.PA_FLAG_FUSED_COMBINE))
    assert st == pb.PA_OK and pbytes > 0
    # with the flag, combine returns before touching the device (no stream, no launch)
    d = _desc(num_splits=2, flags=pb.PA_FLAG_FUSED_COMBINE)
    buf = ctypes.create_string_buffer(1 << 12)
    base = (ctypes.addressof(buf) + 255) // 256 * 256
    p = ctypes.c_void_p
    assert pb.lib().pa_decode_combine(ctypes.byref(d), p(base), p(base), None, p(base), p(base),
                                      None) == pb.PA_OK


def _run(d, base, **over):
    """pa_decode_run with every pointer valid (host memory: only host-side checks run
    before the first failing one) except the overrides."""
    p = ctypes.c_void_p
    a = dict(plan=p(base), q=p(base), k=p(base), v=p(base), ks=p(base), vs=p(base),
             bt=p(base), sl=p(base), idx=None, sinks=None, scale=ctypes.c_float(0.0),
             out=p(base), lse=p(base), ws=p(base))
    a.update(over)
    return pb.lib().pa_decode_run(ctypes.byref(d), a["plan"], a["q"], a["k"], a["v"], a["ks"],
                                  a["vs"], a["bt"], a["sl"], a["idx"], a["sinks"], a["scale"],
                                  a["out"], a["lse"], a["ws"], None)


def test_run_rejects_null_and_misaligned_pointers():
    d = _desc()
    buf = ctypes.create_string_buffer(1 << 16)
    base = (ctypes.addressof(buf) + 255) // 256 * 256
    p = ctypes.c_void_p
    assert _run(d, base, plan=None) == pb.PA_ERR_INVALID
    assert _run(d, base, q=p(base + 2)) == pb.PA_ERR_INVALID
    assert _run(d, base, scale=ctypes.c_float(float("nan"))) == pb.PA_ERR_INVALID
    assert _run(d, base, sinks=p(base + 2)) == pb.PA_ERR_INVALID
    assert _run(d, base, idx=p(base)) == pb.PA_ERR_INVALID            # indices without topk
    d8 = _desc(kv_format=pb.PA_KV_FP8_E4M3_PAGE_HEAD, s_tok=64, s_head=16 * 64, s_page=16 * 64)
    assert _run(d8, base, ks=None, vs=None) == pb.PA_ERR_INVALID
    dm = _desc(kv_format=pb.PA_KV_MLA656, Hkv=1, G=16, D=576, Dv=512, s_tok=656,
               s_page=656 * 16, topk=64)
    assert _run(dm, base, v=None) == pb.PA_ERR_INVALID                # topk without indices


def test_plan_size_check():
    L = pb.lib()
    d = _desc(num_splits=2)
    buf = ctypes.create_string_buffer(4096)
    small = ctypes.c_size_t(8)
    wb = ctypes.c_size_t(0)
    st = L.pa_decode_plan(ctypes.byref(d), ctypes.c_void_p(ctypes.addressof(buf)),
                          ctypes.c_void_p(ctypes.addressof(buf)), ctypes.byref(small),
                          ctypes.byref(wb), None)
    assert st == pb.PA_ERR_SIZE


def test_append_rejects_bad_arguments_on_host():
    L = pb.lib()
    buf = ctypes.create_string_buffer(1 << 12)
    base = (ctypes.addressof(buf) + 255) // 256 * 256
    p = ctypes.c_void_p
    d = _desc()
    args = [p(base)] * 6 + [None, None, None]
    assert L.pa_kv_append(ctypes.byref(d), 0, *args) == pb.PA_ERR_INVALID          # n_new = 0
    assert L.pa_kv_append(ctypes.byref(d), 70000, *args) == pb.PA_ERR_UNSUPPORTED
    assert L.pa_kv_append(ctypes.byref(d), 1, None, *[p(base)] * 5, None, None,
                          None) == pb.PA_ERR_INVALID                                 # no k_new
    assert L.pa_kv_append(ctypes.byref(d), 1, p(base + 8), *[p(base)] * 5, None, None,
                          None) == pb.PA_ERR_INVALID                                 # misaligned
    d8 = _desc(kv_format=pb.PA_KV_FP8_E4M3_PAGE_HEAD)
    assert L.pa_kv_append(ctypes.byref(d8), 1, *[p(base)] * 6, None, None,
                          None) == pb.PA_ERR_INVALID                                 # no scales
    dm = _desc(kv_format=pb.PA_KV_MLA656, Hkv=1, G=16, D=576, Dv=512, s_tok=656, s_page=656 * 16)
    assert L.pa_kv_append(ctypes.byref(dm), 1, *[p(base)] * 6, None, None,
                          None) == pb.PA_ERR_INVALID                                 # v_new given


def _noalloc_status(desc, ptr=0x100000):
    """pa_decode_noalloc with placeholder (never dereferenced) device addresses."""
    p = ctypes.c_void_p(ptr)
    mla = desc.kv_format == pb.PA_KV_MLA656
    return pb.lib().pa_decode_noalloc(ctypes.byref(desc), p, p, None if mla else p, None, None, p,
                                      p, None, None, ctypes.c_float(0.0), p, p, None)


def test_noalloc_rejects_more_than_its_buffer():
    # MLA, 8 draft tokens x 128 heads, 4 fixed splits of 8 requests: 32 chunk partials of
    # 1024 rows x 512 fp32 = 64 MiB, plus their lse and the plan: beyond the buffer
    desc = _desc(B=8, kv_format=pb.PA_KV_MLA656, Hkv=1, G=128, D=576, Dv=512, s_tok=656,
                 s_page=656 * 16, q_len=8, num_splits=4)
    _, pbytes, wbytes = _plan_status(desc)
    assert ((pbytes + 255) // 256 * 256) + wbytes > pb.NOALLOC_SCRATCH_BYTES
    assert _noalloc_status(desc) == pb.PA_ERR_SIZE
    # 3 splits fit (the call then needs the device: no GPU here)
    small = _desc(B=8, kv_format=pb.PA_KV_MLA656, Hkv=1, G=128, D=576, Dv=512, s_tok=656,
                  s_page=656 * 16, q_len=8, num_splits=3)
    _, pbytes, wbytes = _plan_status(small)
    assert ((pbytes + 255) // 256 * 256) + wbytes <= pb.NOALLOC_SCRATCH_BYTES


def test_noalloc_validates_arguments():
    assert _noalloc_status(_desc(B=0)) == pb.PA_ERR_INVALID
    assert _noalloc_status(_desc(), ptr=0x100008) == pb.PA_ERR_INVALID      # misaligned
    p = ctypes.c_void_p(0x100000)
    st = pb.lib().pa_decode_noalloc(ctypes.byref(_desc()), None, p, p, None, None, p, p, None,
                                    None, ctypes.c_float(0.0), p, p, None)
    assert st == pb.PA_ERR_INVALID                                            # no q
