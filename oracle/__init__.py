"""Decode-attention oracle: plain, slow, fp64 CPU definition of paged GQA/MQA decode
attention, its split partials and their merge.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code
with the HIP library in ``mqa_split_kv_amd`` and imports nothing from it; the two
meet only through the seeded input generator ``mqa_split_kv_amd.synth`` (random
draws, bf16 rounding and fp8 packing, no attention arithmetic).

The arithmetic lives in ``oracle.c`` (compiled with gcc, loaded through ctypes);
each function there cites the passage of the pages it follows.  ``plan.py`` holds
the work-partition definitions the plan kernel must reproduce bit for bit.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# ORACLE_LIB selects another build of oracle.c (build(sanitize=True): ASan + UBSan, for the
# pins run under the sanitizers)
_LIB_PATH = os.environ.get("ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_SAN_LIB_PATH = os.path.join(_HERE, "liboracle_san.so")

KV_BF16, KV_FP8_PAGE_HEAD, KV_MLA656 = 0, 1, 2


class _Desc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("G", ctypes.c_int32),
        ("D", ctypes.c_int32), ("Dv", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32),
        ("max_pages", ctypes.c_int32),
        ("s_page", ctypes.c_int64), ("s_head", ctypes.c_int64), ("s_tok", ctypes.c_int64),
        ("kv_format", ctypes.c_int32), ("q_len", ctypes.c_int32),
        ("window", ctypes.c_int32), ("topk", ctypes.c_int32),
    ]


def build(force: bool = True, sanitize: bool = False) -> str:
    """Compile oracle.c into liboracle.so (gcc, -O2, no fast-math, no FP contraction), or
    with sanitize=True into liboracle_san.so (AddressSanitizer + UndefinedBehaviorSanitizer,
    aborting on the first report; load it with the sanitizer runtimes preloaded)."""
    out = _SAN_LIB_PATH if sanitize else _LIB_PATH
    if force or not os.path.exists(out):
        tmp = out + ".tmp%d" % os.getpid()
        flags = ["-O2"] if not sanitize else ["-O1", "-g", "-fsanitize=address,undefined",
                                              "-fno-sanitize-recover=undefined",
                                              "-fno-omit-frame-pointer"]
        subprocess.check_call(["gcc"] + flags + [
            "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
            "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, out)
    return out


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(_LIB_PATH)
        vp = ctypes.c_void_p
        L.oracle_decode.argtypes = [ctypes.POINTER(_Desc), vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                    ctypes.c_double, vp, vp, vp, ctypes.c_int]
        L.oracle_decode.restype = ctypes.c_int
        L.oracle_ranges.argtypes = [ctypes.POINTER(_Desc), vp, vp, vp, vp, vp, vp, vp, vp,
                                    ctypes.c_double, ctypes.c_int, vp, vp, vp, vp, vp, vp,
                                    ctypes.c_int]
        L.oracle_ranges.restype = ctypes.c_int
        L.oracle_merge.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp]
        L.oracle_merge.restype = None
        L.oracle_e4m3_decode_n.argtypes = [vp, vp, ctypes.c_int64]
        L.oracle_e4m3_encode_n.argtypes = [vp, vp, ctypes.c_int64]
        L.oracle_kv_append.argtypes = [ctypes.POINTER(_Desc), ctypes.c_int, vp, vp, vp, vp, vp,
                                       vp, vp, vp]
        L.oracle_kv_append.restype = ctypes.c_int
        L.oracle_bf16_decode_n.argtypes = [vp, vp, ctypes.c_int64]
        L.oracle_mla656_unpack_n.argtypes = [vp, vp, ctypes.c_int64]
        L.oracle_threads.argtypes = [ctypes.c_int]
        L.oracle_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype=None):
    if a is None:
        return None
    a = np.asarray(a)
    if dtype is not None and a.dtype != dtype:
        a = a.astype(dtype)
    return np.ascontiguousarray(a)


def _desc(case) -> _Desc:
    return _Desc(case["B"], case["Hkv"], case["G"], case["D"], case["Dv"], case["page_size"],
                 case["num_pages"], case["max_pages"], case["s_page"], case["s_head"],
                 case["s_tok"], case["kv_format"], case.get("q_len", 1), case.get("window", 0),
                 case.get("topk", 0))


def _arrays(case):
    q = _c(case["q"], np.uint16)
    k = np.ascontiguousarray(case["k_pool"])
    v = None if case.get("v_pool") is None else np.ascontiguousarray(case["v_pool"])
    ks = _c(case.get("k_scale"), np.float32)
    vs = _c(case.get("v_scale"), np.float32)
    bt = _c(case["block_table"], np.int32)
    return q, k, v, ks, vs, bt


def threads(n: int = 0) -> int:
    """Set (n > 0) and return the OpenMP thread count the oracle runs on."""
    return lib().oracle_threads(n)


def _rows_shape(case):
    """Leading output shape: (B, Hq) for one query token, (B, q_len, Hq) for several."""
    nq = case.get("q_len", 1)
    Hq = case["Hkv"] * case["G"]
    return (case["B"], Hq) if nq == 1 else (case["B"], nq, Hq)


def decode(case, scale=None, pairs=None, nthreads: int = 0):
    """Plain definition for every (b, h) pair (or the boolean mask ``pairs`` [B, Hkv]).

    Optional case keys: ``window`` (sliding window), ``sinks`` ([Hq] float32 sink
    logits), ``topk`` and ``indices`` ([B, topk] int32 key positions, sparse).
    Returns (out [B, Hq, Dv] float64, lse [B, Hq] float64) - with q_len > 1 query
    tokens per request, out [B, q_len, Hq, Dv] and lse [B, q_len, Hq]; rows of skipped
    pairs are NaN.
    """
    B, Hkv, G, Dv = case["B"], case["Hkv"], case["G"], case["Dv"]
    q, k, v, ks, vs, bt = _arrays(case)
    sl = _c(case["seq_lens"], np.int32)
    sc = float(case["scale"] if scale is None else scale)
    mask = None if pairs is None else _c(np.asarray(pairs, dtype=bool).reshape(B, Hkv), np.uint8)
    out = np.full(_rows_shape(case) + (Dv,), np.nan)
    lse = np.full(_rows_shape(case), np.nan)
    d = _desc(case)
    idx = _c(case.get("indices"), np.int32)
    sinks = _c(case.get("sinks"), np.float32)
    rc = lib().oracle_decode(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(ks), _ptr(vs),
                             _ptr(bt), _ptr(sl), _ptr(idx), _ptr(sinks), sc, _ptr(mask), _ptr(out),
                             _ptr(lse), nthreads)
    if rc != 0:
        raise MemoryError("oracle_decode failed")
    return out, lse


def ranges(case, rb, rt0, rt1, scale=None, nthreads: int = 0):
    """Partial triples (m, l, Ot) of the XQA multi-block merge for token ranges.

    rb, rt0, rt1: request index and [begin, end) token range of each range (sparse:
    range of index slots).  Sinks are not part of partials.
    Returns m, l [n, Hkv, G] and Ot [n, Hkv, G, Dv] (unnormalised), float64; with
    q_len > 1 query tokens, [n, q_len, Hkv, G] and [n, q_len, Hkv, G, Dv].
    """
    Hkv, G, Dv = case["Hkv"], case["G"], case["Dv"]
    nq = case.get("q_len", 1)
    q, k, v, ks, vs, bt = _arrays(case)
    sl = _c(case["seq_lens"], np.int32)
    rb, rt0, rt1 = _c(rb, np.int32), _c(rt0, np.int32), _c(rt1, np.int32)
    n = int(rb.shape[0])
    lead = (n, Hkv, G) if nq == 1 else (n, nq, Hkv, G)
    m = np.zeros(lead)
    l = np.zeros(lead)
    Ot = np.zeros(lead + (Dv,))
    sc = float(case["scale"] if scale is None else scale)
    d = _desc(case)
    idx = _c(case.get("indices"), np.int32)
    rc = lib().oracle_ranges(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(ks), _ptr(vs),
                             _ptr(bt), _ptr(sl), _ptr(idx), sc, n, _ptr(rb), _ptr(rt0), _ptr(rt1),
                             _ptr(m), _ptr(l), _ptr(Ot), nthreads)
    if rc != 0:
        raise MemoryError("oracle_ranges failed")
    return m, l, Ot


def merge(m, l, Ot):
    """XQA merge of n partial triples.  m, l: [n, *rows]; Ot: [n, *rows, Dv].

    Returns (O [*rows, Dv], lse [*rows]).
    """
    m = _c(m, np.float64)
    l = _c(l, np.float64)
    Ot = _c(Ot, np.float64)
    n = m.shape[0]
    rows_shape = m.shape[1:]
    rows = int(np.prod(rows_shape)) if rows_shape else 1
    Dv = Ot.shape[-1]
    O = np.zeros(rows_shape + (Dv,))
    lse = np.zeros(rows_shape)
    lib().oracle_merge(n, rows, Dv, _ptr(m), _ptr(l), _ptr(Ot), _ptr(O), _ptr(lse))
    return O, lse


def split_decode(case, items, scale=None, nthreads: int = 0):
    """Split-KV evaluation: partial triples per (request, token range) item, merged per
    request with the XQA formula.  ``items`` is a list of (b, t0, t1).

    Returns (out, lse) shaped like ``decode``'s and the per-item partials (m, l, Ot).
    """
    B, Dv = case["B"], case["Dv"]
    rb = np.array([it[0] for it in items], np.int32)
    rt0 = np.array([it[1] for it in items], np.int32)
    rt1 = np.array([it[2] for it in items], np.int32)
    m, l, Ot = ranges(case, rb, rt0, rt1, scale=scale, nthreads=nthreads)
    rows = _rows_shape(case)[1:]
    out = np.zeros((B,) + rows + (Dv,))
    lse = np.full((B,) + rows, -np.inf)
    sinks = case.get("sinks")
    for b in range(B):
        sel = np.nonzero(rb == b)[0]
        mb, lb, ob = m[sel], l[sel], Ot[sel]
        if sinks is not None:
            # the sink joins the merge once per request, as a partial (sink, 1, 0)
            srow = np.broadcast_to(np.asarray(sinks, np.float64).reshape(
                (1,) * (mb.ndim - 2) + (case["Hkv"], case["G"])), (1,) + mb.shape[1:])
            mb = np.concatenate([mb, srow])
            lb = np.concatenate([lb, np.ones((1,) + lb.shape[1:])])
            ob = np.concatenate([ob, np.zeros((1,) + ob.shape[1:])])
        if mb.shape[0] == 0:
            continue
        O, ls = merge(mb, lb, ob)
        out[b] = O.reshape(rows + (Dv,))
        lse[b] = ls.reshape(rows)
    return out, lse, (m, l, Ot)


def kv_append(case, n_new: int, k_new, v_new=None) -> dict:
    """KV append reference: returns a copy of ``case`` whose pools (and fp8 scale tables)
    hold the n_new new tokens per request, written at positions seq_lens[b] - n_new + j
    (seq_lens are the lengths after the append).  k_new, v_new: [B, n_new, Hkv, D] bf16
    bits (MLA: k_new [B, n_new, 576], v_new None).  See oracle.c for the procedure."""
    out = dict(case)
    out["k_pool"] = np.array(case["k_pool"], copy=True)
    out["v_pool"] = None if case.get("v_pool") is None else np.array(case["v_pool"], copy=True)
    for key in ("k_scale", "v_scale"):
        out[key] = None if case.get(key) is None else np.array(case[key], dtype=np.float32, copy=True)
    kn = _c(k_new, np.uint16)
    vn = _c(v_new, np.uint16)
    bt = _c(case["block_table"], np.int32)
    sl = _c(case["seq_lens"], np.int32)
    d = _desc(case)
    rc = lib().oracle_kv_append(ctypes.byref(d), int(n_new), _ptr(kn), _ptr(vn), _ptr(bt), _ptr(sl),
                                _ptr(out["k_pool"]), _ptr(out["v_pool"]), _ptr(out["k_scale"]),
                                _ptr(out["v_scale"]))
    if rc != 0:
        raise ValueError("a request is shorter than n_new")
    return out


def e4m3_encode(x) -> np.ndarray:
    """OCP E4M3FN codes of fp32 values (round to nearest even, saturating at +-448)."""
    a = _c(x, np.float32)
    o = np.zeros(a.shape, np.uint8)
    lib().oracle_e4m3_encode_n(_ptr(a), _ptr(o), a.size)
    return o


def e4m3_decode(codes) -> np.ndarray:
    c = _c(codes, np.uint8)
    o = np.zeros(c.shape)
    lib().oracle_e4m3_decode_n(_ptr(c), _ptr(o), c.size)
    return o


def bf16_decode(bits) -> np.ndarray:
    c = _c(bits, np.uint16)
    o = np.zeros(c.shape)
    lib().oracle_bf16_decode_n(_ptr(c), _ptr(o), c.size)
    return o


def mla656_unpack(tokens) -> np.ndarray:
    """tokens: uint8 [..., 656] -> float64 [..., 576] (nope || rope)."""
    t = _c(tokens, np.uint8)
    n = t.size // 656
    o = np.zeros(t.shape[:-1] + (576,))
    lib().oracle_mla656_unpack_n(_ptr(t), _ptr(o), n)
    return o
