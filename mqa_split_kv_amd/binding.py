"""Thin ctypes binding of libpa_decode.so for PyTorch device tensors.

The functions keep the C names (``pa_decode_plan``, ``pa_decode_run``,
``pa_decode_combine``) and only marshal arguments: every step of the decode runs
in the library's HIP kernels on the caller's current stream.  If the library is
not built this module raises on first use; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
# PA_DECODE_LIB selects another build of the same library (the host-sanitizer build of
# `python -m mqa_split_kv_amd.build --sanitize`, for the CPU checks that run under ASan/UBSan)
LIB_PATH = os.environ.get("PA_DECODE_LIB") or os.path.join(HERE, "lib", "libpa_decode.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "pa_decode.h")

PA_OK, PA_ERR_INVALID, PA_ERR_UNSUPPORTED, PA_ERR_SIZE, PA_ERR_DEVICE = range(5)
PA_KV_BF16, PA_KV_FP8_E4M3_PAGE_HEAD, PA_KV_MLA656 = range(3)
PA_FLAG_FUSED_COMBINE = 1
EXPORTS = ("pa_decode_plan", "pa_decode_run", "pa_decode_combine", "pa_kv_append",
           "pa_decode_noalloc", "pa_decode_num_parts", "pa_status_string")
NOALLOC_SCRATCH_BYTES = 64 << 20


class PaDecodeDesc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("G", ctypes.c_int32),
        ("D", ctypes.c_int32), ("Dv", ctypes.c_int32), ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32),
        ("s_page", ctypes.c_int64), ("s_head", ctypes.c_int64), ("s_tok", ctypes.c_int64),
        ("q_len", ctypes.c_int32), ("num_splits", ctypes.c_int32),
        ("kv_format", ctypes.c_int32), ("flags", ctypes.c_int32),
        ("window", ctypes.c_int32), ("topk", ctypes.c_int32),
    ]


class PaDecodeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m mqa_split_kv_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, dp = ctypes.c_void_p, ctypes.POINTER(PaDecodeDesc)
        szp = ctypes.POINTER(ctypes.c_size_t)
        L.pa_decode_plan.argtypes = [dp, vp, vp, szp, szp, vp]
        L.pa_decode_run.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float,
                                    vp, vp, vp, vp]
        L.pa_decode_combine.argtypes = [dp, vp, vp, vp, vp, vp, vp]
        L.pa_decode_noalloc.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float,
                                        vp, vp, vp]
        L.pa_kv_append.argtypes = [dp, ctypes.c_int32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.pa_decode_num_parts.argtypes = [dp, ctypes.POINTER(ctypes.c_int32)]
        L.pa_status_string.argtypes = [ctypes.c_int]
        L.pa_status_string.restype = ctypes.c_char_p
        for f in ("pa_decode_plan", "pa_decode_run", "pa_decode_combine", "pa_kv_append",
                  "pa_decode_noalloc", "pa_decode_num_parts"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(s: int) -> str:
    return lib().pa_status_string(s).decode()


def make_desc(B, Hkv, G, D, Dv, page_size, num_pages, max_pages_per_seq, s_page, s_head,
              s_tok, num_splits=0, kv_format=PA_KV_BF16, q_len=1, flags=0, window=0,
              topk=0) -> PaDecodeDesc:
    return PaDecodeDesc(B, Hkv, G, D, Dv, page_size, num_pages, max_pages_per_seq, s_page,
                        s_head, s_tok, q_len, num_splits, kv_format, flags, window, topk)


def desc_from_case(case: dict, num_splits: Optional[int] = None,
                   fused: bool = False) -> PaDecodeDesc:
    """Descriptor for an instance drawn by ``mqa_split_kv_amd.synth``."""
    ns = case["num_splits"] if num_splits is None else num_splits
    return make_desc(case["B"], case["Hkv"], case["G"], case["D"], case["Dv"], case["page_size"],
                     case["num_pages"], case["max_pages"], case["s_page"], case["s_head"],
                     case["s_tok"], ns, case["kv_format"], q_len=case.get("q_len", 1),
                     flags=PA_FLAG_FUSED_COMBINE if fused else 0, window=case.get("window", 0),
                     topk=case.get("topk", 0))


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(fn, st):
    if st != PA_OK:
        raise PaDecodeError(fn, st)


def pa_decode_plan(desc: PaDecodeDesc, seq_lens=None, plan=None, stream=None):
    """Size query (plan None) or plan launch.  Returns (plan_bytes, workspace_bytes)."""
    pb = ctypes.c_size_t(0 if plan is None else plan.numel() * plan.element_size())
    wb = ctypes.c_size_t(0)
    st = lib().pa_decode_plan(ctypes.byref(desc), _p(seq_lens), _p(plan), ctypes.byref(pb),
                              ctypes.byref(wb), _stream(stream) if plan is not None else None)
    _check("pa_decode_plan", st)
    return pb.value, wb.value


def pa_decode_run(desc: PaDecodeDesc, plan, q, k_pool, v_pool, k_scale, v_scale, block_table,
                  seq_lens, scale: float, out, lse, workspace, stream=None, indices=None,
                  sinks=None):
    st = lib().pa_decode_run(ctypes.byref(desc), _p(plan), _p(q), _p(k_pool), _p(v_pool),
                             _p(k_scale), _p(v_scale), _p(block_table), _p(seq_lens),
                             _p(indices), _p(sinks), ctypes.c_float(scale), _p(out), _p(lse),
                             _p(workspace), _stream(stream))
    _check("pa_decode_run", st)


def pa_decode_combine(desc: PaDecodeDesc, plan, workspace, out, lse, stream=None, sinks=None):
    st = lib().pa_decode_combine(ctypes.byref(desc), _p(plan), _p(workspace), _p(sinks), _p(out),
                                 _p(lse), _stream(stream))
    _check("pa_decode_combine", st)


def pa_decode_noalloc(desc: PaDecodeDesc, q, k_pool, v_pool, k_scale, v_scale, block_table,
                      seq_lens, scale: float, out, lse, stream=None, indices=None, sinks=None):
    """Plan + decode + combine with the library's own device buffer (no allocation)."""
    st = lib().pa_decode_noalloc(ctypes.byref(desc), _p(q), _p(k_pool), _p(v_pool), _p(k_scale),
                                 _p(v_scale), _p(block_table), _p(seq_lens), _p(indices),
                                 _p(sinks), ctypes.c_float(scale), _p(out), _p(lse),
                                 _stream(stream))
    _check("pa_decode_noalloc", st)


def pa_kv_append(desc: PaDecodeDesc, n_new: int, k_new, v_new, block_table, seq_lens, k_pool,
                 v_pool, k_scale=None, v_scale=None, stream=None):
    st = lib().pa_kv_append(ctypes.byref(desc), int(n_new), _p(k_new), _p(v_new), _p(block_table),
                            _p(seq_lens), _p(k_pool), _p(v_pool), _p(k_scale), _p(v_scale),
                            _stream(stream))
    _check("pa_kv_append", st)


def pa_decode_num_parts(desc: PaDecodeDesc) -> int:
    n = ctypes.c_int32(0)
    _check("pa_decode_num_parts", lib().pa_decode_num_parts(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


class PagedDecode:
    """Owns the plan and workspace tensors for one descriptor (torch allocates them)."""

    def __init__(self, desc: PaDecodeDesc, device="cuda"):
        import torch
        self.desc = desc
        pb, wb = pa_decode_plan(desc)
        self.plan_t = torch.empty((pb + 3) // 4, dtype=torch.int32, device=device)
        self.ws = torch.empty(max(wb, 16) // 4 + 4, dtype=torch.float32, device=device)

    def plan(self, seq_lens, stream=None):
        pa_decode_plan(self.desc, seq_lens, self.plan_t, stream)

    def run(self, q, k_pool, v_pool, block_table, seq_lens, out, lse, k_scale=None,
            v_scale=None, scale: float = 0.0, stream=None, indices=None, sinks=None):
        pa_decode_run(self.desc, self.plan_t, q, k_pool, v_pool, k_scale, v_scale, block_table,
                      seq_lens, scale, out, lse, self.ws, stream, indices=indices, sinks=sinks)

    def combine(self, out, lse, stream=None, sinks=None):
        pa_decode_combine(self.desc, self.plan_t, self.ws, out, lse, stream, sinks=sinks)

    def __call__(self, *args, **kw):
        self.run(*args, **kw)
        self.combine(kw["out"] if "out" in kw else args[5], kw["lse"] if "lse" in kw else args[6],
                     kw.get("stream"), sinks=kw.get("sinks"))


def default_scale(D: int) -> float:
    return 1.0 / math.sqrt(D)
