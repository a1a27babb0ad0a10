"""Work-partition definitions the plan kernel must reproduce bit for bit (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

A request b of length L_b has n_b = ceil(L_b / T) tiles of T = 64 tokens.  The
plan splits every request into chunks (token ranges); each chunk produces one
partial result that the combine step merges.  Two partition rules:

* fixed split count s (FlashAttention tiling page, section 5.3 "Split 在 block.h
  中的实现": per = ceil(n / s), split i covers [i*per, min((i+1)*per, n)) blocks;
  trailing splits may be empty).  Part p is item p, chunk ids b*s + i.

* balanced parts (FlashMLA walk-through, section 调度: a small kernel hands every
  compute unit a roughly equal share of (request, KV-block range) work before the
  main kernel starts).  Reading taken here: the requests' tiles are laid end to end
  (request b owns global tiles [S_b, S_b + n_b), S the exclusive prefix sum of n);
  part p owns global tiles [e_p, e_{p+1}) with e_p = floor(p * N / num_parts), N = sum n.
  Every non-empty intersection of a part with a request is one item (chunk); items
  are numbered in (request, part) order, so a request's chunks are consecutive.

Request spans: request b's tiles cover keys [T * first_b, len_b) with len_b = L_b
(topk index slots for sparse decode) and first_b = floor(max(0, L_b - q_len - W + 1) / T)
under a sliding window W (XQA article, section "分页 KV: 页号怎么变成 TMA 坐标": pages
before the window are skipped), else 0.  The rules above apply to n_b = ceil(len_b / T)
- first_b tiles, offset by first_b.

Plan buffer (int32 words), shared contract with the library:
  [0] magic 0x50414450  [1] mode (0 fixed, 1 balanced)  [2] B  [3] num_parts
  [4] num_items  [5] T  [6] max_items  [7] 0
  part_begin[num_parts + 1] | chunk_off[B + 1] | items[max_items][4] = (b, tok0, tok1, flags)
  | counters[B * n_rowgroups] (all zero: finished-chunk counters of the fused combine)
  flags bit 0: the request has exactly one chunk (its item writes the final output).
"""
from __future__ import annotations

import numpy as np

TILE = 64
MAGIC = 0x50414450
HEADER_WORDS = 8


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def span(L: int, q_len: int = 1, window: int = 0, topk: int = 0, tile: int = TILE):
    """(len, first tile) of a request of length L."""
    if topk > 0:
        return topk, 0
    first = max(0, L - q_len - window + 1) // tile if window > 0 else 0
    return L, first


def fixed_items(seq_lens, num_splits: int, tile: int = TILE, q_len: int = 1, window: int = 0,
                topk: int = 0):
    """Items (b, tok0, tok1) of the fixed-split rule, b-major, split-minor."""
    items = []
    for b, L0 in enumerate(int(x) for x in seq_lens):
        L, f = span(L0, q_len, window, topk, tile)
        n = ceil_div(L, tile) - f
        per = ceil_div(n, num_splits)
        for i in range(num_splits):
            lo = f + i * per
            hi = f + min((i + 1) * per, n)
            t0 = min(lo * tile, L)
            t1 = min(hi * tile, L)
            if t1 < t0:
                t1 = t0
            items.append((b, t0, t1))
    return items


def balanced_items(seq_lens, num_parts: int, tile: int = TILE, q_len: int = 1, window: int = 0,
                   topk: int = 0):
    """Items (p, b, tok0, tok1) of the balanced rule, in (request, part) order."""
    spans = [span(int(L), q_len, window, topk, tile) for L in seq_lens]
    n = [ceil_div(L, tile) - f for (L, f) in spans]
    S = np.concatenate([[0], np.cumsum(n)]).astype(np.int64)
    N = int(S[-1])
    e = [(p * N) // num_parts for p in range(num_parts + 1)]
    items = []
    for b, (L, f) in enumerate(spans):
        if n[b] == 0:
            continue
        for p in range(num_parts):
            lo = max(e[p], int(S[b]))
            hi = min(e[p + 1], int(S[b]) + n[b])
            if lo >= hi:
                continue
            lt0, lt1 = f + lo - int(S[b]), f + hi - int(S[b])
            items.append((p, b, lt0 * tile, min(lt1 * tile, L)))
    return items


def max_items(B: int, num_splits: int, num_parts: int) -> int:
    return B * num_splits if num_splits > 0 else num_parts + B


def plan_words(seq_lens, num_splits: int, num_parts: int, tile: int = TILE,
               n_rowgroups: int = 0, q_len: int = 1, window: int = 0, topk: int = 0) -> np.ndarray:
    """The full plan buffer (int32) the plan kernel must write, for either rule.

    num_splits > 0 selects the fixed rule (num_parts is then B * num_splits);
    num_splits == 0 selects the balanced rule with ``num_parts`` parts.
    n_rowgroups: counter words per request appended after the items (zero).
    """
    B = len(seq_lens)
    if num_splits > 0:
        its = fixed_items(seq_lens, num_splits, tile, q_len, window, topk)
        P = B * num_splits
        flat = [(i, b, t0, t1) for i, (b, t0, t1) in enumerate(its)]
        mode = 0
    else:
        flat = balanced_items(seq_lens, num_parts, tile, q_len, window, topk)
        P = num_parts
        mode = 1
    mi = max_items(B, num_splits, P)
    nitems = len(flat)
    part_begin = np.zeros(P + 1, np.int64)
    for (p, _b, _t0, _t1) in flat:
        part_begin[p + 1] += 1
    part_begin = np.cumsum(part_begin)
    per_req = np.zeros(B, np.int64)
    for (_p, b, _t0, _t1) in flat:
        per_req[b] += 1
    chunk_off = np.concatenate([[0], np.cumsum(per_req)])
    words = np.zeros(HEADER_WORDS + (P + 1) + (B + 1) + 4 * mi + B * n_rowgroups, np.int64)
    words[0:8] = [MAGIC, mode, B, P, nitems, tile, mi, 0]
    o = HEADER_WORDS
    words[o:o + P + 1] = part_begin
    o += P + 1
    words[o:o + B + 1] = chunk_off
    o += B + 1
    for k, (_p, b, t0, t1) in enumerate(flat):
        single = 1 if per_req[b] == 1 else 0
        words[o + 4 * k:o + 4 * k + 4] = [b, t0, t1, single]
    return words.astype(np.int32)


def valid_words(words: np.ndarray) -> int:
    """Number of leading words that are defined (header + arrays + used items)."""
    P, B, nitems = int(words[3]), int(words[2]), int(words[4])
    return HEADER_WORDS + (P + 1) + (B + 1) + 4 * nitems


def counters_slice(words: np.ndarray, n_rowgroups: int) -> slice:
    """Position of the fused-combine counter words in a plan buffer."""
    P, B, mi = int(words[3]), int(words[2]), int(words[6])
    o = HEADER_WORDS + (P + 1) + (B + 1) + 4 * mi
    return slice(o, o + B * n_rowgroups)


def items_of(words: np.ndarray):
    """Decode (b, tok0, tok1, flags) items from a plan buffer."""
    P, B, nitems = int(words[3]), int(words[2]), int(words[4])
    o = HEADER_WORDS + (P + 1) + (B + 1)
    return [tuple(int(x) for x in words[o + 4 * k:o + 4 * k + 4]) for k in range(nitems)]
