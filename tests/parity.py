"""Comparison rules between the HIP path and the fp64 oracle.

Selections (integer results decided by floating-point scores): where the gap
between the m-th and (m+1)-th best oracle scores exceeds 1e-3 relative, the
GPU's set must equal the oracle's exactly; inside that band every block
clearly above the cut must be kept, none clearly below it may be, and the
count must be m.  Order (ascending) and -1 padding are checked bit-exactly.

Attention outputs: max-abs error <= 2e-2 for bf16 inputs, 1e-4 for float32,
against the oracle run on the GPU's own selection (so a legitimate choice
inside a tie band cannot fail the attention check).
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle.qsa_oracle as O

TIE_REL = 1e-3
OUT_ATOL = {"bf16": 2e-2, "f32": 1e-4}
LSE_ATOL = {"bf16": 2e-3, "f32": 1e-4}


def check_selection_row(gpu_row, scores, top_k):
    """gpu_row: int array [top_k]; scores: oracle fp64 scores of the n
    candidates.  Returns (ok, in_tie_band, message)."""
    n = len(scores)
    m = min(top_k, n)
    g = np.asarray(gpu_row, dtype=np.int64)
    if g.shape != (top_k,):
        return False, False, f"row has shape {g.shape}, expected ({top_k},)"
    head, tail = g[:m], g[m:]
    if np.any(tail != -1):
        return False, False, f"padding not -1: {tail.tolist()}"
    if m > 1 and np.any(np.diff(head) <= 0):
        return False, False, f"not strictly ascending: {head.tolist()}"
    if m and (head.min() < 0 or head.max() >= n):
        return False, False, f"ids out of [0,{n}): {head.tolist()}"
    want = O.select_blocks(scores, top_k)
    if m == n:
        return bool(np.array_equal(head, want)), False, "all candidates must be kept"
    srt = np.sort(scores)[::-1]
    sk, sk1 = srt[m - 1], srt[m]
    scale = max(abs(sk), abs(sk1))
    rel = (sk - sk1) / scale if scale > 0 else 0.0
    if rel > TIE_REL:
        ok = np.array_equal(head, want)
        return bool(ok), False, "" if ok else f"set differs outside tie band: {head.tolist()} vs {want.tolist()}"
    tau = TIE_REL * scale
    chosen = set(head.tolist())
    must = set(np.nonzero(scores > sk + tau)[0].tolist())
    banned = set(np.nonzero(scores < sk - tau)[0].tolist())
    ok = must <= chosen and not (banned & chosen)
    return bool(ok), True, "" if ok else "tie-band rule violated"


def check_selection(gpu_sel, iq, cmp, kv_len, block, top_k, rows=None):
    """Check rows of one sequence.  gpu_sel [n_q, top_k]; iq [n_q, Hi, di]
    float64; cmp oracle float64 compressed keys.  Returns (fails, n_tie)."""
    n_q = gpu_sel.shape[0]
    rows = range(n_q) if rows is None else rows
    fails, ties = [], 0
    for i in rows:
        p = kv_len - n_q + i
        n = O.candidate_blocks(p, block)
        s = O.block_scores(iq[i], cmp, n)
        ok, tie, msg = check_selection_row(gpu_sel[i], s, top_k)
        ties += int(tie)
        if not ok:
            fails.append(f"row {i} (p={p}): {msg}")
    return fails, ties


def max_abs(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def stratified_rows(T, block, top_k, total, seed):
    """Query rows for attention parity at full size: rows 0 .. 2*block-1 (short token sets,
    the first block ends), every block-end row ((p+1) % block == 0) in the last 8 blocks,
    the last two rows, then seeded rows drawn uniformly from the rows with a full selection
    (n(p) >= top_k, so |T(p)| >= top_k*block) until there are ``total`` rows."""
    rows = set(range(min(T, 2 * block)))
    rows |= {p for p in range(max(0, T - 8 * block), T) if (p + 1) % block == 0}
    rows |= {p for p in (T - 1, T - 2) if p >= 0}
    lo = min(max(top_k * block - 1, 0), T - 1)
    pool = np.setdiff1d(np.arange(lo, T), np.fromiter(rows, dtype=np.int64))
    need = max(0, min(total - len(rows), len(pool)))
    rows |= set(np.random.default_rng(seed).choice(pool, size=need, replace=False).tolist())
    return sorted(rows)


def attend_rows_threaded(q, k, v, sel, positions, rows, block, sm_scale, threads=8):
    """oracle.attend_rows over ``rows``, split across threads (NumPy releases the GIL in the
    gathers and products; BLAS is held to one thread per call).  Same results as one call."""
    from threadpoolctl import threadpool_limits
    rows = list(rows)
    if not rows:
        return O.attend_rows(q, k, v, sel, positions, rows, block, sm_scale)
    parts = [rows[i::threads] for i in range(threads) if rows[i::threads]]
    with threadpool_limits(limits=1), ThreadPoolExecutor(len(parts)) as ex:
        res = list(ex.map(lambda r: O.attend_rows(q, k, v, sel, positions, r, block, sm_scale),
                          parts))
    out = np.zeros((len(rows),) + res[0][0].shape[1:], dtype=np.float64)
    lse = np.zeros((len(rows),) + res[0][1].shape[1:], dtype=np.float64)
    for i, (o, l) in enumerate(res):
        out[i::threads] = o
        lse[i::threads] = l
    return out, lse
