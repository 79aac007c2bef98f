"""Plain fp64 CPU oracle for Qwen Sparse Attention (QSA).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path (no kernels, headers, helpers or constants) and imports nothing from it.

Source of the method: the Hugging Face Transformers model page "Qwen4-Exp".
  * Overview, QSA paragraph: several indexer query heads score *compressed key
    blocks*, each query keeps the most relevant contiguous token blocks, and
    the incomplete trailing block is kept uncompressed.
  * ``Qwen4ExpTextConfig`` parameters ``indexer_n_heads`` (query heads of the
    token indexer), ``indexer_kv_heads`` (exactly one indexer key head),
    ``indexer_head_dim`` (dim of every indexer query/key head),
    ``indexer_budget`` (max tokens taken from complete compressed blocks per
    query) and ``indexer_compress_ratio`` (consecutive token keys averaged into
    one index block).
  * Usage tips: QSA enables sparse token selection on full-attention layers,
    run as eager/SDPA softmax attention.

Where the page is silent the oracle takes these readings (each is repeated at
the function that applies it):
  R1 compression = arithmetic mean of each *complete* block of B indexer keys;
     the incomplete tail is never compressed.
  R2 block score = plain sum over indexer heads of the dot product between the
     head's query and the compressed key (no scale, activation or weights).
  R3 block j is a candidate for query position p iff it is complete at p,
     i.e. (j+1)*B <= p+1, so n(p) = floor((p+1)/B) candidates.
  R4 m = min(k, n(p)) blocks are kept, k = budget / B; ranking is by score
     descending, ties broken by the lower block index (-0 == +0).
  R5 trailing tokens = [B*n(p), p]; empty when (p+1) % B == 0 (then p's own
     block is an ordinary candidate).
  R6 one selection per query token, shared by all attention heads; attention
     is causal softmax with scale sm_scale over the selected tokens; grouped
     query attention maps query head h to key/value head h // (Hq / Hkv).
  R7 query i of a call with n_q queries over kv_len keys sits at position
     p = kv_len - n_q + i (prefill: n_q == kv_len, decode: n_q == 1).

Every function works on one sequence with exact float64 copies of its inputs
(bf16 -> float64 is exact).  Parity unpinned: only the relation of these
readings to the real model's code, which the page does not print.
"""
from __future__ import annotations

import numpy as np


# --------------------------------------------------------------------------
# step a1: key-block compression
# --------------------------------------------------------------------------
def num_complete_blocks(length: int, block: int) -> int:
    """Number of complete blocks of ``block`` consecutive tokens among the
    first ``length`` tokens (reading R1; ``indexer_compress_ratio``)."""
    return length // block


def compress_keys(ik, block: int, kv_len: int | None = None) -> np.ndarray:
    """Mean of every complete block of ``block`` consecutive indexer keys.

    Qwen4-Exp page, ``Qwen4ExpTextConfig`` / ``indexer_compress_ratio``: that
    many consecutive token keys are averaged into one index block; overview:
    the incomplete trailing block stays uncompressed (reading R1).

    ik: [L, di] indexer keys of one sequence (one key head, ``indexer_kv_heads``
    = 1).  Only the first ``kv_len`` rows count (default: all).
    Returns [floor(kv_len / block), di] float64.
    """
    ik = np.asarray(ik, dtype=np.float64)
    length = ik.shape[0] if kv_len is None else int(kv_len)
    nb = num_complete_blocks(length, block)
    out = np.zeros((nb, ik.shape[1]), dtype=np.float64)
    for j in range(nb):
        out[j] = ik[j * block:(j + 1) * block].mean(axis=0)
    return out


# --------------------------------------------------------------------------
# steps a2 + a3: indexer scores and top-k block selection
# --------------------------------------------------------------------------
def candidate_blocks(p: int, block: int) -> int:
    """n(p): complete blocks visible to query position p (reading R3).

    A block is a candidate only once all of its tokens are at or before p,
    which is what 'complete compressed blocks' (``indexer_budget``) allows.
    """
    return (p + 1) // block


def block_scores(iq_p, cmp, n: int) -> np.ndarray:
    """Indexer score of each candidate block j < n for one query token.

    Qwen4-Exp overview: multiple (indexer) query heads score the compressed
    key blocks.  Reading R2: the score is the sum over indexer heads of
    <iq_p[h], cmp[j]>; computed head by head and then summed.

    iq_p: [Hi, di] indexer queries of the token; cmp: [>= n, di].
    """
    iq_p = np.asarray(iq_p, dtype=np.float64)
    cmp = np.asarray(cmp, dtype=np.float64)
    scores = np.zeros(n, dtype=np.float64)
    for h in range(iq_p.shape[0]):
        scores = scores + cmp[:n] @ iq_p[h]
    return scores


def select_blocks(scores, top_k: int) -> np.ndarray:
    """Keep the min(top_k, n) best blocks, returned in ascending block order.

    Qwen4-Exp overview ('selects the most relevant contiguous token blocks')
    and ``indexer_budget`` (a maximum, so fewer when fewer blocks exist).
    Reading R4: higher score first, then lower block index; numpy's stable
    lexsort does the ranking (-0.0 and +0.0 compare equal).
    """
    scores = np.asarray(scores, dtype=np.float64)
    n = scores.shape[0]
    m = min(int(top_k), n)
    order = np.lexsort((np.arange(n), -scores))
    return np.sort(order[:m]).astype(np.int64)


def trailing_tokens(p: int, block: int) -> np.ndarray:
    """Uncompressed trailing tokens of query position p (reading R5):
    positions B*n(p) .. p, empty when p closes a block."""
    return np.arange(candidate_blocks(p, block) * block, p + 1, dtype=np.int64)


def token_set(sel, p: int, block: int) -> np.ndarray:
    """T(p): tokens of the selected blocks plus the trailing tokens, sorted.

    Qwen4-Exp overview: attention runs over the selected contiguous token
    blocks and the incomplete trailing block (reading R5).
    """
    parts = [np.arange(int(j) * block, (int(j) + 1) * block, dtype=np.int64) for j in sel]
    parts.append(trailing_tokens(p, block))
    return np.unique(np.concatenate(parts))


def index_topk(iq, cmp, kv_len: int, block: int, top_k: int):
    """Selections of the n_q queries of one sequence (reading R7 positions).

    iq: [n_q, Hi, di]; cmp: [>= floor(kv_len/block), di].
    Returns (sel [n_q, top_k] int64 ascending, -1 padded;
             sel_scores [n_q, top_k] float64, -inf padded;
             positions [n_q]).
    """
    iq = np.asarray(iq, dtype=np.float64)
    n_q = iq.shape[0]
    sel = np.full((n_q, top_k), -1, dtype=np.int64)
    sel_scores = np.full((n_q, top_k), -np.inf, dtype=np.float64)
    positions = np.arange(kv_len - n_q, kv_len, dtype=np.int64)
    for i in range(n_q):
        p = int(positions[i])
        n = candidate_blocks(p, block)
        s = block_scores(iq[i], cmp, n)
        chosen = select_blocks(s, top_k)
        sel[i, :len(chosen)] = chosen
        sel_scores[i, :len(chosen)] = s[chosen]
    return sel, sel_scores, positions


# --------------------------------------------------------------------------
# steps a4 + a5: attention over the selected tokens
# --------------------------------------------------------------------------
def attend(q_p, k, v, tokens, sm_scale: float):
    """Softmax attention of one query token over the given token positions.

    Qwen4-Exp usage tips: sparse token selection feeds ordinary (eager/SDPA)
    softmax attention; ``num_attention_heads`` / ``num_key_value_heads``
    give grouped query attention (reading R6, head h reads KV head h // G).

    q_p: [Hq, D]; k, v: [>= max(tokens)+1, Hkv, D]; tokens: 1-D positions.
    Returns (out [Hq, Dv], lse [Hq]) in float64 (Dv = value dim, normally D),
    lse = natural log-sum-exp of the scaled logits.
    """
    q_p = np.asarray(q_p, dtype=np.float64)
    tokens = np.asarray(tokens, dtype=np.int64)
    hq = q_p.shape[0]
    hkv = k.shape[1]
    group = hq // hkv
    out = np.zeros((hq, v.shape[2]), dtype=np.float64)
    lse = np.zeros(hq, dtype=np.float64)
    for h in range(hq):
        g = h // group
        kt = np.asarray(k[tokens, g], dtype=np.float64)
        vt = np.asarray(v[tokens, g], dtype=np.float64)
        logits = sm_scale * (kt @ q_p[h])
        mx = logits.max()
        w = np.exp(logits - mx)
        den = w.sum()
        out[h] = (w / den) @ vt
        lse[h] = mx + np.log(den)
    return out, lse


def attend_rows(q, k, v, sel, positions, rows, block: int, sm_scale: float):
    """attend() for selected query rows with a *given* selection (lets a test
    score the GPU's own selection).  q: [n_q, Hq, D]; sel: [n_q, top_k] with
    -1 padding; positions: [n_q]; rows: iterable of query indices."""
    rows = list(rows)
    hq, dv = q.shape[1], v.shape[2]
    out = np.zeros((len(rows), hq, dv), dtype=np.float64)
    lse = np.zeros((len(rows), hq), dtype=np.float64)
    for r, i in enumerate(rows):
        chosen = [int(j) for j in sel[i] if j >= 0]
        toks = token_set(chosen, int(positions[i]), block)
        out[r], lse[r] = attend(q[i], k, v, toks, sm_scale)
    return out, lse


# --------------------------------------------------------------------------
# whole path, one sequence
# --------------------------------------------------------------------------
def prefill(q, k, v, iq, ik, block: int, top_k: int, sm_scale: float, rows=None):
    """QSA over a whole prompt of T tokens (n_q == kv_len == T).

    q: [T, Hq, D]; k, v: [T, Hkv, D]; iq: [T, Hi, di]; ik: [T, di].
    ``rows`` limits attention to those query indices (selection is always
    computed for every row).  Returns a dict with cmp, sel, sel_scores,
    positions, rows, out [len(rows), Hq, D], lse [len(rows), Hq].
    """
    t = q.shape[0]
    rows = range(t) if rows is None else rows
    cmp = compress_keys(ik, block, t)
    sel, sel_scores, positions = index_topk(iq, cmp, t, block, top_k)
    out, lse = attend_rows(q, k, v, sel, positions, rows, block, sm_scale)
    return dict(cmp=cmp, sel=sel, sel_scores=sel_scores, positions=positions,
                rows=list(rows), out=out, lse=lse)


def decode(q, k_cache, v_cache, kv_len: int, iq, cmp, block: int, top_k: int, sm_scale: float):
    """One new query token of a sequence whose cache already holds kv_len
    keys, the new token's own key/value at position kv_len - 1 (reading R7).

    q: [Hq, D]; caches: [>= kv_len, Hkv, D]; iq: [Hi, di]; cmp: compressed
    indexer keys of the cached prefix (the indexer state kept on device).
    Returns dict(sel [top_k], sel_scores [top_k], out [Hq, D], lse [Hq]).
    """
    sel, sel_scores, positions = index_topk(np.asarray(iq)[None], cmp, kv_len, block, top_k)
    chosen = [int(j) for j in sel[0] if j >= 0]
    toks = token_set(chosen, int(positions[0]), block)
    out, lse = attend(q, k_cache, v_cache, toks, sm_scale)
    return dict(sel=sel[0], sel_scores=sel_scores[0], out=out, lse=lse)
