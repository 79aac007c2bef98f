"""Checks that pin the fp64 oracle to facts outside itself.

Each ``check_*`` takes the oracle module and returns a list of failure strings
(empty = pinned).  They are written so that a plausible slip anywhere in the
oracle (a dropped term, a wrong sign or index, an off-by-one in the block
arithmetic, the wrong tie rule, a transposed operand) makes at least one of
them fail; ``test_oracle_pins.py`` plants such slips and checks that.

What each check compares against:
  golden            hand-worked case in tests/golden (pencil arithmetic)
  compress          closed forms: constant blocks, linear ramps, linearity
  scores            one dot product with the head-summed query (linear algebra)
  select            brute force over every subset of the candidates
  token_set         counting identities of the token set
  dense             torch SDPA (fp64, CPU, is_causal) when top-k covers all blocks
  masked            torch SDPA with an explicit boolean mask built here
  gqa               multi-head attention on repeated key/value heads
  q_zero / one_hot  exact closed forms of softmax attention
  decode            a prefill row equals decode on the prefix
  lse               scipy logsumexp of the masked logits
"""
from __future__ import annotations

import itertools
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "qsa_handworked_b2_l7.txt")


# --------------------------------------------------------------------------
def load_golden(path: str = GOLDEN):
    g = dict(ik=[], cmp=[], iq=[], score=[], rows=[])
    for raw in open(path):
        line = raw.strip()
        if not line or line.startswith("#"):
            continue
        tok = line.split()
        if tok[0] == "block":
            g["block"] = int(tok[1])
        elif tok[0] in ("ik", "cmp", "iq"):
            g[tok[0]].append([float(x) for x in tok[2:]])
        elif tok[0] == "score":
            g["score"].append([float(x) for x in tok[2:]])
        elif tok[0] == "row":
            left, sel, toks, outp = line.split("|")
            k, p = left.split()[1], left.split()[2]
            num, den = outp.strip().split("/")
            g["rows"].append(dict(k=int(k), p=int(p[1:]),
                                  sel=[int(x) for x in sel.split()],
                                  tokens=[int(x) for x in toks.split()],
                                  out=Fraction(int(num), int(den))))
    g["ik"] = np.array(g["ik"])
    g["cmp"] = np.array(g["cmp"])
    iq = np.array(g["iq"])
    g["iq"] = iq.reshape(iq.shape[0], 2, iq.shape[1] // 2)
    return g


def _probe_qkv(length: int):
    """Q = 0, one head, D = 1, V[s] = s: output = mean of attended positions."""
    q = np.zeros((length, 1, 1))
    k = np.zeros((length, 1, 1))
    v = np.arange(length, dtype=np.float64).reshape(length, 1, 1)
    return q, k, v


def check_golden(o) -> list:
    g = load_golden()
    fails = []
    B = g["block"]
    L = g["ik"].shape[0]
    cmp = o.compress_keys(g["ik"], B)
    if cmp.shape != g["cmp"].shape or not np.array_equal(cmp, g["cmp"]):
        fails.append(f"golden cmp {cmp.tolist()} != {g['cmp'].tolist()}")
    for p in range(L):
        n = o.candidate_blocks(p, B)
        s = o.block_scores(g["iq"][p], g["cmp"], n)
        if not np.array_equal(s, np.array(g["score"][p])):
            fails.append(f"golden scores p{p}: {s.tolist()} != {g['score'][p]}")
    q, k, v = _probe_qkv(L)
    for row in g["rows"]:
        res = o.prefill(q, k, v, g["iq"], g["ik"], B, row["k"], 1.0, rows=[row["p"]])
        sel = [int(x) for x in res["sel"][row["p"]] if x >= 0]
        if sel != row["sel"]:
            fails.append(f"golden sel k={row['k']} p{row['p']}: {sel} != {row['sel']}")
        toks = o.token_set(sel, row["p"], B).tolist()
        if toks != row["tokens"]:
            fails.append(f"golden T k={row['k']} p{row['p']}: {toks} != {row['tokens']}")
        if abs(res["out"][0, 0, 0] - float(row["out"])) > 1e-12:
            fails.append(f"golden out k={row['k']} p{row['p']}: {res['out'][0,0,0]} != {row['out']}")
        if row["p"] == L - 1:
            dec = o.decode(q[L - 1], k, v, L, g["iq"][L - 1], cmp, B, row["k"], 1.0)
            dsel = [int(x) for x in dec["sel"] if x >= 0]
            if dsel != row["sel"] or abs(dec["out"][0, 0] - float(row["out"])) > 1e-12:
                fails.append(f"golden decode k={row['k']}: {dsel} {dec['out'][0,0]}")
    return fails


# --------------------------------------------------------------------------
def check_compress(o) -> list:
    fails = []
    rng = np.random.default_rng(11)
    B, nb, di = 4, 5, 3
    consts = rng.standard_normal((nb, di))
    x = np.repeat(consts, B, axis=0)
    x = np.concatenate([x, 100 + rng.standard_normal((3, di))])  # tail must not leak in
    c = o.compress_keys(x, B)
    if c.shape != (nb, di) or not np.allclose(c, consts, rtol=0, atol=1e-13):
        fails.append("compress: constant blocks do not map to their constant")
    t = np.arange(nb * B + 2, dtype=np.float64)
    ramp = np.stack([t, 2 * t - 1], axis=1)
    want = np.stack([np.arange(nb) * B + (B - 1) / 2, 2 * (np.arange(nb) * B + (B - 1) / 2) - 1], axis=1)
    if not np.allclose(o.compress_keys(ramp, B), want, rtol=0, atol=1e-12):
        fails.append("compress: linear ramp does not give block midpoints")
    X = rng.standard_normal((nb * B + 1, di))
    Y = rng.standard_normal((nb * B + 1, di))
    lhs = o.compress_keys(2.5 * X - 0.75 * Y, B)
    rhs = 2.5 * o.compress_keys(X, B) - 0.75 * o.compress_keys(Y, B)
    if not np.allclose(lhs, rhs, rtol=0, atol=1e-12):
        fails.append("compress: not linear")
    if o.compress_keys(X, B, kv_len=B * 2 + 1).shape[0] != 2:
        fails.append("compress: kv_len not respected")
    return fails


def check_scores(o) -> list:
    fails = []
    rng = np.random.default_rng(12)
    hi, di, n = 5, 7, 9
    iq = rng.standard_normal((hi, di))
    cmp = rng.standard_normal((n + 3, di))
    s = o.block_scores(iq, cmp, n)
    want = np.array([float(np.dot(iq.sum(axis=0), cmp[j])) for j in range(n)])
    if s.shape != (n,) or not np.allclose(s, want, rtol=1e-12, atol=1e-12):
        fails.append("scores: not the dot product with the head-summed query")
    one = o.block_scores(iq[:1], cmp, n)
    if not np.allclose(one, cmp[:n] @ iq[0], rtol=1e-12, atol=1e-12):
        fails.append("scores: one indexer head is not a plain dot product")
    return fails


def _brute_topm(scores, m):
    """The unique m-subset X with: x in X, y not in X => x ranks before y,
    where 'ranks before' = higher score, or equal score and lower index."""
    n = len(scores)
    found = []
    for X in itertools.combinations(range(n), m):
        Xs = set(X)
        ok = all((scores[x] > scores[y]) or (scores[x] == scores[y] and x < y)
                 for x in Xs for y in range(n) if y not in Xs)
        if ok:
            found.append(list(X))
    return found


def check_select(o) -> list:
    fails = []
    rng = np.random.default_rng(13)
    for trial in range(60):
        n = int(rng.integers(0, 8))
        s = rng.integers(-2, 3, size=n).astype(np.float64)  # many ties
        if trial % 3 == 0:
            s = np.where(s == 0, -0.0, s)                    # -0 must tie with +0
            s[: n // 2] = np.abs(s[: n // 2]) * 0.0
        for k in range(1, n + 2):
            m = min(k, n)
            want = _brute_topm(s, m)
            got = o.select_blocks(s, k).tolist()
            if len(want) != 1 or got != want[0]:
                fails.append(f"select: scores {s.tolist()} k={k}: {got} != {want}")
    return fails


def check_token_set(o) -> list:
    fails = []
    rng = np.random.default_rng(14)
    for B in (1, 2, 3, 4, 16):
        for p in range(0, 70):
            n = o.candidate_blocks(p, B)
            if n * B > p + 1 or (n + 1) * B <= p + 1:
                fails.append(f"n(p) wrong: p={p} B={B} n={n}")
                continue
            for k in (1, 2, 5):
                m = min(k, n)
                sel = np.sort(rng.choice(n, size=m, replace=False)) if n else np.zeros(0, int)
                T = o.token_set(sel, p, B)
                if len(T) != m * B + (p + 1) % B:
                    fails.append(f"|T| wrong p={p} B={B} k={k}")
                if len(T) and (T.max() > p or T.min() < 0):
                    fails.append(f"T exceeds causal range p={p} B={B}")
                trail = set(range(B * ((p + 1) // B), p + 1))
                if not trail <= set(T.tolist()):
                    fails.append(f"trailing tokens missing p={p} B={B}")
    return fails


# --------------------------------------------------------------------------
def _rand_prefill(rng, T, hq, hkv, D, hi, di):
    return (rng.standard_normal((T, hq, D)), rng.standard_normal((T, hkv, D)),
            rng.standard_normal((T, hkv, D)), rng.standard_normal((T, hi, di)),
            rng.standard_normal((T, di)))


def check_dense(o) -> list:
    import torch
    import torch.nn.functional as F
    fails = []
    rng = np.random.default_rng(15)
    T, B, hq, hkv, D = 53, 4, 6, 2, 8
    q, k, v, iq, ik = _rand_prefill(rng, T, hq, hkv, D, 3, 5)
    scale = 0.37
    res = o.prefill(q, k, v, iq, ik, B, top_k=T // B + 1, sm_scale=scale)
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(k).permute(1, 0, 2)[None]
    vt = torch.from_numpy(v).permute(1, 0, 2)[None]
    ref = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale, enable_gqa=True)
    ref = ref[0].permute(1, 0, 2).numpy()
    if not np.allclose(res["out"], ref, rtol=1e-10, atol=1e-12):
        fails.append(f"dense: k >= blocks differs from causal SDPA by {np.abs(res['out'] - ref).max()}")
    return fails


def _mask(o, sel, T, B):
    """M[p, s] = s attended by row p, written from the definition: s in a
    selected block, or s in [B*floor((p+1)/B), p]."""
    M = np.zeros((T, T), dtype=bool)
    for p in range(T):
        for j in sel[p]:
            if j >= 0:
                M[p, j * B:(j + 1) * B] = True
        M[p, B * ((p + 1) // B):p + 1] = True
    return M


def check_masked(o) -> list:
    import torch
    import torch.nn.functional as F
    fails = []
    rng = np.random.default_rng(16)
    T, B, hq, hkv, D = 45, 4, 4, 2, 8
    q, k, v, iq, ik = _rand_prefill(rng, T, hq, hkv, D, 2, 4)
    scale = 0.29
    for topk in (1, 3):
        res = o.prefill(q, k, v, iq, ik, B, topk, scale)
        M = _mask(o, res["sel"], T, B)
        qt = torch.from_numpy(q).permute(1, 0, 2)[None]
        kt = torch.from_numpy(k).permute(1, 0, 2)[None]
        vt = torch.from_numpy(v).permute(1, 0, 2)[None]
        ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(M),
                                             scale=scale, enable_gqa=True)
        ref = ref[0].permute(1, 0, 2).numpy()
        if not np.allclose(res["out"], ref, rtol=1e-10, atol=1e-12):
            fails.append(f"masked: k={topk} differs from masked SDPA by {np.abs(res['out'] - ref).max()}")
        # lse against scipy on the same mask
        from scipy.special import logsumexp
        for p in range(T):
            for h in range(hq):
                lg = scale * (k[:, h // (hq // hkv)] @ q[p, h])
                want = logsumexp(lg[M[p]])
                if abs(res["lse"][p, h] - want) > 1e-10:
                    fails.append(f"lse: k={topk} p={p} h={h}")
                    break
    return fails


def check_gqa(o) -> list:
    fails = []
    rng = np.random.default_rng(17)
    T, B, hq, hkv, D = 30, 4, 6, 3, 5
    q, k, v, iq, ik = _rand_prefill(rng, T, hq, hkv, D, 2, 3)
    G = hq // hkv
    a = o.prefill(q, k, v, iq, ik, B, 2, 0.5)
    kr = np.repeat(k, G, axis=1)
    vr = np.repeat(v, G, axis=1)
    b = o.prefill(q, kr, vr, iq, ik, B, 2, 0.5)
    if not np.allclose(a["out"], b["out"], rtol=1e-12, atol=1e-13):
        fails.append("gqa: grouped attention != MHA with repeated KV heads")
    return fails


def check_q_zero(o) -> list:
    fails = []
    rng = np.random.default_rng(18)
    T, B, D = 37, 4, 3
    q = np.zeros((T, 2, D))
    k = rng.standard_normal((T, 1, D))
    v = rng.standard_normal((T, 1, D))
    iq = rng.standard_normal((T, 2, 4))
    ik = rng.standard_normal((T, 4))
    res = o.prefill(q, k, v, iq, ik, B, 2, 1.0)
    for p in range(T):
        toks = o.token_set([j for j in res["sel"][p] if j >= 0], p, B)
        want = v[toks, 0].mean(axis=0)
        if not np.allclose(res["out"][p], want[None], rtol=0, atol=1e-13):
            fails.append(f"q=0: row {p} is not the mean of V over T(p)")
        if abs(res["lse"][p, 0] - np.log(len(toks))) > 1e-12:
            fails.append(f"q=0: lse row {p} != log|T|")
    return fails


def check_one_hot(o) -> list:
    """V[s] = e_s (D = T) reads back exactly which tokens row p attended."""
    fails = []
    rng = np.random.default_rng(19)
    T, B = 26, 3
    q = rng.standard_normal((T, 1, 4))
    k = rng.standard_normal((T, 1, 4))
    v = np.eye(T).reshape(T, 1, T)
    iq = rng.standard_normal((T, 2, 3))
    ik = rng.standard_normal((T, 3))
    for topk in (1, 2, 4):
        res = o.prefill(q, k, v, iq, ik, B, topk, 0.8)
        sel = res["sel"]
        M = _mask(o, sel, T, B)
        for p in range(T):
            support = np.nonzero(res["out"][p, 0] > 0)[0]
            if not np.array_equal(support, np.nonzero(M[p])[0]):
                fails.append(f"one-hot: row {p} attends {support.tolist()}")
            if abs(res["out"][p, 0].sum() - 1) > 1e-12:
                fails.append(f"one-hot: row {p} weights do not sum to 1")
    return fails


def check_decode(o) -> list:
    fails = []
    rng = np.random.default_rng(20)
    T, B, hq, hkv, D = 41, 4, 4, 2, 6
    q, k, v, iq, ik = _rand_prefill(rng, T, hq, hkv, D, 3, 5)
    res = o.prefill(q, k, v, iq, ik, B, 3, 0.4)
    for L in range(1, T + 1):
        cmp = o.compress_keys(ik[:L], B)
        d = o.decode(q[L - 1], k, v, L, iq[L - 1], cmp, B, 3, 0.4)
        if not np.array_equal(d["sel"], res["sel"][L - 1]) or \
                not np.allclose(d["out"], res["out"][L - 1], rtol=0, atol=1e-14):
            fails.append(f"decode at L={L} != prefill row {L - 1}")
    return fails


def check_order_free(o) -> list:
    fails = []
    rng = np.random.default_rng(21)
    T, B = 30, 4
    q, k, v, iq, ik = _rand_prefill(rng, T, 2, 1, 4, 2, 3)
    res = o.prefill(q, k, v, iq, ik, B, 3, 0.7)
    sel_rev = res["sel"][:, ::-1].copy()
    out2, _ = o.attend_rows(q, k, v, sel_rev, res["positions"], range(T), B, 0.7)
    if not np.allclose(out2, res["out"], rtol=0, atol=1e-13):
        fails.append("attention depends on the order of the selection")
    return fails


ALL_CHECKS = [check_golden, check_compress, check_scores, check_select, check_token_set,
              check_dense, check_masked, check_gqa, check_q_zero, check_one_hot,
              check_decode, check_order_free]
