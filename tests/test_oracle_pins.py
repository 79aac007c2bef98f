"""The oracle against facts outside itself (CPU only), and planted-mistake
checks showing those pins would catch a slip in the oracle."""
import numpy as np
import pytest

import oracle.qsa_oracle as O
import oracle_pins as P


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pinned(check):
    fails = check(O)
    assert not fails, "\n".join(fails[:10])


def _all_failures():
    out = []
    for c in P.ALL_CHECKS:
        out += c(O)
    return out


# Planted slips: each replaces one oracle function with a plausible wrong
# version (on the CPU, in this process only) and requires the pins to notice.
def _mut_candidates_off_by_one(p, block):
    return p // block


def _mut_tie_higher_index(scores, top_k):
    s = np.asarray(scores, dtype=np.float64)
    n = s.shape[0]
    order = np.lexsort((-np.arange(n), -s))
    return np.sort(order[:min(top_k, n)])


def _mut_trailing_keeps_own_block(p, block):
    return np.arange((p // block) * block, p + 1)


def _mut_scores_mean_heads(iq_p, cmp, n):
    iq_p = np.asarray(iq_p, dtype=np.float64)
    return np.asarray(cmp, dtype=np.float64)[:n] @ iq_p.mean(axis=0)


def _mut_scores_first_head(iq_p, cmp, n):
    return np.asarray(cmp, dtype=np.float64)[:n] @ np.asarray(iq_p, dtype=np.float64)[0]


def _mut_compress_sum(ik, block, kv_len=None):
    ik = np.asarray(ik, dtype=np.float64)
    L = ik.shape[0] if kv_len is None else kv_len
    return np.stack([ik[j * block:(j + 1) * block].sum(0) for j in range(L // block)]) \
        if L // block else np.zeros((0, ik.shape[1]))


def _mut_compress_includes_tail(ik, block, kv_len=None):
    ik = np.asarray(ik, dtype=np.float64)
    L = ik.shape[0] if kv_len is None else kv_len
    nb = -(-L // block)
    return np.stack([ik[j * block:min((j + 1) * block, L)].mean(0) for j in range(nb)]) \
        if nb else np.zeros((0, ik.shape[1]))


def _mut_select_lowest(scores, top_k):
    s = np.asarray(scores, dtype=np.float64)
    n = s.shape[0]
    order = np.lexsort((np.arange(n), s))
    return np.sort(order[:min(top_k, n)])


def _make_attend_mutant(kind):
    real = O.attend

    def attend(q_p, k, v, tokens, sm_scale):
        if kind == "no_scale":
            return real(q_p, k, v, tokens, 1.0)
        if kind == "gqa_mod":
            q_p = np.asarray(q_p)
            hq, hkv = q_p.shape[0], k.shape[1]
            # head h reads kv head h % hkv instead of h // G
            perm = [(h % hkv) * (hq // hkv) + h // hkv for h in range(hq)]
            out, lse = real(q_p[perm], k, v, tokens, sm_scale)
            inv = np.argsort(perm)
            return out[inv], lse[inv]
        if kind == "drop_last_token":
            return real(q_p, k, v, np.asarray(tokens)[:-1] if len(tokens) > 1 else tokens, sm_scale)
        if kind == "v_is_k":
            return real(q_p, k, k, tokens, sm_scale)
        raise ValueError(kind)
    return attend


MUTANTS = {
    "n(p)=floor(p/B)": ("candidate_blocks", _mut_candidates_off_by_one),
    "ties->higher index": ("select_blocks", _mut_tie_higher_index),
    "trailing keeps own block": ("trailing_tokens", _mut_trailing_keeps_own_block),
    "mean over heads": ("block_scores", _mut_scores_mean_heads),
    "first head only": ("block_scores", _mut_scores_first_head),
    "compress sums": ("compress_keys", _mut_compress_sum),
    "compress includes tail": ("compress_keys", _mut_compress_includes_tail),
    "selects lowest": ("select_blocks", _mut_select_lowest),
    "no softmax scale": ("attend", _make_attend_mutant("no_scale")),
    "gqa h % Hkv": ("attend", _make_attend_mutant("gqa_mod")),
    "drops a token": ("attend", _make_attend_mutant("drop_last_token")),
    "V replaced by K": ("attend", _make_attend_mutant("v_is_k")),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    fails = []
    for c in P.ALL_CHECKS:
        try:
            fails += c(O)
        except Exception as exc:  # a crash also counts as caught
            fails.append(f"{c.__name__} raised {exc!r}")
        if fails:
            break
    assert fails, f"planted mistake '{name}' passed every pin"
