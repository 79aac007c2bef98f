"""Seeded synthetic inputs for QSA workloads (shared by tests, bench and smoke).

Holds no part of the method's arithmetic: only random draws, bf16 rounding and
the workload table.  Every tensor is drawn from NumPy's PCG64 seeded with
SeedSequence([workload_seed, tensor_id, seq_id]) as float32 standard normals,
then (for bf16 workloads) rounded to bfloat16 with round-to-nearest-even on the
bit pattern.  Tensor ids: q=0, k=1, v=2, iq=3, ik=4, mu=5, plant=6, lens=7.

Structure of the workloads:
  * "query mean" workloads draw one vector mu ~ N(0, I) and use
    iq = mu + N(0, 1) for every token and indexer head, so indexer queries
    share a direction;
  * "planted" blocks get indexer keys 0.5 * qbar + N(0, 1), qbar = the mean of
    the generated (rounded) indexer queries over tokens and heads, so those
    blocks score high and selection is not trivial;
  * decode workloads draw per-sequence context lengths (tensor id 7) and fill
    the first kv_len rows of each cache; rows past kv_len stay zero.
"""
from __future__ import annotations

import concurrent.futures as cf
from collections import deque
from dataclasses import dataclass, field, replace

import numpy as np

T_Q, T_K, T_V, T_IQ, T_IK, T_MU, T_PLANT, T_LENS = range(8)


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    kind: str                 # "prefill" | "decode" | "varlen" (prefill of mixed lengths)
    dtype: str                # "bf16" | "f32"
    batch: int
    block: int
    top_k: int
    h_q: int
    h_kv: int
    d: int
    h_idx: int
    d_idx: int
    seq: int = 0              # prefill prompt length
    max_len: int = 0          # decode cache rows (varlen: K/V rows per sequence)
    len_lo: int = 0           # decode context (varlen: prompt) lengths, inclusive range
    len_hi: int = 0
    query_mean: bool = False
    plant_frac: float = 0.0   # fraction of complete blocks planted (seeded choice)
    plant_every: int = 0      # or plant blocks j % plant_every == 0
    n_q: int = 0              # chunked prefill: the queries are the last n_q tokens (0 = all)
    note: str = field(default="", compare=False)

    @property
    def sm_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny_prefill_f32": Workload(
        "tiny_prefill_f32", 1, "prefill", "f32", batch=1, seq=250, block=16, top_k=4,
        h_q=4, h_kv=1, d=64, h_idx=2, d_idx=32,
        note="seq 250 = 15 complete blocks + 10 trailing tokens; all N(0,1)"),
    "prefill_bf16_4k": Workload(
        "prefill_bf16_4k", 2, "prefill", "bf16", batch=1, seq=4133, block=64, top_k=16,
        h_q=16, h_kv=2, d=128, h_idx=8, d_idx=64, query_mean=True, plant_frac=0.05,
        note="64 complete blocks + 37 trailing; 3 planted blocks"),
    "decode_bf16_b64": Workload(
        "decode_bf16_b64", 3, "decode", "bf16", batch=64, max_len=32768, len_lo=8192,
        len_hi=32768, block=64, top_k=32, h_q=32, h_kv=4, d=128, h_idx=8, d_idx=64,
        note="context lengths uniform in [8192, 32768]; all N(0,1)"),
    "long_prefill_bf16_128k": Workload(
        "long_prefill_bf16_128k", 4, "prefill", "bf16", batch=1, seq=131072 + 77, block=128,
        top_k=64, h_q=32, h_kv=4, d=128, h_idx=16, d_idx=64, query_mean=True, plant_every=32,
        note="1024 complete blocks + 77 trailing; blocks j % 32 == 0 planted (every 4096 tokens)"),
    "chunk_prefill_bf16_128k": Workload(
        "chunk_prefill_bf16_128k", 4, "prefill", "bf16", batch=1, seq=131072 + 77, block=128,
        top_k=64, h_q=32, h_kv=4, d=128, h_idx=16, d_idx=64, query_mean=True, plant_every=32,
        n_q=4096, note="the last 4096 tokens of the 128k prompt (same inputs) as one chunk "
                       "over the whole sequence"),
    "long_decode_bf16_b128": Workload(
        "long_decode_bf16_b128", 5, "decode", "bf16", batch=128, max_len=131072,
        len_lo=131072, len_hi=131072, block=128, top_k=64, h_q=32, h_kv=4, d=128, h_idx=16,
        d_idx=64, note="context 131072 each (1024 blocks, empty trailing part)"),
    # the model page's default attention shape: 16 query heads over 2 KV heads of dim 256
    "prefill_bf16_d256_32k": Workload(
        "prefill_bf16_d256_32k", 6, "prefill", "bf16", batch=1, seq=32768 + 45, block=128,
        top_k=32, h_q=16, h_kv=2, d=256, h_idx=8, d_idx=64, query_mean=True, plant_every=16,
        note="head dim 256, 16/2 heads; 256 complete blocks + 45 trailing"),
    # a batch of prompts of mixed length, left-padded to the longest (varlen prefill)
    "varlen_prefill_bf16_b8": Workload(
        "varlen_prefill_bf16_b8", 8, "varlen", "bf16", batch=8, max_len=16384, len_lo=1024,
        len_hi=16384, block=64, top_k=16, h_q=16, h_kv=2, d=128, h_idx=8, d_idx=64,
        query_mean=True, plant_frac=0.05,
        note="8 prompts, lengths uniform in [1024, 16384]; queries right-aligned to the longest"),
    "decode_bf16_d256_b64": Workload(
        "decode_bf16_d256_b64", 7, "decode", "bf16", batch=64, max_len=32768, len_lo=8192,
        len_hi=32768, block=64, top_k=32, h_q=16, h_kv=2, d=256, h_idx=8, d_idx=64,
        note="head dim 256, 16/2 heads; context lengths uniform in [8192, 32768]"),
}


# ---------------------------------------------------------------------------
def rng(seed: int, tensor_id: int, seq_id: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor_id, seq_id])))


def normal_f32(seed: int, tensor_id: int, seq_id: int, shape) -> np.ndarray:
    return rng(seed, tensor_id, seq_id).standard_normal(shape, dtype=np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def store(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 draws -> storage array (uint16 bf16 bits or float32)."""
    return bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def to_f64(a: np.ndarray) -> np.ndarray:
    """Storage array -> exact float64 values."""
    if a.dtype == np.uint16:
        return bf16_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def to_torch(a: np.ndarray, device=None):
    """Storage array -> torch tensor (bf16 bits become torch.bfloat16)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.to(device) if device is not None else t


# ---------------------------------------------------------------------------
def _indexer_queries(w: Workload, seq_id: int, n: int) -> np.ndarray:
    x = normal_f32(w.seed, T_IQ, seq_id, (n, w.h_idx, w.d_idx))
    if w.query_mean:
        x = x + normal_f32(w.seed, T_MU, 0, (w.d_idx,))[None, None, :]
    return store(x, w.dtype)


def planted_blocks(w: Workload, n_complete: int) -> np.ndarray:
    if w.plant_every:
        return np.arange(0, n_complete, w.plant_every, dtype=np.int64)
    if w.plant_frac > 0 and n_complete > 0:
        cnt = int(round(w.plant_frac * n_complete))
        return np.sort(rng(w.seed, T_PLANT, 0).choice(n_complete, size=cnt, replace=False))
    return np.zeros(0, dtype=np.int64)


def _indexer_keys(w: Workload, seq_id: int, n: int, iq_store: np.ndarray) -> np.ndarray:
    x = normal_f32(w.seed, T_IK, seq_id, (n, w.d_idx))
    planted = planted_blocks(w, n // w.block)
    if len(planted):
        qbar = to_f64(iq_store).reshape(-1, w.d_idx).mean(axis=0).astype(np.float32)
        for j in planted:
            x[j * w.block:(j + 1) * w.block] += np.float32(0.5) * qbar
    return store(x, w.dtype)


def prefill_inputs(w: Workload, seq_id: int = 0) -> dict:
    """One prompt: q [T,Hq,D], k/v [T,Hkv,D], iq [T,Hi,di], ik [T,di] (storage arrays)."""
    T = w.seq
    q = store(normal_f32(w.seed, T_Q, seq_id, (T, w.h_q, w.d)), w.dtype)
    k = store(normal_f32(w.seed, T_K, seq_id, (T, w.h_kv, w.d)), w.dtype)
    v = store(normal_f32(w.seed, T_V, seq_id, (T, w.h_kv, w.d)), w.dtype)
    iq = _indexer_queries(w, seq_id, T)
    ik = _indexer_keys(w, seq_id, T, iq)
    return dict(q=q, k=k, v=v, iq=iq, ik=ik)


def varlen_inputs(w: Workload, seqs=None):
    """Prompts of a varlen batch: (lens, {b: prefill_inputs of length lens[b]}) for b in
    ``seqs`` (default all); lengths are drawn as for decode (tensor id 7)."""
    lens = decode_lens(w)
    seqs = range(w.batch) if seqs is None else seqs
    return lens, {b: prefill_inputs(w.with_(seq=int(lens[b]), kind="prefill"), seq_id=b)
                  for b in seqs}


def decode_lens(w: Workload) -> np.ndarray:
    if w.len_lo == w.len_hi:
        return np.full(w.batch, w.len_lo, dtype=np.int32)
    return rng(w.seed, T_LENS, 0).integers(w.len_lo, w.len_hi, size=w.batch,
                                           endpoint=True).astype(np.int32)


def decode_sequence(w: Workload, b: int, kv_len: int) -> dict:
    """Sequence b of a decode batch: q [Hq,D], iq [Hi,di], and the first kv_len
    rows of its caches k/v [kv_len,Hkv,D] and indexer keys ik [kv_len,di]."""
    q = store(normal_f32(w.seed, T_Q, b, (w.h_q, w.d)), w.dtype)
    iq = _indexer_queries(w, b, 1)[0]
    k = store(normal_f32(w.seed, T_K, b, (kv_len, w.h_kv, w.d)), w.dtype)
    v = store(normal_f32(w.seed, T_V, b, (kv_len, w.h_kv, w.d)), w.dtype)
    ik = store(normal_f32(w.seed, T_IK, b, (kv_len, w.d_idx)), w.dtype)
    return dict(q=q, iq=iq, k=k, v=v, ik=ik)


def decode_sequences(w: Workload, lens: np.ndarray, seqs=None, threads: int = 16):
    """Yield (b, decode_sequence(w, b, lens[b])) for b in ``seqs`` (default all),
    generated on a thread pool (NumPy releases the GIL while drawing) and
    yielded in order, at most ``threads`` sequences ahead."""
    seqs = list(range(w.batch)) if seqs is None else list(seqs)
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        window = deque()
        nxt = 0
        while nxt < len(seqs) and len(window) < threads:
            window.append((seqs[nxt], ex.submit(decode_sequence, w, seqs[nxt], int(lens[seqs[nxt]]))))
            nxt += 1
        while window:
            b, fut = window.popleft()
            res = fut.result()
            if nxt < len(seqs):
                window.append((seqs[nxt], ex.submit(decode_sequence, w, seqs[nxt], int(lens[seqs[nxt]]))))
                nxt += 1
            yield b, res
