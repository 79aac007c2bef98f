#!/usr/bin/env python3
"""QSA throughput on one MI355X: one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--graph | --no-graph] [--no-cpu-baseline] [--no-calibration]
    python bench.py --calibrate-copy MIB
    python bench.py --calibrate-read MIB
    python bench.py --calibrate-mfma


A step is one pass of the whole QSA path over one batch of synthetic input:
  prefill workloads: key-block compression -> indexer scores + top-k selection
                     -> block-sparse attention;
  varlen workloads:  the same three steps over a batch of prompts of mixed length
                     (queries right-aligned to the longest prompt);
  decode workloads:  indexer step (completes the compressed block the newest
                     token finishes, then scores + top-k over the cached compressed
                     keys) -> block-sparse decode attention (the compressed indexer
                     state of the prefix before the newest token is computed once,
                     before timing).
Inputs are resident in HBM before the timed region starts.  ``value`` is
tokens/s of the whole step (prefill: batch*seq tokens, varlen: the prompts' tokens,
decode: batch tokens).  With ``--graph`` (the default) the steps are launched from a
HIP graph that holds ``steps_per_graph`` consecutive whole steps, replayed
K / steps_per_graph times (at least 20 replays when K allows it): every timed step runs
all of its kernels, in stream order; only the fixed cost of launching a graph is shared.
Each replay is bracketed by its own pair of events; ``ms_per_step`` is the median replay
time per step (the mean is reported beside it).

``roofline`` describes the dominant kernel (the attention kernel): algorithmic
flops (prefill, bf16 matrix cores) or algorithmic bytes (decode, HBM) per launch
divided by its median launch time, measured with events recorded on the stream the
kernels run on around each of >= 20 replays of back-to-back attention calls (enough calls
per replay for ~5 ms of kernel time, at most 16) that follow the timed steps.  ``frac`` is against the vendor peak, ``frac_of_measured`` against the
rate the calibration kernel of the same resource sustains in the same run
(``--no-calibration`` skips it).  ``traffic`` is the HBM byte count per launch from the
committed profiler counter summary of the workload (null when the attention kernel's
sources changed since it was taken); ``traffic_over_compulsory`` divides it by the bytes
the launch must move at least once (every input read once, every output written once).
``cpu_baseline`` times the fp64 oracle (single-threaded BLAS) on a bounded
sample of the same workload; ``tie_band_rows`` is the fraction of that sample's
selection rows whose m-th and (m+1)-th oracle scores lie within 1e-3 relative.

``--calibrate-copy MIB`` runs only a plain device copy of MIB MiB (one
elementwise kernel that reads and writes MIB MiB, five launches): the byte
counters of the profiler (FETCH_SIZE, WRITE_SIZE) read on it give the scale
factors that turn the counters of the attention kernels into bytes.
``--calibrate-read MIB`` / ``--calibrate-mfma`` run only the calibration kernels
(libqsa_calib.so: a streaming read of MIB MiB, a dense bf16 MFMA loop) and print their
rates, for profiler summaries of the measured peaks.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "QSA tokens/s (prefill & decode, 1 GPU); % of HBM / bf16 MFMA roofline"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E peak
DEFAULT_WORKLOAD = "long_prefill_bf16_128k"


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    g = ap.add_mutually_exclusive_group()
    g.add_argument("--graph", dest="graph", action="store_true", default=True,
                   help="replay each step's launches from HIP graphs (default)")
    g.add_argument("--no-graph", dest="graph", action="store_false")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="approximate CPU time budget of the oracle baseline")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="run only a plain device copy of MIB MiB (counter calibration)")
    ap.add_argument("--calibrate-read", type=int, default=0, metavar="MIB",
                    help="run only the streaming-read calibration kernel over MIB MiB")
    ap.add_argument("--calibrate-mfma", action="store_true",
                    help="run only the dense bf16 MFMA calibration kernel")
    ap.add_argument("--no-calibration", action="store_true",
                    help="skip the measured-peak calibration of the default run")
    return ap.parse_args()


def calibrate_copy(mib: int) -> int:
    import torch
    dev = torch.device("cuda:0")
    n = mib * 2**20
    x = torch.ones(n // 4, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(5):
        torch.mul(x, 1.0, out=y)  # one elementwise kernel: reads n bytes, writes n bytes
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / 5
    print(json.dumps({"calibration": "device copy (elementwise multiply by 1.0)",
                      "bytes_read_per_launch": n, "bytes_written_per_launch": n, "launches": 5,
                      "ms_per_launch": round(dt * 1e3, 4)}), flush=True)
    return 0


# ---------------------------------------------------------------------------
def prefill_attention_flops(w, lens=None) -> float:
    """4 * h_q * d * sum_p |T(p)|, |T(p)| = min(k, n(p)) * B + (p+1) mod B, over the query
    positions (the last n_q of the sequence for a chunk; every position of every prompt for
    a varlen batch, padding rows excluded)."""
    def positions_sum(lo, hi):
        p = np.arange(lo, hi, dtype=np.int64)
        n = (p + 1) // w.block
        return float((np.minimum(w.top_k, n) * w.block + (p + 1) % w.block).sum())
    if lens is not None:
        return 4.0 * w.h_q * w.d * sum(positions_sum(0, int(L)) for L in lens)
    return 4.0 * w.h_q * w.d * positions_sum(w.seq - (w.n_q or w.seq), w.seq) * w.batch


def decode_attention_bytes(w, lens) -> float:
    """Selected K and V rows of every KV head + q + out + sel + kv_lens."""
    esz = 2 if w.dtype == "bf16" else 4
    L = lens.astype(np.int64)
    tsz = np.minimum(w.top_k, L // w.block) * w.block + L % w.block
    kv = float(tsz.sum()) * w.h_kv * w.d * esz * 2
    return kv + 2.0 * w.batch * w.h_q * w.d * esz + w.batch * w.top_k * 4 + w.batch * 4


def graph_steps(steps: int, most: int = 16, replays: int = 20) -> int:
    """Steps captured in one graph: the largest divisor of `steps` up to `most` that still
    leaves at least `replays` replays (all `steps` replays when there are fewer steps)."""
    need = min(replays, steps)
    return max(d for d in range(1, min(most, steps) + 1) if steps % d == 0 and steps // d >= need)


def median_ms(pairs) -> tuple:
    """(median, mean) of the elapsed times of (start, end) event pairs, in ms."""
    t = sorted(a.elapsed_time(b) for a, b in pairs)
    n = len(t)
    med = t[n // 2] if n % 2 else 0.5 * (t[n // 2 - 1] + t[n // 2])
    return med, sum(t) / n


def compulsory_bytes(w, lens=None) -> float:
    """Bytes a prefill attention launch moves at least once: q, k, v and sel read, out and
    lse written (varlen: each prompt's own rows)."""
    esz = 2 if w.dtype == "bf16" else 4
    if lens is not None:
        rows = float(np.sum(lens))
        kv_rows = rows
    else:
        rows = float(w.batch * (w.n_q or w.seq))
        kv_rows = float(w.batch * w.seq)
    per_row = w.h_q * w.d * esz * 2 + w.top_k * 4 + w.h_q * 4  # q + out + sel + lse
    return rows * per_row + kv_rows * w.h_kv * w.d * esz * 2


# Sources the attention kernel of each workload kind is compiled from (with the build
# script, whose flags shape the code): the committed counter summaries stay valid while
# these are unchanged.
ATTN_SOURCES = {
    "prefill": ("k_prefill.hip", "k_prefill_rt.hip", "prefill_common.h", "qsa_device.h",
                "qsa_internal.h"),
    "decode": ("k_decode.hip", "qsa_device.h", "qsa_internal.h"),
}


def kernel_src_hash(kind: str) -> str:
    """Hash of the attention kernel's sources for a workload kind (varlen: prefill)."""
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "block_sparse_attention_37_amd")
    files = [os.path.join("csrc", n) for n in ATTN_SOURCES["decode" if kind == "decode" else "prefill"]]
    for name in files + ["build.py"]:
        with open(os.path.join(pkg, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def load_counters(workload: str, kind: str):
    """The committed rocprofv3 counter summary of this workload's attention launch, if it was
    taken on the current attention kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_src_sha") != kernel_src_hash(kind):
        return None
    return t


def prefill_tile_shape(h_q: int, h_kv: int, d: int):
    """(positions per workgroup tile, positions per wave) of the bf16 prefill kernels."""
    g = h_q // h_kv
    pw = 32 // g if d <= 128 else (16 * (2 if g == 32 else 1)) // g
    return 8 * pw, pw


def union_stats(sel, pos, block: int, mq: int, pw: int):
    """Lock-step work of the prefill kernels from a selection: a tile of mq consecutive rows
    walks the union of its rows' selected blocks and own (non-empty trailing) blocks, a wave of
    pw rows computes on the union of its rows'.  sel [n_q, k] (-1 padded) and pos [n_q] (row
    positions; negative = padding) of one sequence.  Returns (sum over tiles of union x rows,
    same over waves, sum over rows of blocks needed)."""
    import numpy as np
    n = np.where(pos >= 0, (pos + 1) // block, 0)
    valid = (sel >= 0) & (sel < n[:, None]) & (pos >= 0)[:, None]
    own = np.where((pos >= 0) & ((pos + 1) % block != 0), pos // block, -1)
    needed = int(valid.sum() + (own >= 0).sum())

    def walked(step):
        tot = 0
        for a in range(0, len(pos), step):
            rows = slice(a, a + step)
            live = int((pos[rows] >= 0).sum())
            if live:
                u = np.union1d(sel[rows][valid[rows]], own[rows][own[rows] >= 0])
                tot += len(u) * live
        return tot

    return walked(mq), walked(pw), needed


# ---------------------------------------------------------------------------
def setup_prefill(w, dev):
    import torch
    from block_sparse_attention_37_amd import qsa as Q
    from block_sparse_attention_37_amd import synth as S
    inps = [S.prefill_inputs(w, seq_id=b) for b in range(w.batch)]
    st = lambda key: torch.stack([S.to_torch(x[key]) for x in inps]).to(dev)
    plan = Q.PrefillPlan(st("q"), st("k"), st("v"), st("iq"), st("ik"), w.block, w.top_k, w.sm_scale,
                         n_q=w.n_q or None)
    return plan, inps


def setup_varlen(w, dev):
    """Prompts of mixed length: q, iq right-aligned in [batch, n_q] with n_q the longest
    prompt; k, v, ik from row 0 of [batch, max_len]."""
    import torch
    from block_sparse_attention_37_amd import qsa as Q
    from block_sparse_attention_37_amd import synth as S
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    lens, seqs = S.varlen_inputs(w)
    n_q = int(lens.max())
    q = torch.zeros(w.batch, n_q, w.h_q, w.d, dtype=dt, device=dev)
    iq = torch.zeros(w.batch, n_q, w.h_idx, w.d_idx, dtype=dt, device=dev)
    k = torch.zeros(w.batch, w.max_len, w.h_kv, w.d, dtype=dt, device=dev)
    v = torch.zeros_like(k)
    ik = torch.zeros(w.batch, w.max_len, w.d_idx, dtype=dt, device=dev)
    for b, x in seqs.items():
        L = int(lens[b])
        q[b, n_q - L:] = S.to_torch(x["q"]).to(dev)
        iq[b, n_q - L:] = S.to_torch(x["iq"]).to(dev)
        k[b, :L] = S.to_torch(x["k"]).to(dev)
        v[b, :L] = S.to_torch(x["v"]).to(dev)
        ik[b, :L] = S.to_torch(x["ik"]).to(dev)
    kvl = torch.from_numpy(lens.astype(np.int32)).to(dev)
    plan = Q.VarlenPrefillPlan(q, k, v, iq, ik, kvl, w.block, w.top_k, w.sm_scale)
    return plan, seqs, lens


def setup_decode(w, dev):
    import torch
    from block_sparse_attention_37_amd import qsa as Q
    from block_sparse_attention_37_amd import synth as S
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    lens = S.decode_lens(w)
    kc = torch.zeros(w.batch, w.max_len, w.h_kv, w.d, dtype=dt, device=dev)
    vc = torch.zeros_like(kc)
    ik = torch.zeros(w.batch, w.max_len, w.d_idx, dtype=dt, device=dev)
    q = torch.zeros(w.batch, w.h_q, w.d, dtype=dt, device=dev)
    iq = torch.zeros(w.batch, 1, w.h_idx, w.d_idx, dtype=dt, device=dev)
    for b, s in S.decode_sequences(w, lens):
        if b % 16 == 0:
            print(f"[bench] generating decode inputs: sequence {b}/{w.batch}", file=sys.stderr, flush=True)
        L = int(lens[b])
        kc[b, :L] = S.to_torch(s["k"]).to(dev)
        vc[b, :L] = S.to_torch(s["v"]).to(dev)
        ik[b, :L] = S.to_torch(s["ik"]).to(dev)
        q[b] = S.to_torch(s["q"]).to(dev)
        iq[b, 0] = S.to_torch(s["iq"]).to(dev)
    kvl = torch.from_numpy(lens).to(dev)
    # indexer state of the prefix before the newest token (not timed); each step's index call
    # completes the block the newest token finishes (qsa_index_topk_decode)
    cmp = Q.compress_keys(ik, w.block, kv_lens=kvl - 1)
    plan = Q.DecodePlan(q, kc, vc, kvl, iq, cmp, w.block, w.top_k, w.sm_scale, ik_cache=ik)
    return plan, lens


# ---------------------------------------------------------------------------
def _tie_band(scores, top_k: int, rel: float = 1e-3) -> bool:
    """True when the m-th and (m+1)-th largest scores of a row lie within `rel` relative
    (m = min(top_k, n); rows that keep every candidate have no band)."""
    n = len(scores)
    m = min(top_k, n)
    if m == n:
        return False
    srt = np.sort(scores)[::-1]
    a, b = srt[m - 1], srt[m]
    scale = max(abs(a), abs(b))
    return scale > 0 and (a - b) / scale <= rel


def baseline_rows(T: int, block: int, top_k: int, seed: int = 0):
    """Stratified oracle sample of a prompt: the first 2*block rows, the block-end rows of the
    last 8 blocks, the last row, then seeded rows drawn uniformly from the whole prompt (in
    that order, so a time budget cuts the seeded tail)."""
    head = list(range(min(T, 2 * block)))
    ends = [p for p in range(max(2 * block, T - 8 * block), T) if (p + 1) % block == 0]
    last = [T - 1] if T - 1 not in head and T - 1 not in ends else []
    fixed = set(head) | set(ends) | set(last)
    rest = [int(p) for p in np.random.default_rng(seed).permutation(T) if int(p) not in fixed]
    return head, ends + last, rest


def cpu_baseline(w, inps, lens, budget_s: float):
    """The fp64 oracle on a bounded sample of the workload, single-threaded BLAS."""
    from threadpoolctl import threadpool_limits
    import oracle.qsa_oracle as O
    from block_sparse_attention_37_amd import synth as S
    t_start = time.perf_counter()
    ties = rows_scored = 0
    with threadpool_limits(limits=1):
        if w.kind in ("prefill", "varlen"):
            if w.kind == "varlen":  # the longest prompt of the batch stands for the others
                b = int(np.argmax(lens))
                x, w = inps[b], w.with_(seq=int(lens[b]), kind="prefill")
            else:
                x = inps[0]
            q, k, v = S.to_f64(x["q"]), S.to_f64(x["k"]), S.to_f64(x["v"])
            iq, ik = S.to_f64(x["iq"]), S.to_f64(x["ik"])
            t0 = time.perf_counter()
            cmp = O.compress_keys(ik, w.block)
            t_cmp = time.perf_counter() - t0
            nq = w.n_q or w.seq
            lo = w.seq - nq
            head, ends, rest = baseline_rows(nq, w.block, w.top_k)
            timed = {}
            for part, rows in (("head", head), ("ends", ends), ("uniform", rest)):
                for i in rows:
                    p = lo + i
                    t0 = time.perf_counter()
                    n = O.candidate_blocks(int(p), w.block)
                    s = O.block_scores(iq[p], cmp, n)
                    sel = O.select_blocks(s, w.top_k)
                    O.attend(q[p], k, v, O.token_set(sel, int(p), w.block), w.sm_scale)
                    timed.setdefault(part, []).append(time.perf_counter() - t0)
                    ties += int(_tie_band(s, w.top_k))
                    rows_scored += 1
                    if part == "uniform" and time.perf_counter() - t_start > budget_s:
                        break
            # the uniform rows stand for the whole prompt; the fixed strata are reported
            uni = timed.get("uniform") or timed.get("ends") or timed["head"]
            per_tok = float(np.mean(uni)) + t_cmp / nq
            sample = (f"compression of all {w.seq} tokens; selection + attention of the rows "
                      f"0..{2 * w.block - 1} ({len(timed.get('head', []))} rows), the block-end "
                      f"rows of the last 8 blocks and the last row ({len(timed.get('ends', []))}), "
                      f"and {len(timed.get('uniform', []))} seeded rows drawn uniformly from all "
                      f"{nq}; tokens/s extrapolated from the uniform rows' mean time per row")
            value = 1.0 / per_tok
            extra = {"extrapolated": True,
                     "ms_per_row": {k2: round(1e3 * float(np.mean(v2)), 3) for k2, v2 in timed.items()}}
        else:
            done, t_seq = 0, 0.0
            order = np.random.default_rng(0).permutation(w.batch)
            for b in order:
                s = S.decode_sequence(w, int(b), int(lens[b]))
                L = int(lens[b])
                cmp = O.compress_keys(S.to_f64(s["ik"]), w.block)
                t0 = time.perf_counter()
                r = O.decode(S.to_f64(s["q"]), S.to_f64(s["k"]), S.to_f64(s["v"]), L,
                             S.to_f64(s["iq"]), cmp, w.block, w.top_k, w.sm_scale)
                t_seq += time.perf_counter() - t0
                scores = O.block_scores(S.to_f64(s["iq"]), cmp, O.candidate_blocks(L - 1, w.block))
                ties += int(_tie_band(scores, w.top_k))
                rows_scored += 1
                done += 1
                del r
                if time.perf_counter() - t_start > budget_s:
                    break
            value = done / t_seq
            sample = (f"{done} of {w.batch} sequences (selection + attention per new token; the "
                      f"compressed indexer state is prepared untimed, as on the GPU)")
            extra = {"extrapolated": done < w.batch}
    out = {"value": round(value, 3), "unit": "tokens/s", "cores": 1, "kind": "oracle",
           "sample": sample, "host_cpus": os.cpu_count(), "blas_threads": 1}
    out.update(extra)
    return out, {"rows": rows_scored, "frac": round(ties / max(rows_scored, 1), 4)}


def run_calibration(mode: str, mib: int = 4096) -> int:
    import torch
    from block_sparse_attention_37_amd import calibrate as C
    dev = torch.device("cuda:0")
    res = C.measure_read_gbs(dev, mib) if mode == "read" else C.measure_mfma_tflops(dev)
    print(json.dumps({"calibration": res}), flush=True)
    return 0


# ---------------------------------------------------------------------------
def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "QSA here runs on exactly one GPU; --gpus must be 1 "
                                   "(sharding across GPUs is not implemented)"}))
        return 2
    if args.calibrate_copy:
        return calibrate_copy(args.calibrate_copy)
    if args.calibrate_read:
        return run_calibration("read", args.calibrate_read)
    if args.calibrate_mfma:
        return run_calibration("mfma")
    import torch
    from block_sparse_attention_37_amd import synth as S
    w = S.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    big = w.name in ("long_prefill_bf16_128k", "long_decode_bf16_b128")
    steps = args.steps if args.steps is not None else (20 if big else 200)
    warmup = args.warmup if args.warmup is not None else (3 if big else 20)

    t_setup = time.perf_counter()
    if w.kind == "prefill":
        plan, inps = setup_prefill(w, dev)
        lens = None
        tokens = w.batch * (w.n_q or w.seq)  # query tokens processed per step
    elif w.kind == "varlen":
        plan, inps, lens = setup_varlen(w, dev)
        tokens = int(lens.sum())  # prompt tokens (padding rows excluded)
    else:
        plan, lens = setup_decode(w, dev)
        inps = None
        tokens = w.batch
    torch.cuda.synchronize()
    t_setup = time.perf_counter() - t_setup
    print(f"[bench] {w.name}: inputs resident after {t_setup:.1f} s; warm-up", file=sys.stderr,
          flush=True)

    stream = torch.cuda.current_stream(dev)
    for _ in range(warmup):
        plan.run()
    torch.cuda.synchronize()
    if args.graph:
        # one graph holds `per_graph` consecutive whole steps (index (+ compression for
        # prefill), then attention, in stream order); a graph launch costs several
        # microseconds of its own, so the timed steps replay it steps / per_graph times
        per_graph = graph_steps(steps)
        g_step = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_step):
            for _ in range(per_graph):
                plan.run()
        g_step.replay()  # untimed: instantiates the graph
        torch.cuda.synchronize()
        run_step, launches = g_step.replay, steps // per_graph
    else:
        per_graph = 1
        run_step, launches = plan.run, steps

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    torch.cuda.synchronize()
    pairs = [(ev(), ev()) for _ in range(launches)]
    for a, b in pairs:
        a.record(stream)
        run_step()
        b.record(stream)
    torch.cuda.synchronize()
    med, mean = median_ms(pairs)
    ms_per_step, ms_per_step_mean = med / per_graph, mean / per_graph
    print(f"[bench] timed {steps} steps: {ms_per_step:.4f} ms per step (median)", file=sys.stderr,
          flush=True)

    # Launch duration of the attention call for the roofline: >= 20 replays of
    # `per_att` back-to-back calls between two events each, on the stream the kernels run on
    # (for short calls several per replay amortise the launch gaps, so the figure compares
    # with a profiler's per-kernel average duration); the median replay.
    reps = max(20, launches)
    # back-to-back calls per replay: enough for ~5 ms of kernel time (at most 16), so that
    # launch gaps of short calls are amortised whatever the step count
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    plan.run_attention()
    t1.record(stream)
    torch.cuda.synchronize()
    per_att = int(min(16, max(1, round(5.0 / max(t0.elapsed_time(t1), 1e-3)))))
    if args.graph:
        g_rep = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_rep):
            for i in range(per_att):
                plan.run_attention()
        torch.cuda.synchronize()
        run_rep = g_rep.replay
    else:
        def run_rep():
            for i in range(per_att):
                plan.run_attention()
    run_rep()
    torch.cuda.synchronize()
    apairs = [(ev(), ev()) for _ in range(reps)]
    for a, b in apairs:
        a.record(stream)
        run_rep()
        b.record(stream)
    torch.cuda.synchronize()
    att_med, att_mean = median_ms(apairs)
    att_ms = att_med / per_att
    value = tokens / (ms_per_step / 1e3)

    calib = None
    if not args.no_calibration:
        from block_sparse_attention_37_amd import calibrate as C
        calib = (C.measure_mfma_tflops(dev) if w.kind in ("prefill", "varlen")
                 else C.measure_read_gbs(dev))
        torch.cuda.synchronize()

    if w.kind in ("prefill", "varlen"):
        work = prefill_attention_flops(w, lens if w.kind == "varlen" else None)
        achieved = work / (att_ms / 1e3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4)}
        if calib:
            roof["peak_measured"] = calib["TFLOP/s"]
            roof["frac_of_measured"] = round(achieved / calib["TFLOP/s"], 4)
    else:
        work = decode_attention_bytes(w, lens)
        achieved = work / (att_ms / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
        if calib:
            roof["peak_measured"] = calib["GB/s"]
            roof["frac_of_measured"] = round(achieved / calib["GB/s"], 4)
    if calib:
        roof["calibration"] = calib
    counters = load_counters(w.name, w.kind)
    roof["traffic"] = counters.get("bytes_per_launch") if counters else None
    if roof["traffic"] and w.kind in ("prefill", "varlen"):
        roof["compulsory_bytes"] = compulsory_bytes(w, lens if w.kind == "varlen" else None)
        roof["traffic_over_compulsory"] = round(roof["traffic"] / roof["compulsory_bytes"], 3)
    elif roof["traffic"]:
        roof["traffic_over_algorithmic"] = round(roof["traffic"] / work, 4)
    if counters and "mfma" in counters:
        roof["mfma_executed_over_algorithmic"] = counters["mfma"]["executed_over_algorithmic"]
        roof["mfma_busy_pct"] = counters["mfma"]["busy_pct"]
    # the attention call: one kernel for prefill; split kernel + merge kernel for decode
    roof["kernel"] = (("qsa::prefill_bf16_rt_kernel" if w.d == 256 else "qsa::prefill_bf16_kernel")
                      if w.kind in ("prefill", "varlen")
                      else "qsa::decode_bf16_kernel + qsa::decode_merge_few_kernel (2-4 splits) or qsa::decode_merge_kernel")
    roof["algorithmic_per_launch"] = work
    roof["kernel_ms"] = round(att_ms, 5)
    roof["kernel_ms_mean"] = round(att_mean / per_att, 5)
    roof["kernel_replays"] = reps
    roof["kernel_calls_per_replay"] = per_att

    cpu, tie = None, None
    if not args.no_cpu_baseline:
        print("[bench] oracle baseline on the host", file=sys.stderr, flush=True)
        cpu, tie = cpu_baseline(w, inps, lens, args.cpu_seconds)

    cfg = {"workload": w.name, "kind": w.kind, "batch": w.batch, "block": w.block,
           "top_k": w.top_k, "h_q": w.h_q, "h_kv": w.h_kv, "d": w.d, "h_idx": w.h_idx,
           "d_idx": w.d_idx, "graph": bool(args.graph), "steps_per_graph": per_graph}
    if w.kind == "prefill":
        cfg["seq"] = w.seq
        if w.n_q:
            cfg["n_q"] = w.n_q
    elif w.kind == "varlen":
        cfg.update(max_len=w.max_len, n_q=int(lens.max()), prompt_len_min=int(lens.min()),
                   prompt_len_max=int(lens.max()), prompt_tokens=int(lens.sum()))
    else:
        cfg.update(max_len=w.max_len, kv_len_min=int(lens.min()), kv_len_max=int(lens.max()))
    if w.kind in ("prefill", "varlen") and w.dtype == "bf16":
        # blocks the kernel walks per row (tile union) and computes on (wave union), over the
        # blocks a row needs, from this run's own selection
        sel = plan.sel.cpu().numpy()
        n_q = sel.shape[1]
        mq, pw = prefill_tile_shape(w.h_q, w.h_kv, w.d)
        kvl = lens if w.kind == "varlen" else [w.seq] * sel.shape[0]
        tt = wv = nd = 0
        for b in range(sel.shape[0]):
            a, c, e = union_stats(sel[b], np.arange(n_q) + int(kvl[b]) - n_q, w.block, mq, pw)
            tt, wv, nd = tt + a, wv + c, nd + e
        roof["union"] = {"tile_positions": mq, "wave_positions": pw,
                         "tile_over_needed": round(tt / max(nd, 1), 3),
                         "wave_over_needed": round(wv / max(nd, 1), 3)}

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(ms_per_step, 5),
        "ms_per_step_mean": round(ms_per_step_mean, 5), "timed_replays": launches,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded; see block_sparse_attention_37_amd/synth.py)",
        "config": cfg, "roofline": roof, "cpu_baseline": cpu,
        "tie_band_rows": tie, "setup_s": round(t_setup, 1),
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
