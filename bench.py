"""Benchmark: page-selected sparse decode attention steps/s on one MI355X.

A step is one layer's decode for the whole batch through one C-ABI call, decode_step:
page_meta_update (tail page), select_pages and sparse_decode, as a single launch when one
workgroup refreshes, ranks and attends each unit. The default workload is the
ragged batch: B=32 sequences of 16K..32K tokens, 32 query / 8 KV heads, D=128, bf16,
5% page budget (sink and tail included). Inputs are resident in HBM before timing; steps
rotate over --rotate device copies of (cache, statistics, q) so that consecutive steps
do not hit in the last-level cache. The other legs run before the W warmup steps and the
K measured ones, so that the measured region runs at steady clocks (a 20-step region
right after the GPU wakes runs about 8 % slower).

Prints one JSON line. Besides the contract fields it carries:
  roofline      achieved algorithmic GB/s of the dominant kernel against 8 TB/s; a
                one-launch step is timed over launches 2..K of the measured region
  cpu_baseline  the fp64 oracle's step on the host: all usable cores (the value), one
                thread, and the oracle's dense step
  calls         per-call average durations (HIP events on the launch stream)
  launch_floor  back-to-back empty kernels on the same stream (the per-launch floor)
  configs       the other measured workloads (tiny, 8B-GQA shape at 32K, 1M tokens, MLA
                latent): one decode step and the dense decode, with the speed-up
  separate      the same step as three calls (page_meta_update, select_pages,
                sparse_decode)
  dense         the dense baseline (psd_dense_decode) on the same inputs
  graph_replay  the same step replayed from a captured HIP graph (launch cost removed),
                with a bit-for-bit check against the eager outputs
  warm          the same step on one copy of the inputs, over and over (caches warm;
                labeled, never the headline)
  host_link     with --v-host: the kept pages' V bytes per step and their rate over the
                host link
  coverage_select  the adaptive coverage selection (--coverage, default 0.95) on the
                same inputs: selection alone and selection plus sparse attention, with
                the algorithmic GB/s of the dense K read the page masses need
  value_tier    V in pinned host memory with a resident hot buffer of 1.5x one step's
                kept slices, over 8 steps of drifting queries: hit rate, host-link bytes
                per step (against reading every kept V row from host memory) and the
                step time (--no-tier skips it)
  kv_tier       the same with K in pinned host memory too (the KV tier: each resident
                slice holds its K and V rows)
  walks         the step's reads with no arithmetic (psd_diag_walk), on the same rotated
                copies: the kept pages' K and V rows and the candidate statistics
                records, with their GB/s (--no-walk skips them)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PREHEAT_CALLS = 160  # step + dense pairs run untimed first (about 0.1 s on the ragged batch)
METRIC = "sparse decode attn steps/s + effective HBM GB/s (% peak), B=32 @32K ctx"


def algorithmic_bytes(w, sel_counts: np.ndarray) -> dict:
    """Bytes each call must move at minimum (reads + writes), from the workload and the
    selection sizes: statistics of the scored pages, K/V of the kept pages' valid tokens,
    q, block-table entries, the tail-page refresh and the outputs."""
    sp = w.spec
    es = 2 if sp.dtype == "bf16" else 4
    B, Hq, Hkv, D, Dv = sp.batch, sp.num_q_heads, sp.num_kv_heads, sp.head_dim, sp.head_dim_v
    lens = w.seq_lens.astype(np.int64)
    n = (lens + 15) // 16
    tail_valid = lens - 16 * (n - 1)
    meta_b = int(np.sum(tail_valid * Hkv * D * es + 2 * Hkv * D * es + 8))  # K tail + stats
    scored = np.where(n > w.budgets, n - 2, 0)  # pages whose bound is computed
    # scoring: statistics and block-table entries of the scored pages, q, and the row
    # headers; merging: the ranked winners it writes
    score_b = int(np.sum(scored) * (Hkv * 2 * D * es + 4) + B * Hq * D * es + B * 8 +
                  B * Hkv * 4)
    ranked = np.where(n > w.budgets, np.maximum(np.minimum(n, w.budgets), 2) - 2, 0)
    merge_b = int(np.sum(ranked) * Hkv * 4)
    select_b = score_b + merge_b
    # valid tokens: every kept page is full except the tail page (always kept)
    kv_tok_valid = int(np.sum(sel_counts.sum(axis=1) * 16 - Hkv * (16 - tail_valid)))
    kdim = D + (0 if sp.latent else Dv)  # latent rows are read once for K and V
    sparse_b = int(kv_tok_valid * kdim * es + B * Hq * D * es +
                   int(sel_counts.sum()) * 8 + B * Hq * Dv * 4)
    dense_tok = int(np.sum(lens)) * Hkv
    dense_b = int(dense_tok * kdim * es + int(np.sum(n)) * 4 + B * Hq * D * es + B * Hq * Dv * 4)
    return dict(meta_update=meta_b, select_score=score_b, select_merge=merge_b,
                select=select_b, sparse_decode=sparse_b, step=meta_b + select_b + sparse_b,
                dense_decode=dense_b, score_stats=int(np.sum(scored) * Hkv * 2 * D * es))


KERNEL_SOURCES = {"score_kernel": ("select.hip",), "merge_kernel": ("select.hip",),
                  "select_attn_kernel": ("select.hip", "attn_core.h"),
                  "prescore_kernel": ("prescore.hip",), "certify_kernel": ("prescore.hip",),
                  "meta_kernel": ("meta.hip",), "attn_kernel": ("attn.hip", "attn_core.h"),
                  "attn_latent_kernel": ("attn.hip", "attn_core.h"),
                  "attn_latent_tile_kernel": ("attn.hip", "attn_core.h"),
                  "lse_merge_kernel": ("attn.hip", "attn_core.h"),
                  "page_mass_mfma_kernel": ("coverage.hip",),
                  "coverage_cut_kernel": ("coverage.hip",)}


def one_call_kernel(w):
    """The kernel behind decode_step and select_sparse_decode when each is a single launch,
    else None.
    Follows the library's planning rule: at least 128 (sequence, KV head) units of at
    most 2048 candidate pages, or block-table rows of at most 256 pages at any batch size;
    groups of up to 4 query heads, D = D_v <= 128 (bf16) or D = D_v = 64 (fp32), and no
    certified pre-score."""
    sp = w.spec
    G = sp.num_q_heads // sp.num_kv_heads
    units = sp.batch * sp.num_kv_heads
    width = w.block_table.shape[1]
    d_ok = sp.head_dim <= 128 if sp.dtype == "bf16" else sp.head_dim == 64
    if (G <= 4 and d_ok and sp.head_dim_v == sp.head_dim and
            ((units >= 128 and width - 2 <= 2048) or width <= 256)):
        return "select_attn_kernel"
    return None


def call_bytes(ab: dict, call: str) -> int:
    """Algorithmic bytes of one C-ABI call."""
    if call == "select_sparse_decode":
        return ab["select"] + ab["sparse_decode"]
    if call == "decode_step":
        return ab["step"]
    return ab[{"page_meta_update": "meta_update"}.get(call, call)]


def selection_kernels(w) -> tuple:
    """Names of the kernels behind select_score and select_merge for a workload. Follows
    the library's planning rule: bf16 groups of 16..128 query heads (a multiple of 16)
    with D of 64, 128 or 576 take the certified MFMA pre-score and its certify stage;
    everything else the exact bound kernel and the chunk merge."""
    sp = w.spec
    G = sp.num_q_heads // sp.num_kv_heads
    max_pages = int(np.max((w.seq_lens + 15) // 16))
    if (sp.dtype == "bf16" and 16 <= G <= 128 and G % 16 == 0 and
            sp.head_dim in (64, 128, 576) and max_pages - 2 <= 7168):
        return "prescore_kernel", "certify_kernel"
    return "score_kernel", "merge_kernel"


def source_digest(kernel: str) -> str:
    """sha256 of the HIP sources a kernel is built from (with the shared device header)."""
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "page_selected_sparse_amd", "csrc")
    for f in (*KERNEL_SOURCES[kernel], "psd_device.h"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed counter summary
    profiles/<kernel>_<workload>_hbm_counters.txt (FETCH_SIZE + WRITE_SIZE, scaled by the
    copy calibration), or None when there is none or the kernel source has changed since
    the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_counters.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("source_sha256") != source_digest(kernel):
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _oracle_seq_time(w, inp, s, prefill, kind: str) -> float:
    """Seconds of the oracle's step for sequence s: the decode step (tail refresh, bound,
    selection, attention; the prefill statistics are given, untimed) or the dense step."""
    from oracle import psd_oracle as O

    L = int(w.seq_lens[s])
    n = O.pages_of(L)
    if kind == "dense":
        t0 = time.perf_counter()
        O.dense_step(inp["q"], inp["k_cache"], inp["v_cache"], w.block_table, w.seq_lens,
                     w.scale, w.spec.head_dim_v, w.spec.num_kv_heads, sequences=[s])
        return time.perf_counter() - t0
    kmin, kmax = (m.copy() for m in prefill[s])
    t0 = time.perf_counter()
    tail = inp["k_cache"][w.block_table[s, n - 1: n]][0, : O.valid_in_page(L, n - 1)]
    kmin[n - 1], kmax[n - 1] = O.page_minmax(tail)
    sel, _ = O.select_sequence(inp["q"][s], kmin, kmax, w.spec.num_kv_heads, n,
                               int(w.budgets[s]))
    O.decode_sequence(inp["q"][s], inp["k_cache"], inp["v_cache"], w.block_table[s], L, sel,
                      w.scale, w.spec.head_dim_v)
    return time.perf_counter() - t0


_FORKED = {}  # the workload, inherited by forked oracle workers


def _oracle_worker(job):
    """One forked worker: its share of the batch (every P-th sequence), `passes` times.
    Returns the seconds of each pass."""
    from threadpoolctl import threadpool_limits

    import synth
    from oracle import psd_oracle as O

    j, P, passes, kind = job
    w = _FORKED["w"]
    inp = synth.oracle_inputs(w)
    seqs = list(range(j, w.spec.batch, P))
    with threadpool_limits(limits=1):
        prefill = {} if kind == "dense" else {
            s: O.sequence_meta(inp["k_cache"], w.block_table[s], int(w.seq_lens[s])) for s in seqs}
        return [sum(_oracle_seq_time(w, inp, s, prefill, kind) for s in seqs)
                for _ in range(passes)]


def _oracle_all_cores(w, kind: str, cores: int, passes: int) -> float:
    """Median seconds of a whole-batch oracle pass with the sequences spread over `cores`
    forked processes (BLAS one thread each): a pass lasts as long as its busiest worker."""
    import multiprocessing as mp

    _FORKED["w"] = w
    P = max(1, min(cores, w.spec.batch))
    with mp.get_context("fork").Pool(P) as pool:
        per_worker = pool.map(_oracle_worker, [(j, P, passes, kind) for j in range(P)])
    return float(np.median(np.max(np.array(per_worker), axis=0)))


def cpu_baseline(w, budget_s: float = 15.0, min_s: float = 10.0) -> dict:
    """The fp64 oracle as it stands, timed on the host. Runs before the GPU is touched
    (it forks worker processes).

    value: the decode step (tail refresh, bound, selection, attention) over the whole
    batch with the sequences spread over all usable cores (one process per core, at most
    16, BLAS one thread each), median of three passes. one_thread: the same step on one
    thread: whole-batch passes repeated until min_s has elapsed (at least three, median
    reported) when a pass takes under min_s / 3, else as many sequences as fit in
    ~budget_s, scaled to the batch. dense: the oracle's dense step on all cores."""
    from threadpoolctl import threadpool_limits

    import synth
    from oracle import psd_oracle as O

    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    t_all = _oracle_all_cores(w, "sparse", cores, 3)
    t_dense = _oracle_all_cores(w, "dense", cores, 1 if w.spec.batch < cores else 3)

    inp = synth.oracle_inputs(w)
    prefill = {}
    with threadpool_limits(limits=1):
        total, done = 0.0, 0
        for s in range(w.spec.batch):
            prefill[s] = O.sequence_meta(inp["k_cache"], w.block_table[s], int(w.seq_lens[s]))
            total += _oracle_seq_time(w, inp, s, prefill, "sparse")
            done += 1
            if total >= budget_s:
                break
        if done == w.spec.batch and total < min_s / 3:
            passes = [total]
            while len(passes) < 3 or sum(passes) < min_s:
                passes.append(sum(_oracle_seq_time(w, inp, s, prefill, "sparse")
                                  for s in range(w.spec.batch)))
            per_step = float(np.median(passes))
            sample = (f"the whole {w.spec.name} step, {len(passes)} passes "
                      f"({sum(passes):.1f} s of fp64 NumPy on one thread), median pass")
        else:
            per_step = total / done * w.spec.batch
            sample = (f"{done} of {w.spec.batch} sequences of the {w.spec.name} step "
                      f"({total:.1f} s of fp64 NumPy on one thread), scaled to the full batch")
    used = min(cores, w.spec.batch)
    return {"value": round(1.0 / t_all, 6), "unit": "steps/s", "cores": used, "kind": "oracle",
            "sample": (f"the whole {w.spec.name} step, sequences spread over {used} processes "
                       f"(BLAS one thread each), median of 3 passes of {t_all:.2f} s"),
            "one_thread": {"value": round(1.0 / per_step, 6), "unit": "steps/s", "cores": 1,
                           "sample": sample},
            "dense": {"value": round(1.0 / t_dense, 6), "unit": "steps/s", "cores": used,
                      "sample": f"the oracle's dense step over the whole batch, {t_dense:.2f} s "
                                f"per pass on {used} processes"},
            "host": host_info()}


def host_info() -> dict:
    """CPU model and the cores this process may use (the oracle above uses one)."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "usable_cores": len(os.sched_getaffinity(0))}


def timed_over(objs, fn, iters: int) -> float:
    """Average ms of fn(objs[i % len(objs)]) over iters back-to-back calls: HIP events on
    torch's current stream (the stream the library's kernels are queued on), bracketed by
    device synchronisations."""
    import torch

    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(iters):
        fn(objs[i % len(objs)])
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


def launch_floor(iters: int) -> dict:
    """Back-to-back empty kernels (torch's spin kernel with zero cycles) on the current
    stream: the per-launch cost below which no dependent launch chain can go."""
    import torch

    for _ in range(10):
        torch.cuda._sleep(0)
    ms = timed_over([None], lambda _: torch.cuda._sleep(0), iters)
    return {"us_per_launch": round(ms * 1e3, 3), "launches": iters,
            "kernel": "torch.cuda._sleep(0), back to back on one stream"}


def value_tier_leg(w, base, dev, steps: int = 8, kv: bool = False) -> dict:
    """The value tier over consecutive decode steps: V (with ``kv``, K and V: the KV tier)
    in pinned host memory, a resident hot buffer of 1.5x one step's kept (block, KV head)
    slices, queries on a random walk (about 5 % per step). Per step: hits, slices copied
    over the host link and their bytes, the step time (selection, staging, attention)
    against the same step reading every kept row from host memory (zero copy)."""
    import torch

    from page_selected_sparse_amd import DecodeStep

    sp = w.spec
    st = DecodeStep(base.q.clone(), base.cache, base.block_table, base.seq_lens, base.budgets,
                    sp.head_dim_v, sp.latent, b_max=base.b_max, v_host=True, kv_host=kv)
    st.build_meta()
    st.select()
    kept0 = int(st.sel_count.clamp(min=0).sum())
    slots = int(1.5 * kept0)
    st.enable_tier(slots, kv=kv)
    es = 2 if sp.dtype == "bf16" else 4
    slice_bytes = 16 * (sp.head_dim_v + (sp.head_dim if kv else 0)) * es
    gen = torch.Generator(device=dev).manual_seed(11)
    q = st.q.float()
    rows = []

    def ev_time(fn):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    for t in range(steps):
        if t:
            q = q + 0.05 * torch.randn(q.shape, generator=gen, device=dev)
        st.q.copy_(q.to(st.q.dtype))
        ms_tier = ev_time(lambda: (st.select(), st.tier_stage(), st.sparse_tiered()))
        c = st.tier_counts()
        kept = int(st.sel_count.clamp(min=0).sum())
        ms_zero = ev_time(lambda: (st.select(), st.sparse()))
        rows.append({"step": t, "kept_slices": kept, "hits": c["hits"],
                     "copied": c["copied"], "from_host": c["from_host"],
                     "link_bytes": c["copied"] * slice_bytes + c["from_host"] * slice_bytes,
                     "zero_copy_link_bytes": kept * slice_bytes,
                     "ms": round(ms_tier, 4), "zero_copy_ms": round(ms_zero, 4)})
    warm = rows[1:]
    res = {"slots": slots, "slice_bytes": slice_bytes,
           "hot_buffer_bytes": slots * slice_bytes,
           "host_pool_bytes": int(st.v.numel() * st.v.element_size() +
                                  (st.k.numel() * st.k.element_size() if kv else 0)),
           "hit_rate": round(sum(r["hits"] for r in warm) / max(1, sum(r["kept_slices"] for r in warm)), 4),
           "link_bytes_per_step": int(np.mean([r["link_bytes"] for r in warm])),
           "zero_copy_link_bytes_per_step": int(np.mean([r["zero_copy_link_bytes"] for r in warm])),
           "ms_per_step": round(float(np.mean([r["ms"] for r in warm])), 4),
           "zero_copy_ms_per_step": round(float(np.mean([r["zero_copy_ms"] for r in warm])), 4),
           "first_step": rows[0], "steps": rows,
           "note": "queries on a random walk of about 5 % per step; steps after the first "
                   "averaged; each step timed alone (selection, staging, attention)"}
    del st
    torch.cuda.empty_cache()
    return res


def measure_config(name: str, args, dev) -> dict:
    """One decode step (psd_decode_step) and the dense decode (psd_dense_decode) of
    another measured workload, on rotated resident copies as for the headline."""
    import torch

    import synth
    from page_selected_sparse_amd import DecodeStep

    w = synth.make_workload(name)
    base = DecodeStep.from_arrays(w.q, w.cache, w.block_table, w.seq_lens, w.budgets,
                                  w.spec.dtype, w.spec.head_dim_v, w.spec.latent, device=dev)
    sts = [base] + [DecodeStep(base.q.clone(), base.cache.clone(), base.block_table.clone(),
                               base.seq_lens.clone(), base.budgets.clone(), w.spec.head_dim_v,
                               w.spec.latent, b_max=base.b_max) for _ in range(args.rotate - 1)]
    for st in sts:
        st.build_meta()
    for i in range(max(args.warmup, 2 * len(sts))):
        sts[i % len(sts)].step()
        sts[i % len(sts)].dense()
    iters = max(100, args.steps)
    ms_step = timed_over(sts, lambda st: st.step(), iters)
    ms_dense = timed_over(sts, lambda st: st.dense(), max(10, iters // 4))
    ab = algorithmic_bytes(w, sts[0].sel_count.cpu().numpy())
    res = {"workload": name, "step_us": round(ms_step * 1e3, 2),
           "dense_us": round(ms_dense * 1e3, 2),
           "speedup_vs_dense": round(ms_dense / ms_step, 3),
           "step_gbs": round(ab["step"] / (ms_step * 1e-3) / 1e9, 1),
           "dense_gbs": round(ab["dense_decode"] / (ms_dense * 1e-3) / 1e9, 1),
           "dtype": w.spec.dtype, "rotated_copies": len(sts)}
    del sts, base
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--no-walk", action="store_true",
                    help="skip the memory walks (the step's reads with no arithmetic)")
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="ragged_b32_32k")
    ap.add_argument("--rotate", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay of the step (reported beside the eager rate)")
    ap.add_argument("--v-host", action="store_true",
                    help="V cache in pinned host memory (value tier in host DRAM): the step reads "
                         "the kept pages' V over the host link")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a 1 GiB device copy (for HBM counter scaling)")
    ap.add_argument("--coverage", type=float, default=0.95,
                    help="target mass of the adaptive coverage selection leg (0: skip it)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the step / dense pairs of the other measured workloads")
    ap.add_argument("--no-tier", action="store_true",
                    help="skip the value-tier leg (V in pinned host memory, hot buffer)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this library has no multi-GPU path; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import synth

    t0 = time.time()
    w = synth.make_workload(args.workload)
    print(f"[bench] workload {w.spec.name} generated in {time.time() - t0:.1f}s", file=sys.stderr,
          flush=True)
    cpu = None
    if not args.no_cpu_baseline:  # forks worker processes: before the GPU is initialised
        t0 = time.time()
        cpu = cpu_baseline(w)
        print(f"[bench] oracle baseline timed in {time.time() - t0:.1f}s", file=sys.stderr,
              flush=True)

    import torch

    from page_selected_sparse_amd import DecodeStep

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    base = DecodeStep.from_arrays(w.q, w.cache, w.block_table, w.seq_lens, w.budgets,
                                  w.spec.dtype, w.spec.head_dim_v, w.spec.latent, device=dev,
                                  v_host=args.v_host)
    steps = [base]
    for _ in range(args.rotate - 1):
        steps.append(DecodeStep(base.q.clone(), base.cache.clone(), base.block_table.clone(),
                                base.seq_lens.clone(), base.budgets.clone(), w.spec.head_dim_v,
                                w.spec.latent, b_max=base.b_max, v_host=args.v_host))
    for st in steps:
        st.build_meta()
    torch.cuda.synchronize()
    R = len(steps)

    def timed(fn, iters, prime=True):
        """Average ms of fn over iters calls on the rotated copies (HIP events on torch's
        current stream); with `prime`, one untimed call per copy first."""
        if prime:
            for st in steps:
                fn(st)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(iters):
            fn(steps[i % R])
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters  # ms

    # The other legs run before the measured region, the other workloads first, so that
    # the measured region runs at steady clocks on inputs the legs just before it have
    # touched (a 20-step region right after the GPU wakes runs about 8 % slower). First,
    # untimed, about 0.1 s of steps and dense walks brings the GPU to its steady clocks.
    for i in range(PREHEAT_CALLS):
        steps[i % R].step()
        steps[i % R].dense()
    torch.cuda.synchronize()
    launch_fl = launch_floor(max(100, args.steps))
    configs = None
    if not args.no_configs:
        configs = [measure_config(name, args, dev) for name in synth.CONFIG_ORDER
                   if name != w.spec.name]
    ms_separate = timed(lambda st: st.step_separate(), args.steps)
    dense_ms = timed(lambda st: st.dense(), max(10, args.steps // 4)) if not args.no_dense else None

    # warm: one copy of the inputs, steps back to back (the Infinity Cache may serve reads)
    ms_warm = timed(lambda st: steps[0].step(), args.steps)

    # Adaptive coverage selection (GQA shapes only): the selection alone, and selection
    # plus the sparse attention over its rows, which hold every page of a sequence.
    cov = None
    if args.coverage > 0 and w.spec.group <= 8 and not w.spec.latent:
        wide = int(w.block_table.shape[1])
        csteps = [DecodeStep(st.q, st.cache, st.block_table, st.seq_lens, st.budgets,
                             w.spec.head_dim_v, w.spec.latent, b_max=wide) for st in steps]

        def ctimed(fn, iters):
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(iters):
                fn(csteps[i % R])
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / iters

        for st in csteps:
            st.select_coverage(args.coverage)
            st.sparse()
        iters = max(10, args.steps // 4)
        ms_sel = ctimed(lambda st: st.select_coverage(args.coverage), iters)
        ms_cstep = ctimed(lambda st: (st.select_coverage(args.coverage), st.sparse()), iters)
        ccounts = csteps[0].sel_count.cpu().numpy()
        es = 2 if w.spec.dtype == "bf16" else 4
        lens = w.seq_lens.astype(np.int64)
        n_pages = (lens + 15) // 16
        # every valid K row once per KV head, q, and the per-head page max and sum written
        # by the mass kernel and read back by the cut kernel
        k_bytes = int(lens.sum()) * w.spec.num_kv_heads * w.spec.head_dim * es
        sel_bytes = (k_bytes + w.q.nbytes + 2 * 2 * 4 * w.spec.num_q_heads * int(n_pages.sum())
                     + ccounts.size * (wide + 1) * 4)
        cstep_bytes = sel_bytes + algorithmic_bytes(w, ccounts)["sparse_decode"]
        cov = {"coverage": args.coverage, "row_entries": wide,
               "kept_pages_mean": round(float(ccounts.mean()), 1),
               "kept_fraction_mean": round(float((ccounts / n_pages[:, None]).mean()), 4),
               "select_ms": round(ms_sel, 5),
               "select_gbs": round(sel_bytes / (ms_sel * 1e-3) / 1e9, 1),
               "select_bytes": sel_bytes,
               "step_ms": round(ms_cstep, 5),
               "step_gbs": round(cstep_bytes / (ms_cstep * 1e-3) / 1e9, 1),
               "step_bytes": cstep_bytes,
               "kernels": "page_mass_mfma_kernel (bf16) or page_mass_kernel (fp32) + "
                          "coverage_cut_kernel",
               # HBM bytes per launch from the committed counters (None when stale)
               "traffic": {k: measured_traffic(k, w.spec.name)
                           for k in ("page_mass_mfma_kernel", "coverage_cut_kernel")}}
        del csteps

    # Per-call averages, each call timed in its own loop with events on the stream the
    # kernels are launched on (torch's current stream). page_meta_update, select_score and
    # select_merge are single kernels (select_merge launches none when each scoring
    # workgroup ranked a whole unit); sparse_decode is the attention kernel, plus the split
    # merge unless one workgroup attends each unit; decode_step and select_sparse_decode are
    # one kernel each where one_call_kernel() names it, else the launches of their calls.
    calls = {"page_meta_update": timed(lambda st: st.refresh_tail(), args.steps),
             "select_sparse_decode": timed(lambda st: st.select_sparse(), args.steps),
             "select_score": timed(lambda st: st.select_score(), args.steps),
             "select_merge": timed(lambda st: st.select_merge(), args.steps),
             "sparse_decode": timed(lambda st: st.sparse(), args.steps)}
    # W untimed warmup steps, then the measured region: K whole steps on the rotated
    # copies; then the same call in its own K-step loop (calls_ms).
    for i in range(args.warmup):
        steps[i % R].step()
    torch.cuda.synchronize()
    # One more event after the first step: launches 2..K run back to back behind it, so
    # their span is K - 1 launch durations without the first launch's start from an idle
    # queue (the kernel's average duration inside the timed region, as rocprofv3 sees it).
    e0, e_first, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    e0.record()
    for i in range(args.steps):
        steps[i % R].step()
        if i == 0:
            e_first.record()
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    ms_launch = e_first.elapsed_time(e1) / (args.steps - 1) if args.steps > 1 else ms_step
    calls["decode_step"] = timed(lambda st: st.step(), args.steps, prime=False)

    graph = None
    if not args.no_graph:
        # The same step replayed from a HIP graph (one captured step per rotated copy),
        # checked bit for bit against the eager outputs.
        for st in steps:
            st.step()
        torch.cuda.synchronize()
        eager_out = [st.out.clone() for st in steps]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for st in steps:
                st.step()
        replays = max(1, args.steps // R)
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        same = all(torch.equal(st.out, o) for st, o in zip(steps, eager_out))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(replays):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        same = same and all(torch.equal(st.out, o) for st, o in zip(steps, eager_out))
        ms_graph = e0.elapsed_time(e1) / (replays * R)
        graph = {"ms_per_step": round(ms_graph, 5), "steps_per_s": round(1000.0 / ms_graph, 3),
                 "matches_eager": bool(same)}
        del g

    # The step's reads with no arithmetic (psd_diag_walk): the kept pages' K and V rows,
    # and the candidate pages' statistics records, on the same rotated copies.
    walk_ms = None
    if not args.no_walk:
        walk_ms = (timed(lambda st: st.walk(0), args.steps), timed(lambda st: st.walk(1), args.steps))

    if args.calibrate_copy:
        x = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        y = torch.empty_like(x)
        for _ in range(5):
            y.copy_(x)
        torch.cuda.synchronize()

    sel_counts = steps[0].sel_count.cpu().numpy()
    ab = algorithmic_bytes(w, sel_counts)
    # The dominant single-kernel call and its achieved algorithmic bandwidth.
    score_k, merge_k = selection_kernels(w)
    kernel_of = {"select_score": (score_k, ab["select_score"]),
                 "select_merge": (merge_k, ab["select_merge"]),
                 "page_meta_update": ("meta_kernel", ab["meta_update"])}
    fused_k = one_call_kernel(w)
    if fused_k:
        kernel_of = {"decode_step": (fused_k, ab["step"])}
    dom = max(kernel_of, key=lambda k: calls[k])
    kname, dom_bytes = kernel_of[dom]
    # a one-launch step is timed inside the measured region; other calls in their loops
    dom_ms = ms_launch if dom == "decode_step" else calls[dom]
    dom_src = ("measured region, launches 2..K" if dom == "decode_step"
               else f"{dom}, its own K-call loop")
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    step_gbs = ab["step"] / (ms_step * 1e-3) / 1e9
    traffic = measured_traffic(kname, w.spec.name)

    result = {
        "metric": METRIC,
        "value": round(1000.0 / ms_step, 3),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.spec.dtype,
        "data": "synthetic",
        "config": {"workload": w.spec.name, "batch": w.spec.batch,
                   "seq_lens": f"uniform [{w.spec.len_range[0]}, {w.spec.len_range[1]}]"
                   if w.spec.len_range else list(map(int, w.seq_lens[:1])),
                   "q_heads": w.spec.num_q_heads, "kv_heads": w.spec.num_kv_heads,
                   "head_dim": w.spec.head_dim, "page": 16,
                   "budget": f"{w.spec.budget_percent}% of pages" if w.spec.budget_percent
                   else f"{w.spec.budget_pages} pages",
                   "rotated_copies": R, "v_in_host_memory": bool(args.v_host)},
        "effective_hbm_gbs": round(step_gbs, 1),
        "effective_hbm_pct_peak": round(100.0 * step_gbs / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "kernel": kname, "call": dom,
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "algorithmic_bytes": dom_bytes, "ms": round(dom_ms, 5),
                     "ms_from": dom_src, "traffic": traffic},
        "calls_ms": {k: round(v, 5) for k, v in calls.items()},
        # algorithmic GB/s of every call (sparse_decode: attention plus the split merge)
        "calls_gbs": {k: round(call_bytes(ab, k) / (v * 1e-3) / 1e9, 1)
                      for k, v in calls.items()},
        "separate": {"ms_per_step": round(ms_separate, 5),
                     "steps_per_s": round(1000.0 / ms_separate, 3)},
        "warm": {"ms_per_step": round(ms_warm, 5), "steps_per_s": round(1000.0 / ms_warm, 3),
                 "note": "one copy of the inputs, caches warm"},
        "algorithmic_bytes": ab,
    }
    if args.v_host:
        # the kept pages' valid V rows cross the host link once per step
        es = 2 if w.spec.dtype == "bf16" else 4
        lens = w.seq_lens.astype(np.int64)
        n = (lens + 15) // 16
        v_tok = int(np.sum(sel_counts.sum(axis=1) * 16 - w.spec.num_kv_heads * (16 - (lens - 16 * (n - 1)))))
        v_bytes = v_tok * w.spec.head_dim_v * es
        result["host_link"] = {"v_bytes_per_step": v_bytes,
                               "gbs": round(v_bytes / (ms_step * 1e-3) / 1e9, 2)}
    if walk_ms is not None:
        es = 2 if w.spec.dtype == "bf16" else 4
        n = (w.seq_lens.astype(np.int64) + 15) // 16
        kept = int(np.clip(sel_counts, 0, None).sum())
        row = w.spec.head_dim + (0 if w.spec.latent else w.spec.head_dim_v)
        kv_bytes = kept * 16 * row * es
        st_bytes = int(np.maximum(n - 2, 0).sum()) * w.spec.num_kv_heads * 2 * w.spec.head_dim * es
        result["walks"] = {
            "kv_ms": round(walk_ms[0], 5), "kv_bytes": kv_bytes,
            "kv_gbs": round(kv_bytes / (walk_ms[0] * 1e-3) / 1e9, 1),
            "stats_ms": round(walk_ms[1], 5), "stats_bytes": st_bytes,
            "stats_gbs": round(st_bytes / (walk_ms[1] * 1e-3) / 1e9, 1),
            "note": "the step's reads with no arithmetic (psd_diag_walk): kv = the kept "
                    "pages' K and V rows (what sparse_decode reads), stats = every candidate "
                    "page's statistics record (what the scoring reads)"}
    if cov is not None:
        result["coverage_select"] = cov
    if graph is not None:
        result["graph_replay"] = graph
    if not args.no_tier and not w.spec.latent and w.spec.head_dim == w.spec.head_dim_v:
        result["value_tier"] = value_tier_leg(w, steps[0], dev)
        result["kv_tier"] = value_tier_leg(w, steps[0], dev, kv=True)
    if dense_ms is not None:
        result["dense"] = {"ms": round(dense_ms, 5),
                           "gbs": round(ab["dense_decode"] / (dense_ms * 1e-3) / 1e9, 1),
                           "step_speedup_vs_dense": round(dense_ms / ms_step, 3)}
    result["launch_floor"] = launch_fl
    if configs is not None:
        result["configs"] = configs
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
