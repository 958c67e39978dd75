"""Benchmark of the KDA state-recurrence hot path on one MI355X.

One step = one pass of the whole path over resident synthetic inputs:
  * kda_chunk_prefill on the single-layer workload (1 sequence, T = 8229 =
    128 full chunks + a tail of 37, H = 32 heads, d_k = d_v = 128, chunk 64,
    bf16 q/k/v/g/b, fp32 pool, zero initial state, snapshot at c = 128);
  * kda_recurrent_verify, kda_commit, kda_commit_align, kda_state_copy and
    the conv-state update on the speculative workload (256 requests, L = 8,
    H = 32, fp32 128 x 128 checkpoints in a 1024-slot pool, accepted
    ~ U{0..8}, in-place commit, fork of 64 committed checkpoints to 4
    children each).
Two passes of K steps each: a warm pass back to back (bracketed by the wall
clock: ms_per_step), and a flushed pass in which, before every step and
outside its timed calls, the checkpoint slots the commits overwrite are
restored from a pristine copy and a 512 MiB write evicts the L2 and the
memory-side cache, so every call starts with its inputs in HBM only.
value = prefill tokens/s = T / median flushed prefill time (the warm figure
is reported beside it).  Each call is bracketed by HIP events on the stream
it is launched on; the roofline object covers the call that dominates the
step.  Informational legs outside the step time the same prefill on the
varlen batch (16 sequences, lengths ~ U[512, 16384]; `prefill_varlen`) and
on one 131072-token sequence (`prefill_long`), each with its own roofline
fractions, and the verify -> commit -> fork copy loop of speculative
decoding back to back (`decode_loop`).  The cpu_baseline leg times the fp64
oracle on the host's cores (one process per group of heads), before the GPU
is touched.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-varlen]
       python bench.py --only-leg long|varlen|graph   (one informational leg alone, for profiling)
"""

import argparse
import json
import os
import platform
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import linear_attention_state_kda_amd as kda  # noqa: E402
import workloads as wl  # noqa: E402

HBM_PEAK = 8.0e12            # bytes/s, MI355X HBM3E
# the launches of one prefill call: a single sequence needs no chunk map
PREFILL_KERNELS = {False: "kda_chunk_prefill (kda_chunk_prep16 + kda_chunk_scan16)",
                   True: "kda_chunk_prefill (kda_chunk_map + kda_chunk_prep16 + kda_chunk_scan16)"}
CSRC = os.path.join(ROOT, "linear_attention_state_kda_amd", "csrc")
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "prefill_traffic.md")
BF16_PEAK = 2.5e15           # FLOP/s, dense bf16 MFMA
METRIC = "KDA chunk-prefill tokens/s + %MFMA peak; verify/commit state GB/s + %HBM"


def i32(x, dev):
    return torch.as_tensor(np.asarray(x, dtype=np.int32), device=dev)


def prefill_setup(dev):
    case = wl.single_layer_prefill()
    toks, cu = wl.prefill_tokens(case)
    H, d, C = case["H"], case["dk"], case["chunk"]
    t = {n: toks[n].to(dev) for n in "qkvgb"}
    pool = torch.zeros((case["n_slots"], H, d, d), dtype=torch.float32, device=dev)
    s, c, slot = case["tracks"][0]
    args = dict(q=t["q"], k=t["k"], v=t["v"], g=t["g"], b=t["b"], cu_seqlens=i32(cu, dev), chunk=C,
                pool=pool, init_slot=i32(case["init_slots"], dev), final_slot=i32(case["final_slots"], dev),
                track_ptr=i32([0, 1], dev), track_chunk=i32([c], dev), track_slot=i32([slot], dev),
                track_f32=torch.empty((1, H, d, d), dtype=torch.float32, device=dev))
    T = int(cu[-1])
    args["o"] = torch.empty((T, H, d), dtype=torch.bfloat16, device=dev)
    args["workspace"] = torch.empty(kda.prefill_workspace_bytes(1, T, H, d, d, C, torch.bfloat16),
                                    dtype=torch.uint8, device=dev)
    # algorithmic traffic and work: per token-head 4d+1 inputs
    # and d outputs in bf16; per sequence-head the zero init reads nothing, the
    # final state and one snapshot are written in fp32 plus the fp32 copy.
    bytes_ = T * H * (4 * d * 2 + 2 + d * 2) + H * d * d * 4 * 3
    flops = T * H * (6 * d * d + 5 * C * d)
    return case, args, T, bytes_, flops


def spec_setup(dev, **sizes):
    case = wl.spec_case(seed=3, **sizes)
    n_req, L, H, d = case["n_req"], case["L"], case["H"], case["dk"]
    toks = wl.token_inputs(n_req * L, H, d, d, "bf16", case["seed"], shape_prefix=(n_req, L))
    t = {n: toks[n].to(dev) for n in "qkvgb"}
    pool = torch.zeros((case["n_slots"], H, d, d), dtype=torch.float32, device=dev)
    gen = torch.Generator(device=dev).manual_seed(case["seed"])
    ck = torch.as_tensor(case["ckpt_slots"], dtype=torch.long, device=dev)
    pool[ck] = torch.randn((n_req, H, d, d), generator=gen, device=dev)
    o = torch.empty((n_req, L, H, d), dtype=torch.bfloat16, device=dev)
    u_rec = torch.empty((n_req, H, L, d), dtype=torch.float32, device=dev)
    kg_rec = torch.empty((n_req, H, L, 2 * d), dtype=torch.bfloat16, device=dev)
    acc = case["accepted"]
    s_in = 2
    verify_bytes = n_req * H * (d * d * 4 + L * (4 * d * s_in + s_in + d * s_in + 4 * d + 2 * d * s_in))
    commit_bytes = sum(H * (2 * d * d * 4 + int(n) * (4 * d + 2 * d * s_in)) for n in acc if n > 0)
    copy_bytes = len(case["fork_src"]) * 2 * H * d * d * 4
    # conv half of the state tuple: q, k, v short-conv windows of H*d channels,
    # width 4 (3 history rows) plus L speculative rows, bf16, one slot per pool slot
    conv_keep, conv_rows, conv_dim = 3, 3 + L, H * d
    conv = [torch.zeros((case["n_slots"], conv_rows, conv_dim), dtype=torch.bfloat16, device=dev)
            for _ in range(3)]
    for c in conv:
        c.normal_(generator=gen)
    conv_op_bytes = 3 * conv_keep * conv_dim * 2 * 2          # read + write of the history rows
    n_fork = len(case["fork_src"])
    # align mode: states per block of 64 tokens; request r holds pos[r] ~ U{1..4096}
    # tokens, its checkpoint is its block's slot, the next block's slot is a fresh one
    bs = 64
    pos = np.random.default_rng([case["seed"], 77]).integers(1, 4097, n_req)
    nb = 4096 // bs + 1
    table = np.full((n_req, nb), -1, dtype=np.int32)
    b0, b1 = (pos - 1) // bs, (pos + acc - 1) // bs
    table[np.arange(n_req), b0] = case["ckpt_slots"]
    table[np.arange(n_req), b0 + 1] = case["fork_dst"][:n_req]
    closes = (b1 > b0) & (b1 * bs - pos > 0)
    align_bytes = int(sum(H * (d * d * 4 * (2 + int(c)) + int(n) * (4 * d + 2 * d * s_in))
                          for n, c in zip(acc, closes) if n > 0))
    return dict(case=case, t=t, pool=pool, o=o, u_rec=u_rec, kg_rec=kg_rec,
                ckpt=i32(case["ckpt_slots"], dev), acc=i32(acc, dev),
                src=i32(case["fork_src"], dev), dst=i32(case["fork_dst"], dev),
                conv=conv, conv_keep=[conv_keep] * 3, zero_shift=i32([0] * n_fork, dev),
                align_table=torch.as_tensor(table, device=dev), align_pos=i32(pos, dev), align_bs=bs,
                bytes=dict(verify=verify_bytes, commit=commit_bytes, copy=copy_bytes,
                           commit_align=align_bytes,
                           conv_compact=conv_op_bytes * int((acc > 0).sum()),
                           conv_fork=conv_op_bytes * n_fork))


def informational_setup(dev, case):
    """A prefill workload for the informational legs, drawn with torch's
    generator on the device: the same distributions as the seeded workload
    (q, k unit rows, v, b ~ N(0, 1), g ~ U(-0.1, -0.001), pool states ~ N(0, 1)),
    without its fp64 host pass (these legs are timed, not checked)."""
    lengths = np.asarray(case["lengths"], dtype=np.int64)
    T, H, d, C = int(lengths.sum()), case["H"], case["dk"], case["chunk"]
    gen = torch.Generator(device=dev).manual_seed(case["seed"])

    def unit(x):
        return x / x.norm(dim=-1, keepdim=True)
    t = {"q": unit(torch.randn((T, H, d), generator=gen, device=dev)),
         "k": unit(torch.randn((T, H, d), generator=gen, device=dev)),
         "v": torch.randn((T, H, d), generator=gen, device=dev),
         "g": torch.empty((T, H, d), device=dev).uniform_(-0.1, -0.001, generator=gen),
         "b": torch.randn((T, H), generator=gen, device=dev)}
    t = {n: x.to(torch.bfloat16) for n, x in t.items()}
    pool = torch.randn((case["n_slots"], H, d, d), generator=gen, device=dev)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    tr = sorted(case["tracks"])
    ptr = np.searchsorted([s_ for s_, _, _ in tr], np.arange(len(lengths) + 1)).astype(np.int32)
    args = dict(q=t["q"], k=t["k"], v=t["v"], g=t["g"], b=t["b"], cu_seqlens=i32(cu, dev), chunk=C,
                pool=pool, init_slot=i32(case["init_slots"], dev), final_slot=i32(case["final_slots"], dev),
                track_ptr=i32(ptr, dev), track_chunk=i32([c for _, c, _ in tr], dev),
                track_slot=i32([sl for _, _, sl in tr], dev),
                track_f32=torch.empty((len(tr), H, d, d), dtype=torch.float32, device=dev),
                o=torch.empty((T, H, d), dtype=torch.bfloat16, device=dev))
    args["workspace"] = torch.empty(kda.prefill_workspace_bytes(len(lengths), T, H, d, d, C, torch.bfloat16),
                                    dtype=torch.uint8, device=dev)
    # per sequence-head: init read (if any) and final write; per snapshot the
    # pool write and the fp32 copy; all fp32
    n_init = sum(1 for s_ in case["init_slots"] if s_ >= 0)
    bytes_ = T * H * (4 * d * 2 + 2 + d * 2) + (n_init + len(lengths) + 2 * len(tr)) * H * d * d * 4
    flops = T * H * (6 * d * d + 5 * C * d)
    return args, T, len(lengths), bytes_, flops


def time_leg(dev, st, case, label, reps=5):
    """Median of `reps` prefill calls (after 2 untimed) on an informational
    workload, with its roofline fractions (HBM: algorithmic bytes; MFMA:
    algorithmic FLOP against the dense bf16 peak)."""
    args, T, n, bytes_, flops = informational_setup(dev, case)
    for _ in range(2):
        kda.chunk_prefill(**args)
    evs = [[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for _ in range(reps)]
    for e0, e1 in evs:
        e0.record(st)
        kda.chunk_prefill(**args)
        e1.record(st)
    torch.cuda.synchronize()
    ms = float(np.median([e0.elapsed_time(e1) for e0, e1 in evs]))
    del args
    s_ = ms * 1e-3
    return {"workload": f"{label}, {n} sequence(s), {T} tokens, H=32, d=128, chunk 64, bf16, fp32 pool",
            "ms_median": ms, "tokens_per_s": T / s_,
            "hbm_GBps": bytes_ / s_ / 1e9, "hbm_frac": bytes_ / s_ / HBM_PEAK,
            "mfma_TFLOPs": flops / s_ / 1e12, "mfma_frac": flops / s_ / BF16_PEAK,
            "roofline": {"kernel": PREFILL_KERNELS[n > 1],
                         "bound": "hbm", "achieved": bytes_ / s_ / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                         "frac": bytes_ / s_ / HBM_PEAK, "algorithmic_bytes_per_launch": bytes_,
                         "algorithmic_flop_per_launch": flops, "mfma_frac": flops / s_ / BF16_PEAK,
                         "avg_launch_ms": ms}}


def decode_loop_leg(sp, st, iters=10, warm=3):
    """The speculative-decoding loop's own order on the speculative workload:
    verify, in-place commit and fork copy, repeated back to back with no
    synchronisation in between; per-call medians and roofline fractions."""
    t = sp["t"]
    names = ("verify", "commit", "copy")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(iters)]
    for i in range(warm + iters):
        e = evs[i - warm] if i >= warm else None
        if e:
            e[0].record(st)
        kda.recurrent_verify(t["q"], t["k"], t["v"], t["g"], t["b"], sp["pool"], sp["ckpt"],
                             o=sp["o"], u_rec=sp["u_rec"], kg_rec=sp["kg_rec"])
        if e:
            e[1].record(st)
        kda.commit(sp["pool"], sp["ckpt"], sp["acc"], sp["u_rec"], sp["kg_rec"])
        if e:
            e[2].record(st)
        kda.state_copy(sp["pool"], sp["src"], sp["dst"])
        if e:
            e[3].record(st)
    torch.cuda.synchronize()
    out = {"workload": "verify -> commit -> fork copy, repeated back to back (256 requests, L=8, "
                       "H=32, fp32 pool), median of %d" % iters}
    for j, c in enumerate(names):
        ms = float(np.median([e[j].elapsed_time(e[j + 1]) for e in evs]))
        out[c] = {"ms": round(ms, 4), "hbm_frac": round(sp["bytes"][c] / (ms * 1e-3) / HBM_PEAK, 4)}
    return out


def graph_loop_leg(dev, batches=(4, 16, 64), iters=200, warm=100):
    """The decoding loop (verify, in-place commit, fork copy) on small
    batches, where each kernel lasts a few microseconds and submitting the
    launches can cost as much as running them: back-to-back iterations
    issued one call at a time against the same iteration captured once as a
    HIP graph and replayed (every call is capturable: no allocation, no
    memset, no host read-back).  Per-iteration time over `iters` iterations,
    after `warm` untimed ones (fewer leave the first batch's eager loop
    several times slower while the device ramps up)."""
    return {"workload": f"verify -> commit -> fork copy, L=8, H=32, fp32 pool, fork of n_req/4 "
                        f"checkpoints to 4 children each; {iters} iterations back to back",
            "by_batch": [_graph_loop(dev, n, iters, warm) for n in batches]}


def _graph_loop(dev, n_req, iters, warm):
    sp = spec_setup(dev, n_req=n_req, n_slots=4 * n_req + 64, n_fork_src=n_req // 4)
    t = sp["t"]

    def one():
        kda.recurrent_verify(t["q"], t["k"], t["v"], t["g"], t["b"], sp["pool"], sp["ckpt"],
                             o=sp["o"], u_rec=sp["u_rec"], kg_rec=sp["kg_rec"])
        kda.commit(sp["pool"], sp["ckpt"], sp["acc"], sp["u_rec"], sp["kg_rec"])
        kda.state_copy(sp["pool"], sp["src"], sp["dst"])

    def timed(run):
        for _ in range(warm):
            run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        w0 = time.perf_counter()
        e0.record()
        for _ in range(iters):
            run()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters * 1e3, (time.perf_counter() - w0) / iters * 1e6

    eager_us, eager_wall = timed(one)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        one()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        one()
    graph_us, graph_wall = timed(g.replay)
    nbytes = sum(sp["bytes"][c] for c in ("verify", "commit", "copy"))
    return {"n_req": n_req, "eager_us_per_iter": round(eager_us, 2), "graph_us_per_iter": round(graph_us, 2),
            "eager_host_us_per_iter": round(eager_wall, 2), "graph_host_us_per_iter": round(graph_wall, 2),
            "hbm_frac_eager": round(nbytes / (eager_us * 1e-6) / HBM_PEAK, 4),
            "hbm_frac_graph": round(nbytes / (graph_us * 1e-6) / HBM_PEAK, 4)}


def measured_prefill_traffic():
    """HBM bytes per prefill call from the committed FETCH_SIZE / WRITE_SIZE
    profile (already scaled by the copy calibration), or None when the
    prefill sources changed since those counters were taken; with a label
    naming where the figure comes from."""
    import hashlib
    h = hashlib.sha256()
    for name in ("prefill.hip", "prefill16.hip", "prefill_common.hpp", "kda_common.hpp", "kda_launch.hpp"):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    try:
        fields = dict(line.split(": ", 1) for line in open(TRAFFIC_PROFILE).read().splitlines()
                      if line.startswith(("traffic_bytes_per_call: ", "source_sha256_16: ")))
    except OSError:
        return None, "none: profiles/prefill_traffic.md missing"
    if fields.get("source_sha256_16", "").strip() != h.hexdigest()[:16]:
        return None, f"none: the prefill sources (sha256 {h.hexdigest()[:16]}) changed since the counters in " \
                     f"profiles/prefill_traffic.md were taken"
    return int(fields["traffic_bytes_per_call"]), \
        f"profiles/prefill_traffic.md: rocprofv3 FETCH_SIZE and WRITE_SIZE of the same kernels, scaled by a " \
        f"plain copy of known size, taken for prefill sources sha256 {h.hexdigest()[:16]} (the ones built " \
        f"here); not measured in this run"


def committed_copy_traffic_ratio():
    """HBM bytes over algorithmic bytes of the fork copy, from the committed
    FETCH_SIZE / WRITE_SIZE profile (the copy reads each shared source once
    for all of its children), or None if absent."""
    try:
        for line in open(os.path.join(ROOT, "profiles", "state_paths_traffic.md")):
            if line.startswith("| copy"):
                return float(line.strip().strip("|").split("|")[-1])
    except (OSError, ValueError):
        pass
    return None


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo when readable)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def _oracle_heads(args):
    """Worker of the CPU baseline: the fp64 token loop on a group of heads
    of the first n tokens (one thread per process)."""
    case, heads, n = args
    from threadpoolctl import threadpool_limits
    from oracle import kda_oracle as ko

    d = case["dk"]
    toks = wl.token_inputs(case["lengths"][0], case["H"], d, d, case["in_dtype"], case["seed"], heads=heads)
    ex = {x: wl.exact(toks[x][:n]) for x in "qkvgb"}
    with threadpool_limits(limits=1):
        ko.run_sequence(*(ex[x][:8] for x in "qkvgb"), np.zeros((len(heads), d, d)))   # first-call costs
        t0 = time.perf_counter()
        ko.run_sequence(*(ex[x] for x in "qkvgb"), np.zeros((len(heads), d, d)))
        return time.perf_counter() - t0


def cpu_baseline(case, seconds_target=20.0):
    """Time the fp64 oracle on the host's cores: the heads are independent,
    so one process per group of heads runs the token loop over the same
    first tokens; the wall time of the slowest group gives tokens/s.  Runs
    before the GPU is initialised (worker processes are spawned, never
    forked from a process holding the GPU)."""
    import concurrent.futures as cf
    import multiprocessing as mp

    H = case["H"]
    cores = max(1, min(len(os.sched_getaffinity(0)), 16, H))
    groups = [list(range(H))[i::cores] for i in range(cores)]
    ctx = mp.get_context("spawn")
    with cf.ProcessPoolExecutor(max_workers=cores, mp_context=ctx) as ex:
        # a short probe sizes the sample to about `seconds_target` of wall time
        probe = 64
        t_probe = max(ex.map(_oracle_heads, [(case, g, probe) for g in groups]))
        n = int(max(256, min(case["lengths"][0], probe * seconds_target / max(t_probe, 1e-6))))
        t0 = time.perf_counter()
        times = list(ex.map(_oracle_heads, [(case, g, n) for g in groups]))
        wall = time.perf_counter() - t0
    worst = max(times)
    # one core's rate on the whole workload: each process's seconds per head, averaged, times H
    per_head = float(np.mean([t / len(g) for t, g in zip(times, groups)]))
    return {"value": n / worst, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "single_core_value": n / (per_head * H),
            "sample": f"first {n} of {case['lengths'][0]} tokens of the single-layer prefill, all {H} heads "
                      f"in {cores} processes of {H // cores}-{-(-H // cores)} heads each, fp64 token loop "
                      f"(slowest process {worst:.1f} s, {wall:.1f} s wall with input setup); "
                      f"single_core_value: all {H} heads on one core, from the processes' mean time per head"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-steps", type=int, default=None,
                    help="steps of the flushed pass (default: --steps; value is taken from this pass)")
    ap.add_argument("--no-varlen", action="store_true",
                    help="skip the informational legs (prefill on the varlen batch of 16 "
                         "sequences and on the long-context sequence of 131072 tokens; the "
                         "speculative-decoding loop, eager and as a replayed HIP graph)")
    ap.add_argument("--only-leg", choices=("long", "varlen", "graph"), default=None,
                    help="run one informational leg alone and print it: a prefill leg (10 timed "
                         "calls) or the small-batch decoding loop, eager and graph-replayed")
    ap.add_argument("--traffic-calibration", action="store_true",
                    help="after the timed steps, run one kda_state_copy of 256 distinct fp32 "
                         "slots (512 MiB read + 512 MiB written) so that FETCH_SIZE / WRITE_SIZE "
                         "counters can be scaled against a copy of known size")
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the KDA path here is built and timed on a single "
              "MI355X (no collectives); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    cold_steps = a.steps if a.cold_steps is None else a.cold_steps
    case = wl.single_layer_prefill()
    # the oracle baseline runs first, on the host's cores, before anything touches the GPU
    cb = None
    if not a.no_cpu_baseline and a.only_leg is None:
        cb = cpu_baseline(case)
        cb["cpu"] = cpu_model()
    dev = torch.device("cuda:0")
    kda.lib()
    st = torch.cuda.current_stream()
    if a.only_leg == "graph":
        print(json.dumps({"leg": a.only_leg, **graph_loop_leg(dev)}), flush=True)
        return
    if a.only_leg is not None:
        leg = wl.long_prefill() if a.only_leg == "long" else wl.varlen_prefill("f32")
        print(json.dumps({"leg": a.only_leg, **time_leg(dev, st, leg, a.only_leg, reps=10)}), flush=True)
        return
    case, pargs, T, p_bytes, p_flops = prefill_setup(dev)
    sp = spec_setup(dev)
    ck_long = sp["ckpt"].long()
    pristine = sp["pool"][ck_long].clone()    # the checkpoints, before any commit

    def ev():
        return torch.cuda.Event(enable_timing=True)

    calls = ["prefill", "verify", "commit", "commit_align", "conv_compact", "copy", "conv_fork"]

    def step(events=None):
        def mark(i):
            if events is not None:
                events[i].record(st)
        mark(0)
        kda.chunk_prefill(**pargs)
        mark(1)
        t = sp["t"]
        kda.recurrent_verify(t["q"], t["k"], t["v"], t["g"], t["b"], sp["pool"], sp["ckpt"],
                             o=sp["o"], u_rec=sp["u_rec"], kg_rec=sp["kg_rec"])
        mark(2)
        kda.commit(sp["pool"], sp["ckpt"], sp["acc"], sp["u_rec"], sp["kg_rec"])
        mark(3)
        kda.commit_align(sp["pool"], sp["align_table"], sp["align_pos"], sp["acc"], sp["align_bs"],
                         sp["u_rec"], sp["kg_rec"])
        mark(4)
        kda.conv_state_update(sp["conv"], sp["conv_keep"], sp["ckpt"], sp["ckpt"], sp["acc"])
        mark(5)
        kda.state_copy(sp["pool"], sp["src"], sp["dst"])
        mark(6)
        kda.conv_state_update(sp["conv"], sp["conv_keep"], sp["dst"], sp["src"], sp["zero_shift"])
        mark(7)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    # ---- warm pass: K steps back to back, wall-clock bracketed
    evs = [[ev() for _ in range(len(calls) + 1)] for _ in range(a.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(a.steps):
        step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = {c: np.array([evs[s][i].elapsed_time(evs[s][i + 1]) for s in range(a.steps)])
           for i, c in enumerate(calls)}
    ms = {c: float(per[c].mean()) for c in calls}
    ms_step = wall / a.steps * 1e3
    # ---- flushed pass: before every step, outside its timed calls, the
    #      checkpoints the commits overwrite are restored and a 512 MiB write
    #      evicts L2 and the MALL
    cold = None
    if cold_steps > 0:
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        cevs = [[ev() for _ in range(len(calls) + 1)] for _ in range(cold_steps)]
        for s in range(cold_steps):
            sp["pool"].index_copy_(0, ck_long, pristine)
            scratch.fill_(s & 0xFF)
            step(cevs[s])
        torch.cuda.synchronize()
        cold = {c: np.array([cevs[s][i].elapsed_time(cevs[s][i + 1]) for s in range(cold_steps)])
                for i, c in enumerate(calls)}
        del scratch
    # Informational legs, outside the step and `value`: the same prefill
    # kernels on the varlen batch, where 16 sequences give the scan 16x more
    # independent chains than the single-layer workload's one, and on the
    # long-context sequence (2048 serial chunks, a snapshot every 64); the
    # speculative-decoding loop in its own order, and on a small batch eager
    # against a replayed HIP graph.
    varlen = long_ctx = loop = graph_loop = None
    if not a.no_varlen:
        loop = decode_loop_leg(sp, st)
        try:
            graph_loop = graph_loop_leg(dev)
        except RuntimeError as e:   # informational: a failed capture must not cost the bench line
            graph_loop = {"error": str(e)[:200]}
        varlen = time_leg(dev, st, wl.varlen_prefill("f32"), "varlen prefill, pool initial states, "
                                                              "one snapshot per sequence")
        long_ctx = time_leg(dev, st, wl.long_prefill(), "long-context prefill, zero initial state, "
                                                         "35 snapshots")
    if a.traffic_calibration:
        ck = sp["case"]["ckpt_slots"]
        fresh = sorted(set(range(sp["case"]["n_slots"])) - set(ck.tolist()))[:len(ck)]
        kda.state_copy(sp["pool"], i32(ck, dev), i32(fresh, dev))
        torch.cuda.synchronize()

    # achievable-bandwidth reference: a plain 1 GiB device-to-device copy
    # (torch's copy kernel), read + write counted; context only, the roofline
    # fractions are taken against the published 8 TB/s
    ref_src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    ref_dst = torch.empty_like(ref_src)
    ref_src.fill_(1)
    ref_dst.copy_(ref_src)
    e0, e1 = ev(), ev()
    torch.cuda.synchronize()
    e0.record(st)
    for _ in range(5):
        ref_dst.copy_(ref_src)
    e1.record(st)
    torch.cuda.synchronize()
    ref_ms = e0.elapsed_time(e1) / 5
    hbm_reference = {"copy_bytes": 2 << 30, "ms": ref_ms, "GBps": (2 << 30) / (ref_ms * 1e-3) / 1e9,
                     "note": "1 GiB device-to-device copy, read + write counted"}
    del ref_src, ref_dst

    def spread(x):
        return {"median": float(np.median(x)), "p10": float(np.percentile(x, 10)),
                "p90": float(np.percentile(x, 90))}

    # value and the per-call figures: the flushed pass's medians (the warm
    # pass's means beside them)
    sel = {c: (float(np.median(cold[c])) if cold is not None else ms[c]) for c in calls}
    basis = ("median of %d flushed steps (L2 and MALL evicted and checkpoints restored before each "
             "step, outside the timed calls)" % cold_steps) if cold is not None else \
        "mean of %d warm steps" % a.steps
    p_s = sel["prefill"] * 1e-3
    tokens_per_s = T / p_s
    state_calls = ("verify", "commit", "commit_align", "conv_compact", "copy", "conv_fork")
    gbs = {c: sp["bytes"][c] / (sel[c] * 1e-3) / 1e9 for c in state_calls}
    dominant = max(calls, key=lambda c: sel[c])
    copy_ratio = committed_copy_traffic_ratio()
    if dominant == "prefill":
        achieved = p_bytes / p_s / 1e9
        traffic, traffic_src = measured_prefill_traffic()
        roof = {"kernel": PREFILL_KERNELS[False],
                "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                "frac": achieved * 1e9 / HBM_PEAK, "traffic": traffic, "traffic_source": traffic_src,
                # the same call's measured HBM bytes over its time: how busy HBM actually is
                "traffic_GBps": None if traffic is None else traffic / p_s / 1e9,
                "traffic_frac": None if traffic is None else traffic / p_s / HBM_PEAK,
                "algorithmic_bytes_per_launch": p_bytes, "algorithmic_flop_per_launch": p_flops,
                "mfma_frac": p_flops / p_s / BF16_PEAK, "avg_launch_ms": sel["prefill"],
                "timing": basis}
    else:
        achieved = gbs[dominant]
        roof = {"kernel": f"kda_{dominant}", "bound": "hbm", "achieved": achieved,
                "peak": HBM_PEAK / 1e9, "unit": "GB/s", "frac": achieved * 1e9 / HBM_PEAK,
                "traffic": None, "traffic_source": "none: not taken for this kernel",
                "algorithmic_bytes_per_launch": sp["bytes"][dominant], "avg_launch_ms": sel[dominant],
                "timing": basis}
    out = {
        "metric": METRIC, "value": tokens_per_s, "unit": "tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "single-layer KDA prefill T=8229 H=32 d_k=d_v=128 chunk=64 bf16 "
                               "fp32-pool + spec-decode verify/commit/fork n_req=256 L=8 H=32 "
                               "+ align-mode commit (64-token blocks) + conv-state compaction/fork "
                               "(3 x 4096 channels, width 4, bf16)",
                   "global_batch": 1, "seq_len": T, "heads": 32, "head_dim": 128, "chunk": 64},
        "value_basis": "prefill tokens/s, T / " + basis,
        "prefill": {"ms": sel["prefill"], "ms_warm_mean": ms["prefill"], "ms_warm_spread": spread(per["prefill"]),
                    "tokens_per_s": tokens_per_s, "tokens_per_s_warm": T / (ms["prefill"] * 1e-3),
                    "hbm_GBps": p_bytes / p_s / 1e9, "hbm_frac": p_bytes / p_s / HBM_PEAK,
                    "mfma_TFLOPs": p_flops / p_s / 1e12, "mfma_frac": p_flops / p_s / BF16_PEAK},
        **{c: {"ms": sel[c], "ms_warm_mean": ms[c], "ms_warm_spread": spread(per[c]), "GBps": gbs[c],
               "hbm_frac": gbs[c] * 1e9 / HBM_PEAK,
               "hbm_frac_warm": sp["bytes"][c] / (ms[c] * 1e-3) / HBM_PEAK} for c in state_calls},
        "roofline": roof,
        "copy_hbm_traffic": None if copy_ratio is None else {
            "GBps": gbs["copy"] * copy_ratio, "hbm_frac": gbs["copy"] * copy_ratio * 1e9 / HBM_PEAK,
            "ratio": copy_ratio,
            "note": "the copy's algorithmic bytes charge every pair a full source read; the kernel reads "
                    "each of the 64 sources once for its four children, so its HBM traffic is this ratio "
                    "of the algorithmic bytes (profiles/state_paths_traffic.md, rocprofv3 FETCH_SIZE + "
                    "WRITE_SIZE; not measured in this run)"},
        "hbm_reference": hbm_reference,
        "cold": None if cold is None else {
            "note": "L2 and MALL flushed by a 512 MiB write and the checkpoints restored before each step",
            "steps": cold_steps,
            **{c: {"ms_median": float(np.median(cold[c])), "ms_p10": float(np.percentile(cold[c], 10)),
                   "ms_p90": float(np.percentile(cold[c], 90))} for c in calls}},
        "prefill_varlen": varlen,
        "prefill_long": long_ctx,
        "decode_loop": loop,
        "decode_loop_graph": graph_loop,
        "device": torch.cuda.get_device_name(0),
    }
    if cb is not None:
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
