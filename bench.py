#!/usr/bin/env python3
"""Benchmark: mixed-length paged GQA decode attention on one MI355X.

One step = one decode-attention layer: the persistent split-KV attention
kernel plus the combine kernel (``lbp_attend``), reusing one task map built
once per decode step (``lbp_plan``).  The single-launch variant
(``lbp_attend_fused``) is timed beside it as "fused_us_per_step".  Inputs are seeded synthetic tensors
already resident in HBM; layers rotate over distinct KV copies (at least
1 GB in all) so the 256 MB Infinity Cache cannot serve the KV bytes.

The headline workload is the mixed-length batch (64 requests, KV lengths
log-uniform in [256, 65536], 64 query / 8 KV heads, head_dim 128, BF16 KV in
64-token pages, 8 layers sharing one task map).  The uniform, skewed and FP8
workloads are reported in the same JSON line under "other_workloads".

Prints exactly one JSON line.
"""

from __future__ import annotations

import argparse
import concurrent.futures
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

METRIC = "µs per decode-attention step + achieved KV HBM GB/s (% of peak), mixed-length"
HBM_PEAK_GBS = 8000.0
LAYERS = {"mixed": 8, "uniform": 4, "skewed": 16, "fp8": 1, "tiny": 1}
ATTEND_KERNEL = {"bf16": "attend_kernel<Bf16Kv>", "fp8_e4m3": "attend_kernel<Fp8Kv>"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attend_traffic.json")
ATTEND_SRC = os.path.join(ROOT, "load_balanced_paged_amd", "csrc", "attend_kernel.hip")
TIMED_REPLAYS = 3   # timed runs of K steps per configuration; the median is reported


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--warmup-seconds", type=float, default=1.0,
                    help="before the W warmup steps, run steps for this long (the GPU's clocks "
                         "need up to about a second of load to settle after an idle spell)")
    ap.add_argument("--settle-seconds", type=float, default=0.25,
                    help="steps run for this long before each later timing of a workload "
                         "(fused, FP8 query, kernel, verification, static sweep)")
    ap.add_argument("--workloads", default="mixed,uniform,skewed,fp8",
                    help="comma list; the first is the headline (default mixed)")
    ap.add_argument("--no-static", action="store_true", help="skip the static split-KV comparison")
    ap.add_argument("--no-fused", action="store_true",
                    help="skip the lbp_attend_fused timing (profiler runs: keeps every launch of "
                         "the attention kernel a plain one)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-verify", action="store_true",
                    help="skip the multi-token verification timings (q_len 2, 4, 6)")
    ap.add_argument("--verify-qlens", default="2,4,6",
                    help="comma list of the verification widths (query tokens per request) "
                         "timed after decode")
    ap.add_argument("--no-table3", action="store_true",
                    help="skip the six FP8-KV length mixes of the vLLM x HPC-Ops page, Table 3")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="wall-clock budget of the CPU oracle sample")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="also run one torch copy of this many MiB (counter calibration)")
    ap.add_argument("--eager", action="store_true", help="time stream launches, not a HIP graph")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# workload set-up
# ---------------------------------------------------------------------------

class Bench:
    def __init__(self, name, lbp, wcfg=None, layers=None):
        from workloads import CONFIGS, make_workload
        self.lbp = lbp
        self.name = name
        self.wcfg = wcfg if wcfg is not None else CONFIGS[name]
        self.layers = layers if layers is not None else LAYERS[name]
        t0 = time.time()
        self.wl = make_workload(self.wcfg, device="cuda", layers=self.layers)
        torch.cuda.synchronize()
        log(f"{name}: generated {self.layers} layer(s), {self.wl.total_tokens} tokens, "
            f"{self.wl.kv_bytes / 1e9:.3f} GB KV/layer in {time.time() - t0:.1f}s")
        self.cfg = lbp.make_config(self.wcfg.num_q_heads, self.wcfg.num_kv_heads, self.wcfg.batch,
                                   self.wl.page_table.shape[1], kv_dtype=self.wcfg.kv_dtype,
                                   num_workgroups=0, min_tiles_per_bin=0,
                                   sm_scale=self.wcfg.sm_scale)
        self.seq = torch.from_numpy(np.asarray(self.wl.lengths, dtype=np.int32)).cuda()
        self.table = torch.from_numpy(self.wl.page_table).cuda()
        self.outs = [torch.empty_like(l.q) for l in self.wl.layers]
        self.plans = {}

    def plan(self, policy=0, param=0):
        key = (policy, param)
        if key not in self.plans:
            lbp = self.lbp
            pb, sb = lbp.lbp_query_workspace(self.cfg, policy, param)
            plan_ws = torch.empty(pb, dtype=torch.uint8, device="cuda")
            split_ws = torch.empty(sb, dtype=torch.uint8, device="cuda")
            if policy == lbp.LBP_POLICY_DYNAMIC:
                # param > 0: the minimum-work floor F for this plan
                cfg = self.cfg
                if param > 0:
                    cfg = lbp.lbp_config.from_buffer_copy(self.cfg)
                    cfg.min_tiles_per_bin = param
                info = lbp.lbp_plan(cfg, self.seq, self.table, plan_ws)
            else:
                info = lbp.lbp_plan_static(self.cfg, policy, param, self.seq, self.table, plan_ws)
            self.plans[key] = (info, plan_ws, split_ws)
        return self.plans[key]

    def used_bins(self, F=0):
        """U, the bins with work, of the dynamic plan with floor F (header word 8)."""
        info, plan_ws, _ = self.plan(self.lbp.LBP_POLICY_DYNAMIC, F)
        return int(self.lbp.read_taskmap(plan_ws, info)["header"][3])

    def verify_setup(self, q_len):
        """Config, dynamic plan, queries and outputs for multi-token
        verification: q_len new tokens per request (the lengths already count
        them), queries [batch, q_len, Hq, 128] drawn like the decode ones."""
        if not hasattr(self, "verify"):
            self.verify = {}
        if q_len not in self.verify:
            lbp, w = self.lbp, self.wcfg
            cfg = lbp.make_config(w.num_q_heads, w.num_kv_heads, w.batch,
                                  self.wl.page_table.shape[1], kv_dtype=w.kv_dtype,
                                  num_workgroups=0, min_tiles_per_bin=0, sm_scale=w.sm_scale,
                                  q_len=q_len)
            pb, sb = lbp.lbp_query_workspace(cfg)
            plan_ws = torch.empty(pb, dtype=torch.uint8, device="cuda")
            split_ws = torch.empty(sb, dtype=torch.uint8, device="cuda")
            info = lbp.lbp_plan(cfg, self.seq, self.table, plan_ws)
            g = torch.Generator(device="cuda")
            g.manual_seed(w.seed + 7919 * q_len)
            qs = [torch.randn((w.batch, q_len, w.num_q_heads, 128), generator=g, device="cuda")
                  .to(torch.bfloat16) for _ in range(self.layers)]
            outs = [torch.empty_like(q) for q in qs]
            self.verify[q_len] = (cfg, (info, plan_ws, split_ws), qs, outs)
        return self.verify[q_len]

    def step_fn(self, policy=0, param=0, fused=False, fp8q=False, q_len=1):
        """A closure launching one attend (lbp_attend, lbp_attend_fused, or
        lbp_attend_fp8q with the layer's query in e4m3) on layer i with
        pre-marshalled arguments; q_len > 1 runs multi-token verification
        (lbp_attend, dynamic plan)."""
        import ctypes
        lbp = self.lbp
        lib = lbp.load()
        cfg, outs, vq = self.cfg, self.outs, None
        if q_len > 1:
            cfg, (info, plan_ws, split_ws), vq, outs = self.verify_setup(q_len)
        else:
            info, plan_ws, split_ws = self.plan(policy, param)
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        cfgp, infop = ctypes.byref(cfg), ctypes.byref(info)
        P = ctypes.c_void_p
        sbytes = split_ws.numel()
        args = []
        if fp8q and not hasattr(self, "q8"):
            from workloads import quantize_query_e4m3
            self.q8 = [quantize_query_e4m3(L.q) for L in self.wl.layers]
        for i, L in enumerate(self.wl.layers):
            ks = P(L.k_scale.data_ptr()) if L.k_scale is not None else None
            vs = P(L.v_scale.data_ptr()) if L.v_scale is not None else None
            q = (P(self.q8[i][0].data_ptr()), P(self.q8[i][1].data_ptr())) if fp8q else \
                (P((vq[i] if vq is not None else L.q).data_ptr()),)
            args.append((cfgp, infop, P(plan_ws.data_ptr())) + q +
                        (P(L.k_cache.data_ptr()), P(L.v_cache.data_ptr()), ks, vs,
                         P(split_ws.data_ptr()), sbytes, P(outs[i].data_ptr()), stream))

        fn = lib.lbp_attend_fp8q if fp8q else lib.lbp_attend_fused if fused else lib.lbp_attend

        def run(i):
            st = fn(*args[i % self.layers])
            if st != 0:
                raise RuntimeError(f"attend: {lbp.status_name(st)}")
        return run, args

    # -- timing ------------------------------------------------------------

    def warm(self, seconds):
        run, _ = self.step_fn()
        t0 = time.time()
        i = 0
        while time.time() - t0 < seconds:
            for _ in range(4):
                run(i)
                i += 1
            torch.cuda.synchronize()

    def time_steps(self, steps, warmup, policy=0, param=0, eager=False, fused=False, fp8q=False,
                   q_len=1):
        run, _ = self.step_fn(policy, param, fused, fp8q, q_len)
        for i in range(warmup):
            run(i)
        torch.cuda.synchronize()
        mode = "eager"
        graph = None
        if not eager:
            try:
                graph = torch.cuda.CUDAGraph()
                s = torch.cuda.Stream()
                s.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(s):
                    run_g, _ = self.step_fn(policy, param, fused, fp8q, q_len)   # capture stream
                    with torch.cuda.graph(graph, stream=s):
                        for i in range(steps):
                            run_g(i)
                torch.cuda.current_stream().wait_stream(s)
                graph.replay()                                # untimed warm replay
                torch.cuda.synchronize()
                mode = f"hip_graph, median of {TIMED_REPLAYS} timed replays"
            except Exception as e:  # graph capture unavailable: time stream launches
                log(f"graph capture failed ({e}); timing stream launches")
                graph = None
        # TIMED_REPLAYS timed runs of exactly `steps` steps, each bracketed by
        # events and a synchronize; the median is reported
        per_step = []
        for _ in range(TIMED_REPLAYS):
            start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            start.record()
            if graph is not None:
                graph.replay()
            else:
                for i in range(steps):
                    run(i)
            end.record()
            torch.cuda.synchronize()
            per_step.append(start.elapsed_time(end) / steps)
        return statistics.median(per_step), mode

    def time_attend_kernel(self, steps):
        """Average duration of the persistent attention kernel alone:
        `steps` lbp_attend_partials launches over the rotating layers captured
        in one HIP graph, timed with HIP events on the capture stream around
        a replay (so launches are back to back, as under the profiler, and
        the host's launch cost stays out).  Returns (mean µs per launch,
        spread over `reps` replays as (min, max))."""
        import ctypes
        lbp = self.lbp
        lib = lbp.load()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            _, args = self.step_fn()          # marshalled on the capture stream
            with torch.cuda.graph(g, stream=s):
                for i in range(steps):
                    st = lib.lbp_attend_partials(*args[i % self.layers])
                    if st != 0:
                        raise RuntimeError(lbp.status_name(st))
        torch.cuda.current_stream().wait_stream(s)
        g.replay()
        torch.cuda.synchronize()
        per = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) * 1e3 / steps)
        return float(np.mean(per)), float(min(per)), float(max(per))

    def time_prologue(self, steps):
        """lbp_prologue for the workload's batch (one new token per request into
        layer 0's cache), HIP-graph timed; FP8 query and cache for FP8 KV."""
        import ctypes
        from workloads import make_prologue_inputs, rope_cos_sin_table
        lbp = self.lbp
        lib = lbp.load()
        w = self.wcfg
        B, Hq, Hkv = w.batch, w.num_q_heads, w.num_kv_heads
        fp8 = w.kv_dtype == "fp8_e4m3"
        qkv, qw, kw = make_prologue_inputs(B, Hq, Hkv, w.seed, device="cuda")
        cs = rope_cos_sin_table(int(max(self.wl.lengths)), device="cuda")
        L = self.wl.layers[0]
        q_out = torch.empty((B, Hq, 128), dtype=torch.uint8 if fp8 else torch.bfloat16,
                            device="cuda")
        q_scale = torch.empty((B, Hq), dtype=torch.float32, device="cuda") if fp8 else None
        a = lbp.lbp_prologue_args()
        P = lambda t: t.data_ptr() if t is not None else None   # noqa: E731
        a.qkv, a.seq_lens, a.page_table = P(qkv), P(self.seq), P(self.table)
        a.page_table_stride = int(self.table.shape[1])
        a.q_norm_weight, a.k_norm_weight, a.rope_cos_sin = P(qw), P(kw), P(cs)
        a.max_position, a.norm_eps, a.q_fp8 = int(cs.shape[0]), 1e-6, int(fp8)
        a.q_out, a.q_scale_out = P(q_out), P(q_scale)
        a.k_cache, a.v_cache, a.k_scale, a.v_scale = (P(L.k_cache), P(L.v_cache), P(L.k_scale),
                                                      P(L.v_scale))
        cfgp, ap = ctypes.byref(self.cfg), ctypes.byref(a)

        def launch(stream):
            st = lib.lbp_prologue(cfgp, B, ap, ctypes.c_void_p(stream))
            if st != 0:
                raise RuntimeError(f"lbp_prologue: {lbp.status_name(st)}")
        for _ in range(3):
            launch(torch.cuda.current_stream().cuda_stream)
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for _ in range(steps):
                    launch(s.cuda_stream)
        torch.cuda.current_stream().wait_stream(s)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        out_row = 128 + 4 if fp8 else 256           # one head row out (codes + scale, or bf16)
        nbytes = (B * (Hq + 2 * Hkv) * 256 + B * 512     # QKV in, one cos/sin row per request
                  + B * Hq * out_row + B * 2 * Hkv * out_row)
        return {"us": round(us, 2), "bytes": nbytes, "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
                "query": "e4m3 + scale" if fp8 else "bf16"}

    def finish_spread(self, policy=0, param=0):
        """Finishing times of the attention kernel's workgroups in one traced
        launch (lbp_attend_traced, layer 0): with equal bins they should end
        together.  Times in µs from the earliest workgroup start; only
        workgroups that drained at least one descriptor count."""
        lbp = self.lbp
        info, plan_ws, split_ws = self.plan(policy, param)
        L = self.wl.layers[0]
        trace = torch.zeros(4 * info.num_bins, dtype=torch.int64, device="cuda")
        for _ in range(2):             # the second launch is the one read
            lbp.lbp_attend_traced(self.cfg, info, plan_ws, L.q, L.k_cache, L.v_cache, L.k_scale,
                                  L.v_scale, split_ws, self.outs[0], trace)
        torch.cuda.synchronize()
        t = trace.view(-1, 4).cpu().numpy()
        t = t[t[:, 3] > 0]
        end = (t[:, 1] - t[:, 0].min()) / 100.0   # 100 MHz real-time counter
        med, mx = float(np.median(end)), float(end.max())
        return {"workgroups": int(len(t)), "end_us_min": round(float(end.min()), 1),
                "end_us_median": round(med, 1), "end_us_max": round(mx, 1),
                "tail_frac": round((mx - med) / mx, 4)}

    def time_plan(self, reps=20):
        """µs per lbp_plan: `reps` plans captured in a HIP graph, as a decode
        step would launch it (eager launches here would time the host)."""
        lbp = self.lbp
        info, plan_ws, _ = self.plan()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for _ in range(reps):
                    lbp.lbp_plan(self.cfg, self.seq, self.table, plan_ws, stream=s)
        torch.cuda.current_stream().wait_stream(s)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    def check_finite(self):
        for o in self.outs:
            if not torch.isfinite(o.float()).all():
                raise RuntimeError(f"{self.name}: non-finite output")

    def free(self):
        self.plans.clear()
        self.verify = {}
        self.outs = None
        self.wl = None
        torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# read-stream reference
# ---------------------------------------------------------------------------

def read_stream_reference(lbp, gib=4, reps=5, rounds=3, warm_seconds=0.2):
    """This GPU's attainable HBM read rate for streaming traffic: the library's
    read-stream kernel over a `gib` GiB buffer, best over a few grid sizes
    and `rounds` batches of `reps` launches each (HIP events around each
    batch), after `warm_seconds` of streaming to bring the clocks up."""
    n = gib << 30
    buf = torch.empty(n, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.empty(1 << 16, dtype=torch.int32, device="cuda")
    t0 = time.time()
    while time.time() - t0 < warm_seconds:
        lbp.lbp_read_stream(buf, sink, 8192)
        torch.cuda.synchronize()
    best, best_blocks = 0.0, 0
    for blocks in (2048, 4096, 8192, 16384):
        for _ in range(rounds):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                lbp.lbp_read_stream(buf, sink, blocks)
            e1.record()
            torch.cuda.synchronize()
            gbs = reps * n / (e0.elapsed_time(e1) * 1e-3) / 1e9
            if gbs > best:
                best, best_blocks = gbs, blocks
    del buf, sink
    torch.cuda.empty_cache()
    log(f"read stream: {best:.0f} GB/s ({gib} GiB, {best_blocks} workgroups)")
    return {"gbs": round(best, 1), "bytes": n, "workgroups": best_blocks,
            "kernel": "read_stream_kernel", "pct_of_hbm_peak": round(100 * best / HBM_PEAK_GBS, 1)}


# ---------------------------------------------------------------------------
# CPU oracle baseline
# ---------------------------------------------------------------------------

def cpu_baseline(b: Bench, seconds: float):
    """The fp64 oracle, unchanged, on a time-bounded sample of layer 0's pairs.

    Pairs are visited in a seeded random order on a thread pool (one BLAS
    thread per worker); a worker starts no new pair after the deadline.  The
    rate is KV bytes of the completed pairs over the wall time.
    """
    import oracle
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    wcfg = b.wcfg
    L = np.asarray(b.wl.lengths)
    H, G = wcfg.num_kv_heads, wcfg.group
    lay = b.wl.layers[0]
    rng = np.random.default_rng(123)
    order = [(int(g), int(r)) for g, r in
             zip(*np.unravel_index(rng.permutation(H * len(L)), (H, len(L))))]
    cores = len(os.sched_getaffinity(0))
    # host copies of the whole layer (outside the timed region)
    q = oracle.attention.bf16_bits_to_f64(
        lay.q.view(torch.int16).cpu().numpy().view(np.uint16))
    kc = lay.k_cache.view(torch.int16).cpu().numpy().view(np.uint16)
    vc = lay.v_cache.view(torch.int16).cpu().numpy().view(np.uint16)
    table = b.wl.page_table
    deadline = [None]
    done = []

    def work(pair):
        if time.perf_counter() > deadline[0]:
            return
        g, r = pair
        oracle.attention.paged_decode_attention(q, kc, vc, table, L, H, wcfg.sm_scale,
                                                pairs=[(g, r)])
        done.append(pair)

    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    if ctx:
        ctx.__enter__()
    try:
        t0 = time.perf_counter()
        deadline[0] = t0 + seconds
        with concurrent.futures.ThreadPoolExecutor(cores) as ex:
            list(ex.map(work, order))
        wall = time.perf_counter() - t0
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    tokens = int(sum(L[r] for _, r in done))
    kv_bytes = tokens * wcfg.kv_bytes_per_token_head
    gbs = kv_bytes / wall / 1e9
    full_us = b.wl.kv_bytes / (gbs * 1e9) * 1e6
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{len(done)} of {H * len(L)} (KV head, request) pairs of layer 0 "
                      f"({tokens} tokens, {kv_bytes / 1e9:.3f} GB KV) in {wall:.1f}s wall; "
                      f"fp64 NumPy oracle, one pair per task on a {cores}-thread pool",
            "us_per_step_extrapolated": round(full_us, 1)}


# ---------------------------------------------------------------------------

def attend_src_sha():
    return hashlib.sha256(open(ATTEND_SRC, "rb").read()).hexdigest()[:16]


def traffic_record(workload):
    """(HBM bytes per launch, source) from the committed rocprofv3 counter
    runs on this workload (FETCH_SIZE and WRITE_SIZE, calibrated against a
    copy), if they were taken on the current attention kernel source; else
    (None, reason).  The counters are not collected in this run."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except Exception:
        return None, "no committed counter record"
    entry = rec.get(workload)
    sha = attend_src_sha()
    if not entry:
        return None, f"no committed counter record for {workload}"
    if entry.get("attend_src_sha") != sha:
        return None, (f"counters taken on attend_kernel.hip {entry.get('attend_src_sha')}, "
                      f"source is now {sha}")
    return entry.get("hbm_bytes_per_launch"), f"profiles/attend_traffic.json@{sha}"


def bench_one(name, lbp, args, headline, stream_gbs=None):
    b = Bench(name, lbp)
    res = {"workload": name}
    info, _, _ = b.plan()
    b.warm(args.warmup_seconds)
    ms, mode = b.time_steps(args.steps, args.warmup, eager=args.eager)
    b.check_finite()
    us = ms * 1e3
    gbs = b.wl.kv_bytes / (us * 1e-6) / 1e9
    res.update(us_per_step=round(us, 2), kv_gbs=round(gbs, 1),
               pct_of_hbm_peak=round(100 * gbs / HBM_PEAK_GBS, 1), timing=mode,
               pct_of_read_stream=round(100 * gbs / stream_gbs, 1) if stream_gbs else None,
               kv_bytes_per_layer=b.wl.kv_bytes, total_tokens=b.wl.total_tokens,
               workgroups=info.num_bins, layers=b.layers)
    if not args.no_fused:
        b.warm(args.settle_seconds)
        fms, _ = b.time_steps(args.steps, args.warmup, eager=args.eager, fused=True)
        res["fused_us_per_step"] = round(fms * 1e3, 2)      # lbp_attend_fused, one launch
    if b.wcfg.kv_dtype == "fp8_e4m3" and not args.no_fused:
        b.warm(args.settle_seconds)
        qms, _ = b.time_steps(args.steps, args.warmup, eager=args.eager, fp8q=True)
        res["fp8q_us_per_step"] = round(qms * 1e3, 2)       # lbp_attend_fp8q: e4m3 query
    b.warm(args.settle_seconds)
    k_mean, k_min, k_max = b.time_attend_kernel(max(20, min(args.steps, 100)))
    res["attend_kernel_us"] = {"mean": round(k_mean, 2), "min_of_replays": round(k_min, 2),
                               "max_of_replays": round(k_max, 2),
                               "timing": "HIP graph of attention-only launches "
                                         "(lbp_attend_partials), events around 3 replays"}
    res["plan_us"] = round(b.time_plan(), 2)
    res["prologue"] = b.time_prologue(min(args.steps, 100))
    if not args.no_verify:
        # multi-token verification: the same KV, q_len query tokens per request
        res["verify"] = {}
        for T in sorted({int(x) for x in args.verify_qlens.split(",") if x.strip()}):
            if T < 2:
                continue
            if b.wcfg.num_q_heads // b.wcfg.num_kv_heads * T > 64:
                continue
            b.warm(args.settle_seconds)
            vms, _ = b.time_steps(args.steps, args.warmup, eager=args.eager, q_len=T)
            vgbs = b.wl.kv_bytes / (vms * 1e-3) / 1e9
            res["verify"][f"q_len={T}"] = {"us_per_step": round(vms * 1e3, 2),
                                           "kv_gbs": round(vgbs, 1)}
    res["amortized_us_per_layer"] = round((res["plan_us"] + b.layers * us) / b.layers, 2)
    if not args.no_static:
        W = info.num_bins
        s0 = max(1, math.ceil(W / (b.wcfg.num_kv_heads * b.wcfg.batch)))
        static = {}
        for S in sorted({s0, 1, 2, 4, 8, 16, 32, 64}):
            b.warm(args.settle_seconds)
            sms, _ = b.time_steps(min(args.steps, 50), 2, lbp.LBP_POLICY_STATIC_SPLITS, S,
                                  eager=args.eager)
            static[S] = sms * 1e3
        best = min(static, key=static.get)
        res["finish_spread"] = {"dynamic": b.finish_spread(),
                                "static_grid_matched": b.finish_spread(
                                    lbp.LBP_POLICY_STATIC_SPLITS, s0)}
        res["static_splits"] = {"S_grid_matched": s0, "us_grid_matched": round(static[s0], 2),
                                "best_S": best, "us_best": round(static[best], 2),
                                "dynamic_speedup_vs_grid_matched": round(static[s0] / us, 3),
                                "dynamic_speedup_vs_best": round(static[best] / us, 3),
                                "us_by_S": {str(k): round(v, 2) for k, v in static.items()}}
    if headline and not args.no_cpu_baseline:
        log(f"{name}: CPU oracle baseline ({args.cpu_seconds:.0f}s budget)")
        res["cpu_baseline"] = cpu_baseline(b, args.cpu_seconds)
    traffic, traffic_source = traffic_record(name)
    achieved = b.wl.kv_bytes / (k_mean * 1e-6) / 1e9
    res["roofline"] = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                       "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                       "traffic": traffic, "traffic_source": traffic_source,
                       "kernel": ATTEND_KERNEL[b.wcfg.kv_dtype],
                       "algorithmic_bytes_per_launch": b.wl.kv_bytes,
                       "avg_kernel_us": round(k_mean, 2),
                       "read_stream_gbs": stream_gbs,
                       "frac_of_read_stream": round(achieved / stream_gbs, 4) if stream_gbs else None}
    log(f"{name}: {us:.1f} us/step ({mode}), {gbs:.0f} GB/s KV, kernel {k_mean:.1f} us "
        f"({achieved:.0f} GB/s), plan {res['plan_us']:.1f} us")
    b.free()
    return res


# vLLM x HPC-Ops page, Table 3 (H20, FP8 KV): dynamic ms, static split-KV ms,
# dynamic-vs-static ratio per A x B mix.  Context only: other hardware.
H20_TABLE3 = {
    "64x0.5K": (0.013, 0.013, 1.00),
    "64x4K": (0.033, 0.043, 1.32),
    "32x0.125K+32x4K": (0.020, 0.033, 1.59),
    "2x32K+30x4K": (0.032, 0.056, 1.76),
    "1x64K+15x4K": (0.042, 0.097, 2.32),
    "1x128K+31x4K": (0.063, 0.186, 2.95),
}
ROTATE_BYTES = 1 << 30     # rotating KV set per mix: 4x the 256 MB Infinity Cache


def bench_table3(lbp, args):
    """Dynamic against static split-KV on the six Table 3 mixes (8/1 heads, FP8 KV)."""
    from workloads import TABLE3
    out = {}
    for mix, wcfg in TABLE3.items():
        tokens = sum(wcfg.fixed_lengths)
        kv = tokens * wcfg.num_kv_heads * wcfg.kv_bytes_per_token_head
        layers = max(1, min(128, math.ceil(ROTATE_BYTES / kv)))
        b = Bench(wcfg.name, lbp, wcfg=wcfg, layers=layers)
        info, _, _ = b.plan()
        b.warm(args.settle_seconds)
        ms, mode = b.time_steps(args.steps, args.warmup, eager=args.eager)
        b.warm(args.settle_seconds)
        fms, _ = b.time_steps(args.steps, args.warmup, eager=args.eager, fused=True)
        b.warm(args.settle_seconds)
        qms, _ = b.time_steps(args.steps, args.warmup, eager=args.eager, fp8q=True)
        b.check_finite()
        us = ms * 1e3
        W = info.num_bins
        s_grid = max(1, math.ceil(W / (wcfg.num_kv_heads * wcfg.batch)))
        static = {}
        for S in sorted({s_grid, 1, 2, 4, 8, 16, 32, 64}):
            b.warm(args.settle_seconds)
            sms, _ = b.time_steps(min(args.steps, 50), 2, lbp.LBP_POLICY_STATIC_SPLITS, S,
                                  eager=args.eager)
            static[S] = sms * 1e3
        best = min(static, key=static.get)
        # the minimum-work floor F (tiles per bin) of the dynamic plan; the
        # library's default is 1 (no floor), and F binds only while
        # T <= (F - 1) W.  The default plan runs first before each F, so
        # that no F is timed straight after another plan's timing.
        by_f = {}
        for F in (1, 2, 4):
            b.warm(args.settle_seconds)
            fms_f, _ = b.time_steps(min(args.steps, 50), 2, lbp.LBP_POLICY_DYNAMIC, F,
                                    eager=args.eager)
            by_f[F] = {"us_per_step": round(fms_f * 1e3, 2), "bins_used": b.used_bins(F)}
        h20 = H20_TABLE3[mix]
        out[mix] = {
            "us_per_step": round(us, 2), "fused_us_per_step": round(fms * 1e3, 2),
            "fp8q_us_per_step": round(qms * 1e3, 2),
            "kv_gbs": round(kv / (us * 1e-6) / 1e9, 1), "kv_bytes_per_layer": kv,
            "layers": layers, "timing": mode,
            "static_S_grid_matched": s_grid, "static_us_grid_matched": round(static[s_grid], 2),
            "static_best_S": best, "static_us_best": round(static[best], 2),
            "dynamic_vs_static_grid_matched": round(static[s_grid] / us, 3),
            "dynamic_vs_static_best": round(static[best] / us, 3),
            "static_us_by_S": {str(k): round(v, 2) for k, v in static.items()},
            "dynamic_by_min_tiles_per_bin": {str(k): v for k, v in by_f.items()},
            "h20_context": {"dynamic_us": h20[0] * 1e3, "static_us": h20[1] * 1e3,
                            "dynamic_vs_static": h20[2]},
        }
        log(f"table3 {mix}: dynamic {us:.1f} us, static S={s_grid} {static[s_grid]:.1f} us "
            f"({static[s_grid] / us:.2f}x), best static S={best} {static[best]:.1f} us "
            f"({static[best] / us:.2f}x); H20: {h20[2]:.2f}x")
        b.free()
    return out


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path is "
              "single-GPU by design and has no multi-GPU mode", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import load_balanced_paged_amd as lbp
    lbp.load()
    names = [n.strip() for n in args.workloads.split(",") if n.strip()]
    torch.cuda.synchronize()

    if args.copy_calib_mib:
        n = args.copy_calib_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {n} bytes read + {n} bytes written")
        del src, dst

    stream = read_stream_reference(lbp)
    results = [bench_one(n, lbp, args, headline=(i == 0), stream_gbs=stream["gbs"])
               for i, n in enumerate(names)]
    head = results[0]
    wcfg = __import__("workloads").CONFIGS[names[0]]
    out = {
        "metric": METRIC,
        "value": head["kv_gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_seconds": args.warmup_seconds,
        "ms_per_step": round(head["us_per_step"] / 1e3, 5),
        "us_per_step": head["us_per_step"],
        "pct_of_hbm_peak": head["pct_of_hbm_peak"],
        "pct_of_read_stream": head["pct_of_read_stream"],
        "read_stream": stream,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wcfg.kv_dtype == "bf16" else "fp8_e4m3-kv/bf16-q",
        "data": "synthetic",
        "config": {
            "workload": (f"{names[0]}: batch {wcfg.batch}, "
                         + ("KV lengths log-uniform [%d, %d]" % (wcfg.length_lo, wcfg.length_hi)
                            if wcfg.lengths_kind == "loguniform" else wcfg.lengths_kind)
                         + f" (seed {wcfg.seed}), {wcfg.num_q_heads} query / {wcfg.num_kv_heads}"
                         f" KV heads, head_dim 128, {wcfg.kv_dtype} paged KV (page 64), "
                         f"{head['layers']} layers sharing one task map"),
            "batch": wcfg.batch, "num_q_heads": wcfg.num_q_heads,
            "num_kv_heads": wcfg.num_kv_heads, "head_dim": 128, "page_size": 64,
            "layers": head["layers"], "total_tokens": head["total_tokens"],
            "kv_bytes_per_layer": head["kv_bytes_per_layer"], "workgroups": head["workgroups"],
            "min_tiles_per_bin": 1, "timing": head["timing"],
        },
        "roofline": head["roofline"],
        "plan_us": head["plan_us"],
        "amortized_us_per_layer": head["amortized_us_per_layer"],
        "attend_kernel_us": head["attend_kernel_us"],
    }
    for k in ("fused_us_per_step", "fp8q_us_per_step", "prologue", "verify"):
        if k in head:
            out[k] = head[k]
    if "static_splits" in head:
        out["static_splits"] = head["static_splits"]
        out["finish_spread"] = head["finish_spread"]
    if "cpu_baseline" in head:
        out["cpu_baseline"] = head["cpu_baseline"]
    if len(results) > 1:
        out["other_workloads"] = {r["workload"]: {k: v for k, v in r.items() if k != "workload"}
                                  for r in results[1:]}
    if not args.no_table3:
        out["table3"] = {
            "workload": "vLLM x HPC-Ops page Table 3 A x B mixes, FP8 e4m3 KV + fp32 scales, "
                        "8 query / 1 KV head, head_dim 128, page 64",
            "mixes": bench_table3(lbp, args),
        }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
