#!/usr/bin/env python3
"""Benchmark of the fused matmul + tensor-parallel collective path on one MI355X.

A step is one TP8 + sequence-parallel MLP pass of one rank at LLaMA2-70B shapes:
  ALL_GATHER_MATMUL     8 shards of 512 x 8192 gathered to G 4096 x 8192, G @ W
                        with W 8192 x 7168 (fused gate/up, 2 * 28672 / 8)
  MATMUL_REDUCE_SCATTER X 4096 x 3584 @ W 3584 x 8192, the 8 ranks' partials
                        reduce-scattered to this rank's 512 x 8192 slice
both bf16, split into `--split` m-chunks.  The other ranks' shards and partial
sums are seeded buffers in the same HBM.  Prints one JSON line on stdout
(progress goes to stderr).  Before the W warmup steps, untimed steps run for
--prewarm-s seconds (default 0.5) so that the K timed steps see the GPU at its
steady clocks; the JSON line reports them under "prewarm".

    python bench.py [--steps K] [--warmup W] [--split S] [--prewarm-s T] [--no-cpu-baseline]
                    [--operands constant]   (clock diagnostic, not a benchmark figure)
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "per-rank GEMM+reduce TFLOP/s & % bf16 MFMA peak at LLaMA2-70B TP8 shapes"


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "gemm_ring_chunks_llama70b_tp8_sp_step_hbm_traffic.md")
KERNEL_SOURCE = os.path.join(ROOT, "tensor_gemm_collective_amd", "csrc", "kernels.hip")


def measured_traffic():
    """HBM bytes per matmul launch from the committed rocprofv3 counter summary, or
    None when kernels.hip has changed since those counters were taken."""
    import hashlib
    try:
        fields = {}
        for line in open(TRAFFIC_SUMMARY):
            if ":" in line and not line.startswith(("#", "|", " ", "`")):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
        digest = hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()
        if fields.get("kernels_sha256") != digest:
            return None
        return float(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def make_inputs(torch, tgc, synth, split, dev):
    ag = synth.WORKLOADS["llama70b_ag"]
    rs = synth.WORKLOADS["llama70b_rs"]
    world, rank = 8, 0
    bf16 = torch.bfloat16
    inp = {"world": world, "rank": rank, "ag": ag, "rs": rs}
    shard = ag.m // world
    shards = [synth.normal(ag.wid, synth.T_PEER, r, (shard, ag.k), ag.x_sigma, "bf16") for r in range(world)]
    inp["ag_shards_cpu"] = shards
    inp["ag_x"] = shards[rank].to(dev)
    inp["ag_peers"] = [None if r == rank else shards[r].to(dev) for r in range(world)]
    inp["ag_w_cpu"] = synth.normal(ag.wid, synth.T_W, 0, (ag.k, ag.n), ag.w_sigma, "bf16")
    inp["ag_w"] = inp["ag_w_cpu"].to(dev)
    inp["ag_y"] = torch.empty((ag.m, ag.n), dtype=bf16, device=dev)
    need = tgc.workspace_bytes(tgc.OP_ALLGATHER_MATMUL, ag.m, ag.n, ag.k, tgc.COC_BF16, world, split)
    inp["ag_ws"] = torch.empty(need, dtype=torch.uint8, device=dev)

    b = rs.m // world
    inp["rs_x_cpu"] = synth.normal(rs.wid, synth.T_X, rank, (rs.m, rs.k), rs.x_sigma, "bf16")
    inp["rs_w_cpu"] = synth.normal(rs.wid, synth.T_W, rank, (rs.k, rs.n), rs.w_sigma, "bf16")
    inp["rs_x"] = inp["rs_x_cpu"].to(dev)
    inp["rs_w"] = inp["rs_w_cpu"].to(dev)
    peers, peers_cpu = [], []
    for r in range(world):
        if r == rank:
            peers.append(None)
            peers_cpu.append(None)
            continue
        sl = synth.normal(rs.wid, synth.T_PEER, r, (b, rs.n), rs.peer_sigma, "bf16")
        full = torch.full((rs.m, rs.n), float("nan"), dtype=bf16, device=dev)  # rows never read
        full[rank * b:(rank + 1) * b] = sl.to(dev)
        peers.append(full)
        peers_cpu.append(sl)
    inp["rs_peers"] = peers
    inp["rs_peer_slices_cpu"] = peers_cpu
    inp["rs_y"] = torch.empty((b, rs.n), dtype=bf16, device=dev)
    inp["rs_part"] = torch.empty((rs.m, rs.n), dtype=bf16, device=dev)
    return inp


def sample_clock(step, torch, seconds=1.0, batch=40, per_batch=5, period=0.003):
    """GFX clock and socket power read through amdsmi while steps run back to back for
    `seconds` s: each round queues `batch` steps (tens of ms of GPU work), reads the
    clock `per_batch` times `period` s apart while the GPU works through them, then
    synchronises.  One thread throughout.  None when amdsmi is unavailable."""
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        h = amdsmi.amdsmi_get_processor_handles()[0]
        info = amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX)
        limit = amdsmi.amdsmi_get_power_info(h).get("power_limit")
    except Exception as e:   # no amdsmi, or no access to the device's metrics
        log(f"clock sampling unavailable: {e}")
        return None
    clk, pw = [], []
    for _ in range(100):   # reach the load's clock before sampling
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(batch):
            step()
        for _ in range(per_batch):
            time.sleep(period)
            c = amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX).get("clk")
            p = amdsmi.amdsmi_get_power_info(h).get("current_socket_power")
            if isinstance(c, (int, float)):
                clk.append(c)
            if isinstance(p, (int, float)):
                pw.append(p)
        torch.cuda.synchronize()
    try:
        amdsmi.amdsmi_shut_down()
    except Exception:
        pass
    if not clk:
        return None
    mean = sum(clk) / len(clk)
    med = sorted(clk)[len(clk) // 2]   # robust to a read that catches the GPU between kernels
    out = {"source": f"amdsmi GFX clock, {per_batch} reads {period * 1e3:g} ms apart while each batch of "
                     f"{batch} queued steps runs, for {seconds:g} s after the timed region",
           "samples": len(clk), "mhz_median": med, "mhz_mean": round(mean, 1), "mhz_min": min(clk),
           "mhz_max": max(clk), "mhz_rated_max": info.get("max_clk"),
           "bf16_peak_at_median_clock_tflops": round(256 * 4096 * med * 1e6 / 1e12, 1)}
    if pw:
        out["socket_power_w_mean"] = round(sum(pw) / len(pw), 1)
    if isinstance(limit, (int, float)) and limit > 0:
        out["power_limit_w"] = round(limit / 1e6, 1)
    return out


def run_mfma_loop(torch, tgc, dev, iters=4000, reps=20):
    """The MFMA-rate diagnostic (coc_diag_mfma_loop): v_mfma_f32_32x32x16_bf16
    on register operands, 8 waves per CU (as the ring matmul), random N(0,1)
    operands against one repeated value; launch time by events, then the clock
    and socket power amdsmi reads while it runs.  One JSON line."""
    props = torch.cuda.get_device_properties(dev)
    wgs = 2 * props.multi_processor_count   # two 4-wave workgroups per CU
    g = torch.Generator(device=dev).manual_seed(7)
    kinds = {"random": torch.randn(1 << 15, generator=g, device=dev).to(torch.bfloat16),
             "constant": torch.full((1 << 15,), 1.0, device=dev, dtype=torch.bfloat16)}
    out = torch.empty(wgs * 256, device=dev, dtype=torch.float32)
    res = {"diagnostic": "MFMA register loop: v_mfma_f32_32x32x16_bf16, 8 independent accumulators per wave, "
                         "operands in registers, no memory traffic",
           "workgroups": wgs, "waves_per_cu": 8, "iters": iters}
    for name, ops in kinds.items():
        def launch():
            return tgc.diag_mfma_loop(ops, out, wgs, iters)
        t_end = time.perf_counter() + 0.5
        while time.perf_counter() < t_end:   # reach the load's clock
            for _ in range(20):
                launch()
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        flops = sum(launch() for _ in range(reps))
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        res[name] = {"launch_ms": round(ms, 4), "tflops": round(flops / reps / (ms * 1e-3) / 1e12, 1),
                     "gpu_clock": sample_clock(launch, torch, seconds=1.0, batch=40)}
        log(f"mfma loop, {name} operands: {res[name]['tflops']} TFLOP/s")
    print(json.dumps(res), flush=True)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


STAMP_RECORDS = 1 << 16


def stamp_buffer(torch, dev):
    """Device buffer for the kernels' activity records (layout in include/coc.h)."""
    return torch.zeros(3 * STAMP_RECORDS, dtype=torch.int64, device=dev)


def stamped(torch, tgc, buf, fn):
    """Run fn once with the activity records on; returns (kind, chunk, start_us,
    end_us) per record written (the device counter runs at 100 MHz)."""
    buf.zero_()
    torch.cuda.synchronize()
    tgc.profile_stamps(buf)
    try:
        fn()
        torch.cuda.synchronize()
        n = tgc.profile_stamp_count()
    finally:
        tgc.profile_stamps(None)
    h = buf[:3 * n].cpu().numpy().reshape(n, 3)
    return [((int(w) & 255) - 1, (int(w) >> 8) & 255, t0 / 100.0, t1 / 100.0) for w, t0, t1 in h if w != 0]


def _union(iv):
    out = []
    for a, b in sorted(iv):
        if out and a <= out[-1][1]:
            out[-1][1] = max(out[-1][1], b)
        else:
            out.append([a, b])
    return out


def overlap_of(recs, comm_bytes):
    """The Overlap blog's profiler view of one op call, from the kernels' own
    activity records: the matmul's span (first tile started to last tile
    stored), the communication's active time (union of the reduce / gather
    workgroups' intervals, waiting excluded), how much of it falls inside the
    matmul's span (hidden) and outside it (exposed)."""
    mm = [(a, b) for k, c, a, b in recs if k == 0]
    comm = _union([(a, b) for k, c, a, b in recs if k in (1, 2)])
    active = sum(b - a for a, b in comm)
    if not mm:
        return {"comm_active_us": round(active, 2), "comm_hidden_us": 0.0, "comm_exposed_us": round(active, 2)}
    s0, s1 = min(a for a, b in mm), max(b for a, b in mm)
    hidden = sum(max(0.0, min(b, s1) - max(a, s0)) for a, b in comm)
    return {
        "matmul_span_us": round(s1 - s0, 2),
        "comm_active_us": round(active, 2),
        "comm_hidden_us": round(hidden, 2),
        "comm_exposed_us": round(active - hidden, 2),
        "overlap_frac": round(hidden / active, 4) if active > 0 else None,
        "comm_gbs_active": round(comm_bytes / (active * 1e-6) / 1e9, 1) if active > 0 else None,
    }


def mean_dicts(ds):
    keys = [k for k in ds[0] if all(isinstance(d.get(k), (int, float)) for d in ds)]
    return {k: round(sum(d[k] for d in ds) / len(ds), 4) for k in keys}


def serial_parts(torch, tgc, fn, iters=10):
    """Per-call launch time of the matmul and of the communication kernels of
    fn (the serial, split-1 form: each runs alone), from the library's
    per-launch events."""
    fn()
    torch.cuda.synchronize()
    tgc.profile_enable(True)
    tgc.profile_read()
    for _ in range(iters):
        fn()
    torch.cuda.synchronize()
    pr = tgc.profile_read()
    tgc.profile_enable(False)
    return pr["gemm"]["ms"] / iters, (pr["reduce"]["ms"] + pr["gather"]["ms"]) / iters


def flops_of(inp):
    ag, rs = inp["ag"], inp["rs"]
    return 2.0 * ag.m * ag.n * ag.k, 2.0 * rs.m * rs.n * rs.k


def blas_threads():
    """Threads the host BLAS (numpy's matmul) uses."""
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        return len(os.sched_getaffinity(0))


def cpu_baseline(inp, frac, min_seconds=10.0):
    """The oracle on the same step with m scaled by `frac` (all n and k), repeated
    until at least `min_seconds` have passed; the rate is the mean over the passes."""
    import numpy as np

    import oracle

    threads = blas_threads()

    def f64(t):
        return oracle.decode(t.contiguous().view(__import__("torch").int16).numpy().view(np.uint16), "bf16")

    ag, rs, world, rank = inp["ag"], inp["rs"], inp["world"], inp["rank"]
    shard_rows = max(1, int(ag.m // world * frac))
    slice_rows = max(1, int(rs.m // world * frac))
    b = rs.m // world
    rows = np.concatenate([np.arange(r * b, r * b + slice_rows) for r in range(world)])

    def one_pass():
        # ALL_GATHER_MATMUL on the first `shard_rows` rows of every shard
        shards = [f64(s[:shard_rows]) for s in inp["ag_shards_cpu"]]
        y_ag, _ = oracle.allgather_matmul(shards, f64(inp["ag_w_cpu"]))
        # MATMUL_REDUCE_SCATTER on the first `slice_rows` rows of every rank's slice
        x = f64(inp["rs_x_cpu"][rows])
        peers = []
        for r in range(world):
            if r == rank:
                peers.append(None)
                continue
            full = np.zeros((world * slice_rows, rs.n))
            full[rank * slice_rows:(rank + 1) * slice_rows] = f64(inp["rs_peer_slices_cpu"][r][:slice_rows])
            peers.append(full)
        y_rs, _ = oracle.matmul_reduce_scatter(x, f64(inp["rs_w_cpu"]), peers, rank)
        assert np.all(np.isfinite(y_ag)) and np.all(np.isfinite(y_rs))

    passes = 0
    t0 = time.perf_counter()
    while True:
        one_pass()
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    flops = passes * (2.0 * world * shard_rows * ag.n * ag.k + 2.0 * world * slice_rows * rs.n * rs.k)
    return {
        "value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": f"the same step with m scaled by {frac:g} (AG {world}x{shard_rows} gathered rows, "
                  f"RS {world}x{slice_rows} rows), all n and k; float64 numpy oracle incl. decoding the "
                  f"bf16 inputs; {passes} passes in {dt:.2f} s",
    }


def run_cpu_configs(synth, min_seconds=3.0, target_flops=6e10):
    """The oracle (host, float64 numpy) on every workload: a bounded sample of
    the op's rows with all n and k (about target_flops of matmul per pass),
    repeated until min_seconds have passed, inputs decoded from their stored
    format inside the timed passes.  One JSON line per workload on stderr; no
    GPU is used."""
    import numpy as np

    import oracle

    def f64(t, dt):
        if dt == "f32":
            return t.numpy().astype(np.float64)
        if dt == "i8":
            return t.numpy().astype(np.float64)
        return oracle.decode(t.contiguous().view(__import__("torch").int16).numpy().view(np.uint16), dt)

    threads = blas_threads()
    for wl in synth.WORKLOADS.values():
        T, dt, n, k = wl.world, wl.dtype, wl.n, wl.k
        per = max(1, int(target_flops / (2.0 * n * k)))
        if wl.op in ("all_reduce", "w8a16"):
            rows = min(wl.m, per)
            x = synth.normal(wl.wid, synth.T_X, 0, (rows, k), wl.x_sigma, dt)
            peers = [None] + [synth.normal(wl.wid, synth.T_PEER, r, (rows, n), wl.peer_sigma, dt) for r in range(1, T)]
            if wl.op == "w8a16":
                q = synth.integers(wl.wid, synth.T_W, 0, (k, n), -127, 127, "i8")
                sc = synth.uniform(wl.wid, synth.T_SCALES, 0, (n,), 0.001, 0.02, "f16")

                def one_pass():
                    return oracle.matmul_all_reduce_w8a16(f64(x, dt), f64(q, "i8"), f64(sc, "f16"), "per_channel", 0,
                                                         [None] + [f64(p, dt) for p in peers[1:]], 0)[0]
            else:
                w = synth.normal(wl.wid, synth.T_W, 0, (k, n), wl.w_sigma, dt)

                def one_pass():
                    return oracle.matmul_all_reduce(f64(x, dt), f64(w, dt), [None] + [f64(p, dt) for p in peers[1:]],
                                                    0)[0]
        elif wl.op == "reduce_scatter":
            rl = max(1, min(wl.m // T, per // T))
            rows = T * rl
            x = synth.normal(wl.wid, synth.T_X, 0, (rows, k), wl.x_sigma, dt)
            w = synth.normal(wl.wid, synth.T_W, 0, (k, n), wl.w_sigma, dt)
            peers = [None] + [synth.normal(wl.wid, synth.T_PEER, r, (rows, n), wl.peer_sigma, dt) for r in range(1, T)]

            def one_pass():
                return oracle.matmul_reduce_scatter(f64(x, dt), f64(w, dt), [None] + [f64(p, dt) for p in peers[1:]],
                                                    0)[0]
        else:   # allgather
            rl = max(1, min(wl.m // T, per // T))
            rows = T * rl
            shards = [synth.normal(wl.wid, synth.T_PEER, r, (rl, k), wl.x_sigma, dt) for r in range(T)]
            w = synth.normal(wl.wid, synth.T_W, 0, (k, n), wl.w_sigma, dt)

            def one_pass():
                return oracle.allgather_matmul([f64(sh, dt) for sh in shards], f64(w, dt))[0]
        passes, t0 = 0, time.perf_counter()
        while True:
            y = one_pass()
            passes += 1
            dt_s = time.perf_counter() - t0
            if dt_s >= min_seconds:
                break
        assert np.all(np.isfinite(y))
        flops = passes * 2.0 * rows * n * k
        print(json.dumps({"case": wl.name, "op": wl.op, "dtype": dt, "sample_rows": rows, "of_rows": wl.m,
                          "n": n, "k": k, "passes": passes, "seconds": round(dt_s, 3),
                          "oracle_tflops": round(flops / dt_s / 1e12, 6), "threads": int(threads),
                          "cpu_model": cpu_model()}), file=sys.stderr, flush=True)


def run_configs(torch, tgc, synth, dev, iters=10):
    """Time every workload at its configured splits; one JSON line per case on stderr.
    The GEMM-only comparator is torch.matmul (hipBLASLt) on the same shapes."""
    def timeit(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(iters):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / iters

    def emit(name, flops, ms, ref_ms, **kw):
        line = {"case": name, "ms": round(ms, 5), "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
                "pct_bf16_peak": round(100 * flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                "hipblaslt_gemm_only_ms": round(ref_ms, 5)}
        line.update(kw)
        print(json.dumps(line), file=sys.stderr, flush=True)

    W = synth.WORKLOADS
    wl = W["toy_f32"]
    x = synth.uniform(wl.wid, synth.T_X, 0, (wl.m, wl.k), -1, 1, "f32").to(dev)
    w = synth.uniform(wl.wid, synth.T_W, 0, (wl.k, wl.n), -1, 1, "f32").to(dev)
    pr = [None, synth.uniform(wl.wid, synth.T_PEER, 1, (wl.m, wl.n), -1, 1, "f32").to(dev)]
    ms = timeit(lambda: tgc.matmul_all_reduce(x, w, pr, 0, split=2))
    emit("toy_f32 AR split2", 2.0 * wl.m * wl.n * wl.k, ms, timeit(lambda: torch.matmul(x, w)))

    for name, det_list, splits in (("bloom7b_ar", (0, 1), (4, 2, 8)), ("bloom176b_ar", (1,), (2, 4, 8))):
        wl = W[name]
        x = synth.normal(wl.wid, synth.T_X, 0, (wl.m, wl.k), 1.0, "bf16").to(dev)
        w = synth.normal(wl.wid, synth.T_W, 0, (wl.k, wl.n), 0.02, "bf16").to(dev)
        pr = [None] + [synth.normal(wl.wid, synth.T_PEER, r, (wl.m, wl.n), wl.peer_sigma, "bf16").to(dev)
                       for r in range(1, wl.world)]
        y = torch.empty((wl.m, wl.n), dtype=torch.bfloat16, device=dev)
        po = torch.empty_like(y)
        ref = timeit(lambda: torch.matmul(x, w))
        for det in det_list:
            for sp in splits:
                ms = timeit(lambda: tgc.matmul_all_reduce(x, w, pr, 0, y=y, partial_out=po, split=sp,
                                                          deterministic=det))
                emit(f"{name} split{sp} det{det}", 2.0 * wl.m * wl.n * wl.k, ms, ref)
        del x, w, pr, y, po

    wl = W["w8a16_ar"]
    x = synth.normal(wl.wid, synth.T_X, 0, (wl.m, wl.k), 1.0, "f16").to(dev)
    q = synth.integers(wl.wid, synth.T_W, 0, (wl.k, wl.n), -127, 127, "i8").to(dev)
    pr = [None] + [synth.normal(wl.wid, synth.T_PEER, r, (wl.m, wl.n), wl.peer_sigma, "f16").to(dev)
                   for r in range(1, wl.world)]
    wf = q.to(torch.float16)
    ref = timeit(lambda: torch.matmul(x, wf))
    for mode, shape in (("per_tensor", (1,)), ("per_channel", (wl.n,)), ("per_group", (wl.k // wl.group, wl.n))):
        sc = synth.fp16_scales(wl.wid, 0, shape).to(dev)
        ms = timeit(lambda: tgc.matmul_all_reduce_w8a16(x, q, sc, mode, pr, 0, group_size=wl.group, split=4))
        emit(f"w8a16_ar {mode} split4", 2.0 * wl.m * wl.n * wl.k, ms, ref)
    del x, q, pr, wf

    run_backward(torch, tgc, synth, dev, timeit, emit)


def run_backward(torch, tgc, synth, dev, timeit, emit, warm_passes=0):
    """The backward of the LLaMA2-70B pair: dX of the down projection (AG(dY) @ W^T,
    the 3584 x 8192 forward weight read transposed), dX of the gate/up layer
    (dY @ W^T reduce-scattered, W 8192 x 7168 read transposed), and dW of the
    gate/up layer from the gathered G.  Inputs are drawn once; `warm_passes`
    untimed passes over the cases first; then one JSON line per case (emit)."""
    W = synth.WORKLOADS
    wl = W["llama70b_ag"]
    shard = wl.m // wl.world
    dys = [synth.normal(wl.wid, synth.T_PEER, 9 + r, (shard, wl.k), 1.0, "bf16").to(dev) for r in range(wl.world)]
    w_down = synth.normal(wl.wid, synth.T_W, 9, (3584, wl.k), 0.02, "bf16").to(dev)
    w_up = synth.normal(wl.wid, synth.T_W, 0, (wl.k, wl.n), 0.02, "bf16").to(dev)
    dy = synth.normal(wl.wid, synth.T_X, 9, (wl.m, wl.n), 1.0, "bf16").to(dev)
    pr = [None] + [synth.normal(wl.wid, synth.T_PEER, 20 + r, (wl.m, wl.k), 1.0, "bf16").to(dev)
                   for r in range(1, wl.world)]
    g = torch.cat(dys)
    cases = [
        ("llama70b backward dX down-proj: AG(dY 8x512x8192) @ W^T (8192 -> 3584) split4",
         2.0 * wl.m * 3584 * wl.k,
         lambda: tgc.allgather_matmul(dys[0], dys, w_down, 0, split=4, trans_w=True),
         lambda: torch.matmul(torch.cat(dys), w_down.t())),
        ("llama70b backward dX gate/up: dY 4096x7168 @ W^T (7168 -> 8192) reduce-scattered split4",
         2.0 * wl.m * wl.k * wl.n,
         lambda: tgc.matmul_reduce_scatter(dy, w_up, pr, 0, split=4, trans_w=True),
         lambda: torch.matmul(dy, w_up.t())),
        ("llama70b backward dW gate/up: G^T (8192x4096) @ dY (4096x7168)",
         2.0 * wl.m * wl.k * wl.n,
         lambda: tgc.weight_grad(g, dy),
         lambda: torch.matmul(g.t(), dy)),
    ]
    for _ in range(warm_passes):
        for _, _, fn, _ in cases:
            for _ in range(10):
                fn()
        torch.cuda.synchronize()
    for name, flops, fn, ref in cases:
        ms = timeit(fn)
        emit(name, flops, ms, timeit(ref))


def run_backward_only(torch, tgc, synth, dev, iters=10, warm_passes=3):
    """Only the backward cases (stderr lines), after `warm_passes` untimed passes
    so the GPU is at its steady clocks."""
    def timeit(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(iters):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / iters

    def emit(name, flops, ms, ref_ms, **kw):
        line = {"case": name, "ms": round(ms, 5), "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
                "pct_bf16_peak": round(100 * flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                "hipblaslt_gemm_only_ms": round(ref_ms, 5)}
        line.update(kw)
        print(json.dumps(line), file=sys.stderr, flush=True)

    run_backward(torch, tgc, synth, dev, timeit, emit, warm_passes=warm_passes)


def run_lone(torch, tgc, synth, dev, iters=20, reps=3):
    """The lone matmuls of the LLaMA2-70B pair against hipBLASLt (torch.matmul):
    the all-gather op's 4096x7168x8192 and the reduce-scatter op's 4096x8192x3584
    (k x n weights), and the backward 4096x8192x7168 with the weight read
    transposed (n x k).  Each is one matmul of the library with one rank and
    split 1; its launch time comes from the library's per-launch events (the op
    itself also copies partial_out into y).  The cases run interleaved, in a
    seeded shuffled order per repetition; one stderr JSON line per case and
    repetition."""
    import random

    W = synth.WORKLOADS
    ag, rs = W["llama70b_ag"], W["llama70b_rs"]
    m = ag.m
    x_ag = synth.normal(ag.wid, synth.T_X, 30, (m, ag.k), 1.0, "bf16").to(dev)
    w_ag = synth.normal(ag.wid, synth.T_W, 30, (ag.k, ag.n), 0.02, "bf16").to(dev)
    x_rs = synth.normal(rs.wid, synth.T_X, 31, (m, rs.k), 1.0, "bf16").to(dev)
    w_rs = synth.normal(rs.wid, synth.T_W, 31, (rs.k, rs.n), 0.02, "bf16").to(dev)
    dy = synth.normal(ag.wid, synth.T_X, 32, (m, ag.n), 1.0, "bf16").to(dev)
    outs = {}

    def ours(name, x, w, trans_w=False):
        n = w.shape[0] if trans_w else w.shape[1]
        y, p = (torch.empty((x.shape[0], n), dtype=x.dtype, device=dev) for _ in range(2))
        outs[name] = (y, p)
        return lambda: tgc.matmul_all_reduce(x, w, [None], 0, y=y, partial_out=p, split=1, trans_w=trans_w)

    def ref(x, w):
        y = torch.empty((x.shape[0], w.shape[1]), dtype=x.dtype, device=dev)
        return lambda: torch.matmul(x, w, out=y)

    cases = {
        "NN 4096x7168x8192 (all-gather op's matmul)": (2.0 * m * ag.n * ag.k, ours("ag", x_ag, w_ag),
                                                      ref(x_ag, w_ag)),
        "NN 4096x8192x3584 (reduce-scatter op's matmul)": (2.0 * m * rs.n * rs.k, ours("rs", x_rs, w_rs),
                                                          ref(x_rs, w_rs)),
        "NT 4096x8192x7168 (backward dX, weight read transposed)": (2.0 * m * ag.k * ag.n,
                                                                    ours("nt", dy, w_ag, trans_w=True),
                                                                    ref(dy, w_ag.t())),
    }

    def timeit(fn):
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(iters):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / iters

    def kernel_ms(fn):
        torch.cuda.synchronize()
        tgc.profile_read()
        tgc.profile_enable(True)
        for _ in range(iters):
            fn()
        torch.cuda.synchronize()
        tgc.profile_enable(False)
        gm = tgc.profile_read()["gemm"]
        return gm["ms"] / gm["launches"]

    order = random.Random(7)
    for rep in range(reps):
        names = list(cases)
        order.shuffle(names)
        for name in names:
            flops, fn, rfn = cases[name]
            op_ms, k_ms, r_ms = timeit(fn), kernel_ms(fn), timeit(rfn)
            print(json.dumps({"case": name, "rep": rep, "matmul_launch_ms": round(k_ms, 5),
                              "matmul_launch_tflops": round(flops / (k_ms * 1e-3) / 1e12, 1),
                              "op_ms": round(op_ms, 5), "hipblaslt_ms": round(r_ms, 5),
                              "hipblaslt_tflops": round(flops / (r_ms * 1e-3) / 1e12, 1)}),
                  file=sys.stderr, flush=True)


def run_moe(torch, tgc, synth, dev, iters=10, prewarm_s=0.5):
    """The MoE expert all-to-all + grouped matmul pair on the Ampipe page's
    scenario (hidden 12288, ffn 49152, 8192 tokens per rank, 4 experts, top 2,
    EP 2; rank 0's share) at 1, 2 and 4 sequence pieces: dispatch then the
    first expert matmul, the second expert matmul then combine.  Rows and
    weights come from a seeded GPU generator (2.4 GB of weights per matmul).
    One JSON line per case on stderr; the GEMM-only comparator is one
    torch.matmul (hipBLASLt) per expert over its rows."""
    import dataclasses

    import numpy as np
    wl0 = synth.MOE_WORKLOADS["moe_ampipe"]
    g = torch.Generator(device=dev).manual_seed(wl0.wid)
    bf = torch.bfloat16
    k1, n1 = wl0.hidden, wl0.ffn
    w1 = (torch.randn(wl0.local, k1, n1, device=dev, generator=g) * 0.02).to(bf)
    w2 = (torch.randn(wl0.local, n1, k1, device=dev, generator=g) * 0.02).to(bf)

    def timeit(fn, warm=2):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(iters):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / iters

    first = True
    for pieces in (1, 2, 4):
        wl = dataclasses.replace(wl0, pieces=pieces)
        counts = synth.moe_counts(wl)
        total = int(counts.sum())
        rows = counts.sum(axis=(0, 2))
        sends = [torch.randn(int(rows[r]), k1, device=dev, generator=g).to(bf) for r in range(wl.world)]
        peers = [None if r == wl.rank else sends[r] for r in range(wl.world)]
        y1 = torch.empty(total, n1, dtype=bf, device=dev)
        recv = torch.empty(total, k1, dtype=bf, device=dev)
        y2 = torch.empty(total, k1, dtype=bf, device=dev)
        outs = [torch.empty(int(rows[r]), k1, dtype=bf, device=dev) for r in range(wl.world)]
        po = [None if r == wl.rank else outs[r] for r in range(wl.world)]

        def dispatch():
            tgc.alltoall_grouped_matmul(sends[wl.rank], peers, counts, w1, wl.rank, y=y1, recv_out=recv)

        def combine():
            tgc.grouped_matmul_alltoall(y1, w2, counts, wl.rank, y_own=outs[wl.rank], peer_out=po, y_local=y2)

        if first and prewarm_s > 0:
            t0 = time.perf_counter()
            while time.perf_counter() - t0 < prewarm_s:
                dispatch()
                torch.cuda.synchronize()
            first = False
        per_expert = counts.sum(axis=(0, 1))
        ref1 = ref2 = None
        if pieces == 1:
            # one matmul per expert over all its rows (the received order groups them)
            starts = np.concatenate([[0], np.cumsum(per_expert)])
            a1 = [recv[starts[e]:starts[e + 1]] for e in range(wl.local)]
            a2 = [y1[starts[e]:starts[e + 1]] for e in range(wl.local)]
            dispatch()
            ref1 = timeit(lambda: [torch.matmul(a1[e], w1[e]) for e in range(wl.local)])
            ref2 = timeit(lambda: [torch.matmul(a2[e], w2[e]) for e in range(wl.local)])
        flops = 2.0 * total * k1 * n1
        for name, fn, ref in (("dispatch + expert matmul 1", dispatch, ref1),
                              ("expert matmul 2 + combine", combine, ref2)):
            ms = timeit(fn)
            line = {"case": f"moe_ampipe {name} pieces{pieces}", "rows": total, "ms": round(ms, 5),
                    "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
                    "pct_bf16_peak": round(100 * flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2)}
            if ref is not None:
                line["hipblaslt_gemm_only_ms"] = round(ref, 5)
            print(json.dumps(line), file=sys.stderr, flush=True)
        del sends, peers, y1, recv, y2, outs, po
        torch.cuda.empty_cache()


CASES = ("bloom7b_ar", "bloom176b_ar", "w8a16_ar", "llama70b_ag", "llama70b_rs")


def run_case(args, torch, tgc, synth, dev):
    """One workload's op alone (--case NAME) at --split, timed like the step:
    prewarm, W warmup calls, K timed calls on the caller's stream; then the
    serial (split 1) form and the overlap view.  One JSON line on stdout."""
    W = synth.WORKLOADS
    wl = W[args.case]
    world, rank = wl.world, 0
    det = 1 if args.case == "bloom176b_ar" else 0
    split = {"split": args.split}
    if args.case in ("bloom7b_ar", "bloom176b_ar"):
        x = synth.normal(wl.wid, synth.T_X, 0, (wl.m, wl.k), 1.0, "bf16").to(dev)
        w = synth.normal(wl.wid, synth.T_W, 0, (wl.k, wl.n), wl.w_sigma, "bf16").to(dev)
        pr = [None] + [synth.normal(wl.wid, synth.T_PEER, r, (wl.m, wl.n), wl.peer_sigma, "bf16").to(dev)
                       for r in range(1, world)]
        y = torch.empty((wl.m, wl.n), dtype=torch.bfloat16, device=dev)
        po = torch.empty_like(y)

        def op():
            tgc.matmul_all_reduce(x, w, pr, rank, y=y, partial_out=po, split=split["split"], deterministic=det)
        comm_bytes = (world + 1.0) * wl.m * wl.n * 2
        what = f"MATMUL_ALL_REDUCE bf16 X {wl.m}x{wl.k} @ W {wl.k}x{wl.n}, {world} partials"
    elif args.case == "w8a16_ar":
        x = synth.normal(wl.wid, synth.T_X, 0, (wl.m, wl.k), 1.0, "f16").to(dev)
        q = synth.integers(wl.wid, synth.T_W, 0, (wl.k, wl.n), -127, 127, "i8").to(dev)
        sc = synth.fp16_scales(wl.wid, 0, (wl.n,)).to(dev)
        pr = [None] + [synth.normal(wl.wid, synth.T_PEER, r, (wl.m, wl.n), wl.peer_sigma, "f16").to(dev)
                       for r in range(1, world)]
        y = torch.empty((wl.m, wl.n), dtype=torch.float16, device=dev)
        po = torch.empty_like(y)

        def op():
            tgc.matmul_all_reduce_w8a16(x, q, sc, "per_channel", pr, rank, y=y, partial_out=po,
                                        split=split["split"], deterministic=det)
        comm_bytes = (world + 1.0) * wl.m * wl.n * 2
        what = f"w8A16 MATMUL_ALL_REDUCE per channel, X {wl.m}x{wl.k} fp16 @ int8 W {wl.k}x{wl.n}, {world} partials"
    else:
        inp = make_inputs(torch, tgc, synth, args.split, dev)
        if args.case == "llama70b_ag":
            def op():
                tgc.allgather_matmul(inp["ag_x"], inp["ag_peers"], inp["ag_w"], rank, y=inp["ag_y"], ws=inp["ag_ws"],
                                     split=split["split"])
            comm_bytes = 2.0 * wl.m * wl.k * 2
            what = f"ALL_GATHER_MATMUL bf16 {world}x({wl.m // world}x{wl.k}) @ W {wl.k}x{wl.n}"
        else:
            def op():
                tgc.matmul_reduce_scatter(inp["rs_x"], inp["rs_w"], inp["rs_peers"], rank, y=inp["rs_y"],
                                          partial_out=inp["rs_part"], split=split["split"])
            comm_bytes = (world + 1.0) * (wl.m // world) * wl.n * 2
            what = f"MATMUL_REDUCE_SCATTER bf16 X {wl.m}x{wl.k} @ W {wl.k}x{wl.n} -> {wl.m // world}x{wl.n}"
    flops = 2.0 * wl.m * wl.n * wl.k
    log(f"case {args.case}: {what}, split {args.split}, det {det}")
    t_pre = time.perf_counter()
    while time.perf_counter() - t_pre < args.prewarm_s:
        for _ in range(10):
            op()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        op()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        op()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    log(f"timed {args.steps} calls: {ms:.4f} ms")
    out = {"case": args.case, "op": what, "split": args.split, "deterministic": det, "ms": round(ms, 5),
           "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
           "pct_bf16_peak": round(100 * flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2)}
    if not args.no_breakdown:
        split["split"] = 1
        e0.record()
        for _ in range(args.steps):
            op()
        e1.record()
        torch.cuda.synchronize()
        out["serial_ms"] = round(e0.elapsed_time(e1) / args.steps, 5)
        g1, c1 = serial_parts(torch, tgc, op)
        split["split"] = args.split
        sbuf = stamp_buffer(torch, dev)
        o = mean_dicts([overlap_of(stamped(torch, tgc, sbuf, op), comm_bytes) for _ in range(5)])
        o["serial_matmul_ms"] = round(g1, 5)
        o["serial_comm_ms"] = round(c1, 5)
        o["hidden_frac_vs_serial"] = round((g1 + c1 - ms) / c1, 4) if c1 > 0 else None
        o["unhidden_frac_vs_serial"] = None if o["hidden_frac_vs_serial"] is None else \
            round(1 - o["hidden_frac_vs_serial"], 4)
        out["overlap"] = o
        out["vs_serial_matmul"] = round(ms / g1, 4) if g1 > 0 else None
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--prewarm-s", type=float, default=0.5,
                    help="before the warmup steps, run untimed steps for this many seconds so the GPU "
                         "reaches its steady clocks (0: off)")
    ap.add_argument("--split", type=int, default=4, choices=[1, 2, 4, 8])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-frac", type=float, default=1.0)
    ap.add_argument("--no-breakdown", action="store_true",
                    help="skip the per-op and serial timings after the timed region (profiling runs)")
    ap.add_argument("--configs", action="store_true",
                    help="after the main line, time every workload at its configured splits (stderr)")
    ap.add_argument("--moe", action="store_true",
                    help="only time the MoE expert all-to-all + grouped matmul pair on the Ampipe "
                         "scenario (stderr lines) and exit")
    ap.add_argument("--operands", choices=["seeded", "constant"], default="seeded",
                    help="constant: every matmul operand of the step holds one value (same kernels, same "
                         "work) -- a diagnostic of the clock the GPU sustains when the MFMA inputs do not "
                         "toggle; its line is marked as such and is not a benchmark figure")
    ap.add_argument("--backward", action="store_true",
                    help="only time the backward cases of the LLaMA2-70B pair (stderr lines) and exit")
    ap.add_argument("--lone", action="store_true",
                    help="only time the lone matmuls of the step's two ops and of the backward dX "
                         "against hipBLASLt, interleaved (stderr lines), and exit")
    ap.add_argument("--case", choices=CASES,
                    help="only time one workload's op at --split (prewarm, W warmup calls, K timed calls), "
                         "then its serial form and the overlap view; one JSON line, and exit")
    ap.add_argument("--mfma-loop", action="store_true",
                    help="diagnostic: the bf16 MFMA rate on register operands, random against constant values")
    ap.add_argument("--weights", choices=["kn", "nk"], default="kn",
                    help="storage of the step's weights: kn (k x n, the default) or nk (n x k, a Linear "
                         "layer's out x in layout, through the *_trans_w entry points; the same products)")
    ap.add_argument("--cpu-configs", action="store_true",
                    help="only time the CPU oracle on every workload (a bounded sample of rows, all n and k; "
                         "stderr lines, no GPU) and exit")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain elementwise copy of 1 GiB (read 1 GiB, write 1 GiB) three "
                         "times, for scaling the HBM byte counters, and exit")
    args = ap.parse_args()

    world_env = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world_env != 1:
        print(f"bench.py measures one rank's share on a single GPU; --gpus {args.gpus} "
              f"(WORLD_SIZE={world_env}) is not supported: the other ranks are emulated as "
              f"buffers in the same HBM, so run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import tensor_gemm_collective_amd as tgc
    from tensor_gemm_collective_amd import synth

    if args.cpu_configs:
        run_cpu_configs(synth)
        return
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        n = 1 << 28
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "elementwise copy", "bytes_read_per_launch": 4 * n,
                          "bytes_written_per_launch": 4 * n, "launches": 3}), flush=True)
        return
    tgc.lib()
    if args.mfma_loop:
        run_mfma_loop(torch, tgc, dev)
        return
    if args.moe:
        run_moe(torch, tgc, synth, dev, prewarm_s=args.prewarm_s)
        return
    if args.lone:
        run_lone(torch, tgc, synth, dev)
        return
    if args.backward:
        run_backward_only(torch, tgc, synth, dev, warm_passes=3 if args.prewarm_s > 0 else 0)
        return
    if args.case:
        run_case(args, torch, tgc, synth, dev)
        return
    log("generating inputs ...")
    inp = make_inputs(torch, tgc, synth, args.split, dev)
    if args.operands == "constant":
        # 2^-4 activations, 2^-6 weights: every product is exact and every sum
        # stays far inside bf16's range (k * 2^-10 <= 8)
        for key in ("ag_x", "rs_x"):
            inp[key].fill_(0.0625)
        for t in inp["ag_peers"]:
            if t is not None:
                t.fill_(0.0625)
        for key in ("ag_w", "rs_w"):
            inp[key].fill_(0.015625)
        b = inp["rs"].m // inp["world"]
        for t in inp["rs_peers"]:
            if t is not None:
                t[inp["rank"] * b:(inp["rank"] + 1) * b].fill_(1.0)
        args.no_cpu_baseline = True
    trans = args.weights == "nk"
    if trans:
        # the same weights stored n x k (a Linear layer's out x in layout),
        # multiplied through the *_trans_w entry points: the same products
        inp["ag_w"] = inp["ag_w"].t().contiguous()
        inp["rs_w"] = inp["rs_w"].t().contiguous()
    torch.cuda.synchronize()
    f_ag, f_rs = flops_of(inp)
    rank, split = inp["rank"], args.split

    def run_ag():
        tgc.allgather_matmul(inp["ag_x"], inp["ag_peers"], inp["ag_w"], rank, y=inp["ag_y"], ws=inp["ag_ws"],
                             split=split, trans_w=trans)

    def run_rs():
        tgc.matmul_reduce_scatter(inp["rs_x"], inp["rs_w"], inp["rs_peers"], rank, y=inp["rs_y"],
                                  partial_out=inp["rs_part"], split=split, trans_w=trans)

    def step():
        run_ag()
        run_rs()

    # The GPU idles while the inputs are generated on the host; a few
    # milliseconds of warmup steps leave it short of its steady clocks, which
    # costs about a tenth of the step rate.  Untimed steps for prewarm_s
    # seconds first (not counted in the K timed steps).
    prewarm_steps, t_pre = 0, time.perf_counter()
    while time.perf_counter() - t_pre < args.prewarm_s:
        for _ in range(20):
            step()
        torch.cuda.synchronize()
        prewarm_steps += 20
    log(f"prewarm {prewarm_steps} steps, then warmup {args.warmup} steps ...")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps (no per-kernel events)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / args.steps
    log(f"timed {args.steps} steps: {ms_step:.4f} ms/step (host wall {wall / args.steps * 1e3:.4f} ms/step)")

    # ---- the same K steps again with HIP events around every library launch
    # (recorded by the library on the stream each kernel goes to)
    log("per-launch events pass ...")
    tgc.profile_enable(True)
    tgc.profile_records()
    torch.cuda.synchronize()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    recs = tgc.profile_records()
    tgc.profile_enable(False)
    prof = {c: {"ms": 0.0, "launches": 0, "work": 0.0, "busy_ms": 0.0} for c in ("gemm", "reduce", "gather")}
    for c in prof:
        iv = sorted((a, b) for k, a, b, w in recs if k == c)
        prof[c]["launches"] = len(iv)
        prof[c]["ms"] = sum(b - a for a, b in iv)
        prof[c]["work"] = sum(w for k, a, b, w in recs if k == c)
        busy, cur = 0.0, None
        for a, b in iv:                      # union of the launch intervals
            if cur is None or a > cur[1]:
                if cur is not None:
                    busy += cur[1] - cur[0]
                cur = [a, b]
            else:
                cur[1] = max(cur[1], b)
        if cur is not None:
            busy += cur[1] - cur[0]
        prof[c]["busy_ms"] = busy

    # ---- per-op breakdown and the serial (split 1) form, outside the timed region
    def time_op(fn, iters=10):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        torch.cuda.synchronize()
        a.record()
        for _ in range(iters):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / iters

    def time_cold(fn, iters=50):
        """Per-call times with the caches cold: before each call a 512 MB write
        evicts the L2s and the 256 MB memory-side cache (outside the events).
        Returns (median, p10, p90) in ms."""
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        ts = []
        for i in range(iters + 1):
            flush.fill_(i & 0xff)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            if i > 0:
                ts.append(a.elapsed_time(b))
        del flush
        ts.sort()
        q = lambda f: ts[min(len(ts) - 1, int(round(f * (len(ts) - 1))))]
        return q(0.5), q(0.1), q(0.9)

    ag, rs, world = inp["ag"], inp["rs"], inp["world"]
    comm_bytes = {"allgather_matmul": 2.0 * ag.m * ag.k * 2,                     # gathered rows read + written
                  "matmul_reduce_scatter": (world + 1.0) * (rs.m // world) * rs.n * 2}   # 8 partial slices + y
    cold = None
    overlap = None
    if args.no_breakdown:
        ms_ag = ms_rs = ms_serial = float("nan")
    else:
        log("per-op and serial timings ...")
        ms_ag = time_op(run_ag)
        ms_rs = time_op(run_rs)
        split_saved = split
        split = 1
        ms_serial = time_op(step)
        serial = {"allgather_matmul": serial_parts(torch, tgc, run_ag),
                  "matmul_reduce_scatter": serial_parts(torch, tgc, run_rs)}
        split = split_saved
        # Overlap (the Overlap blog's profiler view; SURVEY's definitions):
        # from the kernels' activity records, the communication's active time
        # and the part of it inside the matmul's span; and hidden =
        # (T_matmul alone + T_comm alone - T_pipelined) / T_comm alone, with
        # the split-1 launches as the "alone" times.
        log("overlap (activity records) ...")
        sbuf = stamp_buffer(torch, dev)
        overlap = {}
        tot_active = tot_exposed = 0.0
        for name, fn, ms_op in (("allgather_matmul", run_ag, ms_ag), ("matmul_reduce_scatter", run_rs, ms_rs)):
            per = [overlap_of(stamped(torch, tgc, sbuf, fn), comm_bytes[name]) for _ in range(5)]
            o = mean_dicts(per)
            g1, c1 = serial[name]
            o["serial_matmul_ms"] = round(g1, 5)
            o["serial_comm_ms"] = round(c1, 5)
            o["pipelined_ms"] = round(ms_op, 5)
            o["hidden_frac_vs_serial"] = round((g1 + c1 - ms_op) / c1, 4) if c1 > 0 else None
            overlap[name] = o
            tot_active += o.get("comm_active_us", 0.0)
            tot_exposed += o.get("comm_exposed_us", 0.0)
        overlap["step_unhidden_comm_frac"] = round(tot_exposed / tot_active, 4) if tot_active > 0 else None
        del sbuf
        log("cold-cache timings ...")
        cold = {"flush_bytes": 512 << 20, "iterations": 50}
        for name, fn, fl in (("allgather_matmul", run_ag, f_ag), ("matmul_reduce_scatter", run_rs, f_rs),
                             ("step", step, f_ag + f_rs)):
            med, p10, p90 = time_cold(fn)
            cold[name] = {"median_ms": round(med, 5), "p10_ms": round(p10, 5), "p90_ms": round(p90, 5),
                          "tflops_median": round(fl / (med * 1e-3) / 1e12, 2)}

    # ---- the GPU clock under this load (after everything above is measured)
    if not args.no_breakdown:
        log("clock sampling ...")
    clock = None if args.no_breakdown else sample_clock(step, torch)

    value = (f_ag + f_rs) / (ms_step * 1e-3) / 1e12
    g = prof["gemm"]
    avg_ms = g["ms"] / max(1, g["launches"])
    flops_per_launch = g["work"] / max(1, g["launches"])
    achieved = g["work"] / (g["busy_ms"] * 1e-3) / 1e12 if g["busy_ms"] > 0 else 0.0
    gemm_ms = g["busy_ms"] / args.steps

    def tf(flops, ms):
        return None if ms != ms else round(flops / (ms * 1e-3) / 1e12, 2)

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "prewarm": {"seconds": args.prewarm_s, "steps": prewarm_steps},
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": ("synthetic (seeded N(0,1) activations, N(0,0.02^2) weights, emulated peer shards/partials)"
                 if args.operands == "seeded" else
                 "DIAGNOSTIC, not a benchmark figure: every matmul operand constant (clock under MFMA load "
                 "without operand toggling)"),
        "config": {
            "workload": "LLaMA2-70B TP8+SP MLP, one rank: ALL_GATHER_MATMUL 8x(512x8192) @ 8192x7168 "
                        "then MATMUL_REDUCE_SCATTER 4096x3584 @ 3584x8192 -> 512x8192",
            "world": inp["world"], "rank": rank, "split": split, "deterministic": 0,
            "weight_layout": "n x k (transposed, *_trans_w)" if trans else "k x n",
        },
        "pct_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "breakdown": {
            "allgather_matmul": {"ms": round(ms_ag, 5), "tflops": tf(f_ag, ms_ag)},
            "matmul_reduce_scatter": {"ms": round(ms_rs, 5), "tflops": tf(f_rs, ms_rs)},
            "serial_split1": {"ms": round(ms_serial, 5), "tflops": tf(f_ag + f_rs, ms_serial)},
            "cold_cache": cold,
            "kernel_busy_ms_per_step": {k: round(v["busy_ms"] / args.steps, 5) for k, v in prof.items()},
            "kernel_launches_per_step": {k: v["launches"] / args.steps for k, v in prof.items()},
            "overlap": overlap,
            # the part of the step with no matmul launch running: exposed
            # communication, launch gaps and the reduce of the last round
            "no_matmul_ms_per_step": round(ms_step - gemm_ms, 5),
            "no_matmul_frac_of_step": round(max(0.0, ms_step - gemm_ms) / ms_step, 4),
            "overlap_note": "comm_active_us: union of the reduce / gather workgroups' active intervals "
                            "(waiting on counters excluded), from the kernels' activity records; "
                            "comm_hidden_us: the part inside the matmul's span; comm_gbs_active: the op's "
                            "communication bytes over its active time; hidden_frac_vs_serial: "
                            "(T_matmul + T_comm of the split-1 launches - T_pipelined) / T_comm",
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "gemm_ring_chunks (one launch walks every m-chunk of an op)",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic(),
            "gpu_clock": clock,
            "frac_of_peak_at_measured_clock": (round(achieved / clock["bf16_peak_at_median_clock_tflops"], 4)
                                               if clock else None),
            "avg_launch_us": round(avg_ms * 1e3, 3),
            "launches_per_step": g["launches"] / args.steps,
            "flops_per_launch": flops_per_launch,
            "note": "achieved = matmul flops / matmul launch time, one launch per op (the "
                    "all-gather launch includes waiting for its first gathered chunk)",
        },
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_frac)
    print(json.dumps(out), flush=True)
    if args.configs:
        del inp
        torch.cuda.empty_cache()
        run_configs(torch, tgc, synth, dev)
        run_moe(torch, tgc, synth, dev, prewarm_s=0)


if __name__ == "__main__":
    main()
