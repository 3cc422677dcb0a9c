"""Benchmark of the BF16 hyper-connection read on one MI355X.

Workload (the cold-weight T sweep): real geometry (4 streams x 2560, R = 320,
13,107,200 bytes of BF16 weights per read), 32 independent weight sets
(419 MB, more than the 256 MB MALL) rotated call by call, T = 1..8 tokens,
x ~ N(0, 1), no pending write or injection.  One step = for T = 1..8, one read
per weight set (256 reads), captured once as a HIP graph and replayed; inputs
are resident in HBM before the timed region starts.

Prints ONE JSON line: value = microseconds per read over the whole step
(lower is better), per-T microseconds and algorithmic GB/s, the roofline of
the read, and the FP64 CPU reference timed on the host as a baseline.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs per cold HC read (norm+down+up) at T=1..8; achieved HBM GB/s vs peak"
HBM_PEAK_GBPS = 8000.0
S, D, R, TMAX = 4, 2560, 320, 8
T_WIDE = 16  # larger verify windows, reported per T beside the step
# A graph replay costs ~6 us of its own on this stack (a graph of two 96-read windows takes 2 W + 6 us, one
# window W + 6 us), so the per-T graphs pass ROT times over the rotated sets (256 reads each) and a replay
# boundary adds ~0.02 us to a read instead of ~0.2 us with one pass of 32
ROT = 8
W_BYTES = 2 * R * S * D * 2


def algorithmic_bytes(T, pending=False, inj=False):
    """Weights once + w_norm + x read + out and mean written (+ pending, + inj)."""
    b = W_BYTES + S * D * 4 + T * (S * D * 4 + S * D * 4 + D * 4)
    if pending:
        b += T * S * D * 4
    if inj:
        b += T * R * 4
    return b


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hc_read_cold_sweep_traffic.json")


def algorithmic_bytes_q8(T):
    """Q8_0 codes and scales of both projections once + w_norm + x read + out and mean written."""
    return 2 * (R * S * D + R * S * D // 32 * 2) + S * D * 4 + T * (S * D * 4 + S * D * 4 + D * 4)


def measured_traffic(fmt="bf16"):
    """HBM bytes per read (mean over T = 1..8) from the committed counter summary, or None if the
    library's sources changed since the counters were taken."""
    from bf16_hyper_connection_amd import build
    try:
        with open(TRAFFIC_FILE) as fh:
            d = json.load(fh)
    except (OSError, ValueError):
        return None
    if d.get("source_sha256") != build.source_hash():
        return None
    return d.get(fmt, {}).get("bytes_per_read_mean_T1_8")


def measured_matvec_traffic():
    """HBM bytes per matvec call (mean over T = 1..4) from the same counter summary, or None."""
    from bf16_hyper_connection_amd import build
    try:
        with open(TRAFFIC_FILE) as fh:
            d = json.load(fh)
    except (OSError, ValueError):
        return None
    mv = d.get("matvec_bf16")
    if d.get("source_sha256") != build.source_hash() or not mv:
        return None
    return round(sum(v["hbm_bytes"] for v in mv.values()) / len(mv))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_model():
    """The host CPU's model name (Linux /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(budget_s=8.0):
    """The FP64 reference, as it stands, on a bounded sample of the same sweep: once on the host's BLAS
    threads, once on one core (BLAS limited to one thread)."""
    import oracle
    from bf16_hyper_connection_amd import inputs as gen
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001
        threadpool_limits, threads = None, 1
    ws = [gen.weight_set(2, k) for k in range(4)]
    xs = {T: gen.cold_sweep_x(T) for T in range(1, TMAX + 1)}

    def run(budget):
        n, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < budget:
            for T in range(1, TMAX + 1):
                w = ws[n % len(ws)]
                oracle.hc_read(xs[T], w.w_norm, w.w_down, w.w_up)
                n += 1
        return n, time.perf_counter() - t0

    n, el = run(budget_s)
    res = {"value": round(el / n * 1e6, 1), "unit": "µs per read", "cores": int(threads), "kind": "oracle",
           "sample": f"{n} reads of the same sweep (T = 1..8 in turn, 4 of the 32 weight sets), "
                     f"{el:.1f} s of float64 numpy on the host",
           "cpu_model": cpu_model(), "host_cpus": os.cpu_count()}
    if threadpool_limits is not None:
        with threadpool_limits(limits=1, user_api="blas"):
            n1, el1 = run(budget_s)
        res["one_core"] = {"value": round(el1 / n1 * 1e6, 1), "unit": "µs per read", "cores": 1,
                           "sample": f"{n1} reads of the same sweep, {el1:.1f} s, BLAS limited to one thread"}
    return res


def calib_lib():
    """libhcr_calib.so (include/hcr_calib.h): the read's two launches empty, and with only their loads."""
    import ctypes
    from bf16_hyper_connection_amd import build
    if not os.path.exists(build.CALIB_LIB):
        raise RuntimeError(f"{build.CALIB_LIB} is missing: build first")
    L = ctypes.CDLL(build.CALIB_LIB)
    vp = ctypes.c_void_p
    L.hcrc_read_floor.restype = ctypes.c_int
    L.hcrc_read_floor.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp, vp]
    return L


def ab_compare(args, readers, xs, outs, means, stream, timed):
    """Time the per-T cold sweep through several builds of libhcr.so (same C ABI), alternating between
    them round by round in one process; returns the comparison (median µs per read per T and library)."""
    import ctypes
    import torch
    Ts = list(range(1, args.ab_tmax + 1))
    libs = []
    for path in args.ab:
        L = ctypes.CDLL(os.path.abspath(path), mode=os.RTLD_LOCAL)
        vp = ctypes.c_void_p
        L.hcr_scratch_bytes.restype, L.hcr_scratch_bytes.argtypes = ctypes.c_size_t, []
        L.hcr_create.restype, L.hcr_create.argtypes = ctypes.c_int, [vp, vp, vp, vp, ctypes.c_size_t, ctypes.POINTER(vp)]
        L.hcr_read.restype, L.hcr_read.argtypes = ctypes.c_int, [vp, ctypes.c_int, vp, vp, vp, vp, vp, vp]
        L.hcr_quantize_q8_0.restype = ctypes.c_int
        L.hcr_quantize_q8_0.argtypes = [vp, ctypes.c_int, ctypes.c_int, vp, vp, vp]
        L.hcr_create_q8_0.restype = ctypes.c_int
        L.hcr_create_q8_0.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_size_t, ctypes.POINTER(vp)]
        nb = L.hcr_scratch_bytes()
        handles, scratch = [], []  # scratch: every device buffer a handle needs alive
        for r in readers:
            dev = r.w_down.device
            sc = torch.empty(nb, dtype=torch.uint8, device=dev)
            h = vp()
            if args.ab_q8:
                bufs = []
                for w in (r.w_down, r.w_up):
                    rows, cols = w.shape
                    c = torch.empty((rows, cols), dtype=torch.int8, device=dev)
                    sg = torch.empty((rows, cols // 32), dtype=torch.int16, device=dev)
                    rc = L.hcr_quantize_q8_0(w.data_ptr(), rows, cols, c.data_ptr(), sg.data_ptr(),
                                             vp(torch.cuda.current_stream().cuda_stream))
                    assert rc == 0, (path, rc)
                    bufs += [c, sg]
                rc = L.hcr_create_q8_0(bufs[0].data_ptr(), bufs[1].data_ptr(), bufs[2].data_ptr(), bufs[3].data_ptr(),
                                       r.w_norm.data_ptr(), sc.data_ptr(), nb, ctypes.byref(h))
                scratch.append((sc, bufs))
            else:
                rc = L.hcr_create(r.w_down.data_ptr(), r.w_up.data_ptr(), r.w_norm.data_ptr(), sc.data_ptr(), nb,
                                  ctypes.byref(h))
                scratch.append(sc)
            assert rc == 0, (path, rc)
            handles.append(h)
        torch.cuda.synchronize()
        graphs = {}
        for T in Ts:
            g = torch.cuda.CUDAGraph()
            stream.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(stream):
                with torch.cuda.graph(g, stream=stream):
                    for h in handles * ROT:
                        rc = L.hcr_read(h, T, xs[T].data_ptr(), None, None, outs[T].data_ptr(), means[T].data_ptr(),
                                        vp(stream.cuda_stream))
                        assert rc == 0, (path, T, rc)
            torch.cuda.current_stream().wait_stream(stream)
            graphs[T] = g
        libs.append((os.path.basename(path), L, handles, scratch, graphs))
    times = {name: {T: [] for T in Ts} for name, *_ in libs}
    for rnd in range(args.ab_rounds):
        for name, L, handles, scratch, graphs in libs:
            for T in Ts:
                times[name][T].append(timed(graphs[T], args.per_t_reps, 2) * 1000.0 / (args.per_t_reps * ROT * len(handles)))
            log(f"bench: A/B round {rnd} {name}: " + " ".join(f"{times[name][T][-1]:.3f}" for T in Ts))
    res = {}
    for name in times:
        med = {T: round(float(np.median(times[name][T])), 3) for T in Ts}
        res[name] = {"per_T_us": med, "mean_us": round(sum(med.values()) / len(med), 3),
                     "per_T_spread_us": {T: round(max(v) - min(v), 3) for T, v in times[name].items()}}
    return res


def ab_window(args, stream, timed):
    """The 96-read verify window (the bench's own workload: residual chain, T = 6, pending on, distinct weight
    sets) through several builds of libhcr.so, alternating round by round in one process; median µs per window
    and per read for each build."""
    import ctypes
    import torch
    from bf16_hyper_connection_amd import inputs as gen
    dev = torch.device("cuda:0")
    n_win, t_win = 96, 6
    cw = gen.verify_window(n_win, t_win)
    wts = [(torch.from_numpy(w.w_down.view(np.int16)).to(dev), torch.from_numpy(w.w_up.view(np.int16)).to(dev),
            torch.from_numpy(w.w_norm).to(dev)) for w in cw["weights"]]
    del cw["weights"]
    wpend = [torch.from_numpy(p_).to(dev) for p_ in cw["pending"]]
    wx0 = torch.from_numpy(cw["x0"]).to(dev)
    wouts = [torch.empty((t_win, S, D), device=dev) for _ in range(n_win)]
    wmeans = [torch.empty((t_win, D), device=dev) for _ in range(n_win)]
    vp = ctypes.c_void_p
    libs = []
    for path in args.ab:
        L = ctypes.CDLL(os.path.abspath(path), mode=os.RTLD_LOCAL)
        L.hcr_scratch_bytes.restype, L.hcr_scratch_bytes.argtypes = ctypes.c_size_t, []
        L.hcr_create.restype, L.hcr_create.argtypes = ctypes.c_int, [vp, vp, vp, vp, ctypes.c_size_t, ctypes.POINTER(vp)]
        L.hcr_read.restype, L.hcr_read.argtypes = ctypes.c_int, [vp, ctypes.c_int, vp, vp, vp, vp, vp, vp]
        nb = L.hcr_scratch_bytes()
        handles, scratch = [], []
        for wd, wu, wn in wts:
            sc = torch.empty(nb, dtype=torch.uint8, device=dev)
            h = vp()
            rc = L.hcr_create(wd.data_ptr(), wu.data_ptr(), wn.data_ptr(), sc.data_ptr(), nb, ctypes.byref(h))
            assert rc == 0, (path, rc)
            handles.append(h)
            scratch.append(sc)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                xx = wx0
                for i, h in enumerate(handles):
                    rc = L.hcr_read(h, t_win, xx.data_ptr(), wpend[i].data_ptr(), None, wouts[i].data_ptr(),
                                    wmeans[i].data_ptr(), vp(stream.cuda_stream))
                    assert rc == 0, (path, rc)
                    xx = wouts[i]
        torch.cuda.current_stream().wait_stream(stream)
        libs.append((os.path.basename(path), L, handles, scratch, g))
    reps = 20
    times = {name: [] for name, *_ in libs}
    for rnd in range(args.ab_rounds):
        for name, L, handles, scratch, g in libs:
            times[name].append(timed(g, reps, 2) * 1000.0 / reps)
            log(f"bench: A/B window round {rnd} {name}: {times[name][-1]:.2f} us")
    return {name: {"us_per_window": round(float(np.median(v)), 2), "us_per_read": round(float(np.median(v)) / n_win, 3),
                   "spread_us": round(max(v) - min(v), 2)} for name, v in times.items()}


def sha256_of(*tensors):
    """sha256 (hex) of the bytes of device tensors, in order."""
    import hashlib
    h = hashlib.sha256()
    for t in tensors:
        h.update(t.detach().contiguous().cpu().numpy().tobytes())
    return h.hexdigest()


def main():
    import ctypes
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--sets", type=int, default=32)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-window", action="store_true", help="skip the 96-read verify window measurement")
    ap.add_argument("--no-q8", action="store_true", help="skip the Q8_0 copies' per-T measurement")
    ap.add_argument("--per-t-reps", type=int, default=10, help="graph replays per T for the per-T figures")
    ap.add_argument("--no-matvec", action="store_true", help="skip the skinny BF16 matvec measurement")
    ap.add_argument("--no-calibration", action="store_true",
                    help="skip the calibration leg (the read's two launches empty, and with only their loads)")
    ap.add_argument("--ab", nargs="+", metavar="LIB",
                    help="A/B mode: time the per-T sweep through each of these builds of libhcr.so in turn "
                         "(alternating, --ab-rounds rounds), print one JSON line of the comparison and exit")
    ap.add_argument("--ab-rounds", type=int, default=3)
    ap.add_argument("--ab-tmax", type=int, default=8, help="A/B mode: T = 1..this")
    ap.add_argument("--ab-q8", action="store_true", help="A/B mode: read Q8_0 copies (each build quantises)")
    ap.add_argument("--ab-window", action="store_true",
                    help="A/B mode: time the 96-read verify window (T = 6, pending on, residual chain) through "
                         "each build instead of the per-T sweep")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the timed steps, run a plain 64 MiB device copy (scale for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this read runs on one GPU only (asked for --gpus {args.gpus}); "
              "run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from bf16_hyper_connection_amd import hcr
    from bf16_hyper_connection_amd import inputs as gen
    if not os.path.exists(hcr.LIB_PATH):
        from bf16_hyper_connection_amd import build
        build.build()
    dev = torch.device("cuda:0")

    log(f"bench: generating {args.sets} weight sets")
    readers = []
    for k in range(args.sets):
        w = gen.weight_set(2, k)
        readers.append(hcr.HCRead(torch.from_numpy(w.w_down.view(np.int16)).to(dev),
                                  torch.from_numpy(w.w_up.view(np.int16)).to(dev),
                                  torch.from_numpy(w.w_norm).to(dev)))
    xs = {T: torch.from_numpy(gen.cold_sweep_x(T)).to(dev) for T in range(1, T_WIDE + 1)}
    outs = {T: torch.empty((T, S, D), device=dev) for T in xs}
    means = {T: torch.empty((T, D), device=dev) for T in xs}
    torch.cuda.synchronize()

    stream = torch.cuda.Stream()

    def capture(Ts, calls_per_T):
        g = torch.cuda.CUDAGraph()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                for T in Ts:
                    for i in range(calls_per_T):
                        readers[i % len(readers)].read(xs[T], out=outs[T], mean=means[T])
        torch.cuda.current_stream().wait_stream(stream)
        return g

    marker = torch.zeros(1, device=dev)

    def timed(g, reps, warm, mark=False):
        """ms for reps replays of g on the bench stream (events on that stream).  With mark, a tiny
        torch kernel (neg_) runs just before and just after the timed region, outside the events,
        so that a kernel trace can find the region."""
        with torch.cuda.stream(stream):
            for _ in range(warm):
                g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            if mark:
                marker.neg_()
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
            if mark:
                marker.neg_()
            torch.cuda.synchronize()
        return e0.elapsed_time(e1)  # ms

    if args.ab and args.ab_window:
        res = ab_window(args, stream, timed)
        print(json.dumps({"ab_window": res, "rounds": args.ab_rounds,
                          "note": "median µs per 96-read verify window over the rounds, libraries alternating"}),
              flush=True)
        return
    if args.ab:
        res = ab_compare(args, readers, xs, outs, means, stream, timed)
        print(json.dumps({"ab": res, "rounds": args.ab_rounds, "weight_sets": len(readers),
                          "note": "median µs per read over the rounds, cold 32-set rotation, libraries alternating"}),
              flush=True)
        return

    # per-T: 32 rotated reads per graph, replayed 10 times (320 calls per T); T = 9..16 reported beside
    # The output hashes: after the replays, out and mean hold the last read of the graph (the last weight
    # set); the same read made directly must give the same bytes
    per_T_us, per_T_gbps, hashes = {}, {}, {"cold_sweep": {}}
    replay_equals_direct = True
    for T in range(1, T_WIDE + 1):
        g = capture([T], ROT * len(readers))
        ms = timed(g, args.per_t_reps, 2)
        us = ms * 1000.0 / (args.per_t_reps * ROT * len(readers))
        per_T_us[T] = round(us, 3)
        per_T_gbps[T] = round(algorithmic_bytes(T) / us / 1e3, 1)
        log(f"bench: T={T} {us:.3f} us/read  {per_T_gbps[T]:.0f} GB/s")
        del g
        h_out, h_mean = sha256_of(outs[T]), sha256_of(means[T])
        d_out, d_mean = readers[-1].read(xs[T])
        torch.cuda.synchronize()
        replay_equals_direct &= (sha256_of(d_out), sha256_of(d_mean)) == (h_out, h_mean)
        hashes["cold_sweep"][T] = {"out": h_out, "mean": h_mean}

    # cold-cache check: T = 1 and T = 8 with 1 weight set (MALL- and L2-resident), the 32 sets, and 64 sets
    # (the 32 and copies of them in other memory); 32 and 64 must agree if the rotation defeats the MALL
    extra = [hcr.HCRead(r.w_down.clone(), r.w_up.clone(), r.w_norm.clone()) for r in readers]
    cold_check = {}
    for T in (1, TMAX):
        row = {}
        for name, pool in (("1_set", readers[:1] * (ROT * len(readers))), ("32_sets", readers * ROT),
                           ("64_sets", (readers + extra) * (ROT // 2))):
            gc = torch.cuda.CUDAGraph()
            stream.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(stream):
                with torch.cuda.graph(gc, stream=stream):
                    for r in pool:
                        r.read(xs[T], out=outs[T], mean=means[T])
            torch.cuda.current_stream().wait_stream(stream)
            row[name] = round(timed(gc, args.per_t_reps, 2) * 1000.0 / (args.per_t_reps * len(pool)), 3)
            del gc
        cold_check[T] = row
        log(f"bench: cold check T={T}: {row}")
    del extra

    # the calibration leg: the read's two launches on the same grids and the same 32 rotated sets, empty, and
    # with only their global loads (include/hcr_calib.h), per T
    calibration = None
    if not args.no_calibration:
        cal = calib_lib()
        calibration = {"empty_pair_us": {}, "loads_pair_us": {}, "loads_store_pair_us": {}}
        for kind, key in ((0, "empty_pair_us"), (1, "loads_pair_us"), (2, "loads_store_pair_us")):
            for T in range(1, T_WIDE + 1):
                gk = torch.cuda.CUDAGraph()
                stream.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(stream):
                    with torch.cuda.graph(gk, stream=stream):
                        for r in readers * ROT:
                            rc = cal.hcrc_read_floor(kind, T, r.w_down.data_ptr(), r.w_up.data_ptr(),
                                                     r.w_norm.data_ptr(), r.scratch.data_ptr(), xs[T].data_ptr(),
                                                     stream.cuda_stream)
                            assert rc == hcr.HCR_OK, rc
                torch.cuda.current_stream().wait_stream(stream)
                calibration[key][T] = round(timed(gk, args.per_t_reps, 2) * 1000.0 / (args.per_t_reps * ROT * len(readers)), 3)
                del gk
            log(f"bench: calibration {key}: {calibration[key]}")
        # the pages' down shape (10 rows x a 1,280-column slab) and its last-arriver finish, as load / store /
        # finish probes (include/hcr_calib.h, hcrc_slab_pair), T = 1..8, one zero-filled slab scratch
        cal.hcrc_slab_pair.restype = ctypes.c_int
        cal.hcrc_slab_pair.argtypes = [ctypes.c_int, ctypes.c_int] + [ctypes.c_void_p] * 6
        slab_sc = torch.zeros(256 * 1024, dtype=torch.uint8, device=dev)
        for kind, key in ((0, "slab_loads_pair_us"), (1, "slab_stores_pair_us"), (2, "slab_finish_pair_us")):
            calibration[key] = {}
            for T in range(1, TMAX + 1):
                gk = torch.cuda.CUDAGraph()
                stream.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(stream):
                    with torch.cuda.graph(gk, stream=stream):
                        for r in readers * ROT:
                            rc = cal.hcrc_slab_pair(kind, T, r.w_down.data_ptr(), r.w_up.data_ptr(),
                                                    r.w_norm.data_ptr(), slab_sc.data_ptr(), xs[T].data_ptr(),
                                                    stream.cuda_stream)
                            assert rc == hcr.HCR_OK, rc
                torch.cuda.current_stream().wait_stream(stream)
                calibration[key][T] = round(timed(gk, args.per_t_reps, 2) * 1000.0 / (args.per_t_reps * ROT * len(readers)), 3)
                del gk
            log(f"bench: calibration {key}: {calibration[key]}")
        # the whole read in the pages' shape, with its arithmetic (hcrc_slab_read: slab down kernel, last-arriver
        # finish writing lo and rs, the read's up kernel on lo), the sweep's x, T = 1..8, beside per_T_us
        cal.hcrc_slab_read.restype = ctypes.c_int
        cal.hcrc_slab_read.argtypes = [ctypes.c_int] + [ctypes.c_void_p] * 10
        calibration["slab_read_us"] = {}
        for T in range(1, TMAX + 1):
            gk = torch.cuda.CUDAGraph()
            stream.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(stream):
                with torch.cuda.graph(gk, stream=stream):
                    for r in readers * ROT:
                        rc = cal.hcrc_slab_read(T, r.w_down.data_ptr(), r.w_up.data_ptr(), r.w_norm.data_ptr(),
                                                slab_sc.data_ptr(), xs[T].data_ptr(), None, None, outs[T].data_ptr(),
                                                means[T].data_ptr(), stream.cuda_stream)
                        assert rc == hcr.HCR_OK, rc
            torch.cuda.current_stream().wait_stream(stream)
            calibration["slab_read_us"][T] = round(timed(gk, args.per_t_reps, 2) * 1000.0 / (args.per_t_reps * ROT * len(readers)), 3)
            del gk
        log(f"bench: calibration slab_read_us: {calibration['slab_read_us']}")
        del slab_sc
        calibration["read_over_loads_us"] = {T: round(per_T_us[T] - calibration["loads_pair_us"][T], 3)
                                             for T in range(1, T_WIDE + 1)}
        # the two up kernels alone, per T (graphs of 32, each on a set's W_up and scratch): the read dispatches
        # the matrix-core one at every T
        cal.hcrc_up_kernel.restype = ctypes.c_int
        cal.hcrc_up_kernel.argtypes = [ctypes.c_int, ctypes.c_int] + [ctypes.c_void_p] * 5
        for kind, key in ((0, "up_valu_us"), (1, "up_mfma_us")):
            calibration[key] = {}
            for T in range(1, T_WIDE + 1):
                gk = torch.cuda.CUDAGraph()
                stream.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(stream):
                    with torch.cuda.graph(gk, stream=stream):
                        for r in readers * ROT:
                            rc = cal.hcrc_up_kernel(kind, T, r.w_up.data_ptr(), r.scratch.data_ptr(),
                                                    outs[T].data_ptr(), means[T].data_ptr(), stream.cuda_stream)
                            assert rc == hcr.HCR_OK, rc
                torch.cuda.current_stream().wait_stream(stream)
                calibration[key][T] = round(timed(gk, args.per_t_reps, 2) * 1000.0 / (args.per_t_reps * ROT * len(readers)), 3)
                del gk
            log(f"bench: calibration {key}: {calibration[key]}")
        calibration["note"] = ("per T, graphs of 32 pairs on the read's grids and work-group sizes over the 32 rotated "
                               "weight sets, replayed like the per-T figures: empty_pair = two empty kernels, "
                               "loads_pair = the read's global loads only (same order, widths and cache policy; no "
                               "arithmetic, LDS, barrier or store); loads_store_pair = loads_pair with one store per down "
                               "work-group; read_over_loads = per_T_us - loads_pair; slab_* = the pages' 10-row x "
                               "1,280-column down shape: its loads (up kernel loading lo only), + its partial stores, "
                               "+ the last-arriver finish (agent-scope acquire-release counter); slab_read = the whole read in "
                               "that shape with its arithmetic (slab partials, the finish applying rs and writing lo, "
                               "the read's up kernel on lo), µs per read beside per_T_us; "
                               "up_valu / up_mfma = the read's two up kernels alone, µs per launch")

    # the full epilogue (pending write and injection on) over the same 32 rotated weight sets: T = 4 with the
    # seeded x, pending and injection of the full-epilogue workload, and T = 8 with those of the numerics-stress
    # workload (heavy-tailed x); the weight values do not change the time of a read
    full_epilogue = {}
    for T, seed, xgen in ((4, 7, gen.activations), (TMAX, 5, gen.heavy_tailed_activations)):
        ex = [torch.from_numpy(xgen(seed, T, index=k)).to(dev) for k in range(len(readers))]
        ep = [torch.from_numpy(gen.pending(seed, T, index=k)).to(dev) for k in range(len(readers))]
        ei = [torch.from_numpy(gen.injection(seed, T, index=k)).to(dev) for k in range(len(readers))]
        ge = torch.cuda.CUDAGraph()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            with torch.cuda.graph(ge, stream=stream):
                for _ in range(ROT):
                    for k, r in enumerate(readers):
                        r.read(ex[k], ep[k], ei[k], out=outs[T], mean=means[T])
        torch.cuda.current_stream().wait_stream(stream)
        us = timed(ge, args.per_t_reps, 2) * 1000.0 / (args.per_t_reps * ROT * len(readers))
        full_epilogue[T] = {"us_per_read": round(us, 3),
                            "algorithmic_GBps": round(algorithmic_bytes(T, pending=True, inj=True) / us / 1e3, 1)}
        hashes.setdefault("full_epilogue", {})[T] = {"out": sha256_of(outs[T]), "mean": sha256_of(means[T])}
        d_out, d_mean = readers[-1].read(ex[-1], ep[-1], ei[-1])
        torch.cuda.synchronize()
        replay_equals_direct &= (sha256_of(d_out), sha256_of(d_mean)) == (hashes["full_epilogue"][T]["out"],
                                                                          hashes["full_epilogue"][T]["mean"])
        log(f"bench: full epilogue T={T} {us:.3f} us/read")
        del ge, ex, ep, ei
    full_epilogue["note"] = ("pending write and injection on, 32 rotated weight sets; T = 4: the full-epilogue "
                             "inputs (seed 7), T = 8: the numerics-stress inputs (seed 5); not part of the "
                             "timed step")

    # the timed steps: the whole sweep per step
    g = capture(range(1, TMAX + 1), len(readers))
    reads_per_step = TMAX * len(readers)
    timed(g, args.warmup, 0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms = timed(g, args.steps, 0, mark=True)
    wall = time.perf_counter() - t0
    ms_per_step = ms / args.steps
    us_per_read = ms_per_step * 1000.0 / reads_per_step
    bytes_step = sum(algorithmic_bytes(T) for T in range(1, TMAX + 1)) * len(readers)
    achieved = bytes_step / (ms_per_step * 1e-3) / 1e9
    log(f"bench: {args.steps} steps in {wall:.3f} s wall, {ms_per_step:.3f} ms/step, {us_per_read:.3f} us/read")
    if args.calibrate_copy:
        src = torch.ones(16 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("bench: calibration copy of 64 MiB done (4 launches)")
    traffic = measured_traffic("bf16")
    del g

    q8 = None
    if not args.no_q8:
        # Q8_0 copies of the 32 sets, made on the device, and 32 more copies of them in other memory:
        # 64 rotated sets (445 MB, more than the 256 MB MALL)
        log("bench: making the Q8_0 copies")
        qsets = []
        for r in readers:
            dc, ds = hcr.quantize_q8_0(r.w_down)
            uc, us = hcr.quantize_q8_0(r.w_up)
            qsets.append((dc, ds, uc, us, r.w_norm))
        qsets += [tuple(t.clone() for t in q) for q in qsets]
        q8_readers = [hcr.HCRead.q8_0(*q) for q in qsets]
        # the quantiser itself: both projections of each of the 32 sets (cold), as one graph
        gq = torch.cuda.CUDAGraph()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            with torch.cuda.graph(gq, stream=stream):
                for r, q in list(zip(readers, qsets)) * (ROT // 2):
                    for w, c, sc in ((r.w_down, q[0], q[1]), (r.w_up, q[2], q[3])):
                        rc = hcr.hcr_quantize_q8_0(w.data_ptr(), w.shape[0], w.shape[1], c.data_ptr(),
                                                   sc.data_ptr(), stream.cuda_stream)
                        assert rc == hcr.HCR_OK
        torch.cuda.current_stream().wait_stream(stream)
        q_us = timed(gq, 5, 1) * 1000.0 / (5 * 2 * (ROT // 2) * len(readers))
        del gq
        q_bytes = R * S * D * (2 + 1) + R * S * D // 32 * 2  # BF16 read, codes and scales written
        q8_T_us, q8_T_gbps = {}, {}
        for T in range(1, T_WIDE + 1):
            gq = torch.cuda.CUDAGraph()
            stream.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(stream):
                with torch.cuda.graph(gq, stream=stream):
                    for qr in q8_readers * (ROT // 2):
                        qr.read(xs[T], out=outs[T], mean=means[T])
            torch.cuda.current_stream().wait_stream(stream)
            us = timed(gq, args.per_t_reps, 2) * 1000.0 / (args.per_t_reps * (ROT // 2) * len(q8_readers))
            q8_T_us[T] = round(us, 3)
            q8_T_gbps[T] = round(algorithmic_bytes_q8(T) / us / 1e3, 1)
            if T <= TMAX:
                hashes.setdefault("q8_0", {})[T] = {"out": sha256_of(outs[T]), "mean": sha256_of(means[T])}
            log(f"bench: Q8_0 T={T} {us:.3f} us/read  {q8_T_gbps[T]:.0f} GB/s")
            del gq
        mean_us = sum(q8_T_us[T] for T in range(1, TMAX + 1)) / TMAX
        mean_bytes = sum(algorithmic_bytes_q8(T) for T in range(1, TMAX + 1)) / TMAX
        q8 = {"per_T_us": q8_T_us, "per_T_algorithmic_GBps": q8_T_gbps, "mean_us_T1_8": round(mean_us, 3),
              "weight_sets": len(q8_readers), "weight_bytes_per_read": algorithmic_bytes_q8(0) - S * D * 4,
              "roofline": {"bound": "hbm", "achieved": round(mean_bytes / mean_us / 1e3, 1), "peak": HBM_PEAK_GBPS,
                           "unit": "GB/s", "frac": round(mean_bytes / mean_us / 1e3 / HBM_PEAK_GBPS, 4),
                           "traffic": measured_traffic("q8_0")},
              "quantize_us_per_matrix": round(q_us, 3),
              "quantize_GBps": round(q_bytes / q_us / 1e3, 1),
              "note": "Q8_0 copies (GGML block rule) made on the device; 64 rotated sets; per-T graphs of 64 "
                      "reads replayed 10 times; not part of the timed step"}
        del q8_readers, qsets

    matvec = None
    if not args.no_matvec:
        # the skinny BF16 matvec, 12288 x 2560 (63 MB), 8 copies rotated (503 MB, more than the MALL)
        log("bench: generating the matvec weights")
        n_mv, rows, cols = 8, gen.MV_ROWS, gen.MV_COLS
        mw = [torch.from_numpy(gen.matvec_weights(30, k).view(np.int16)).to(dev) for k in range(n_mv)]
        mv_T_us, mv_T_gbps = {}, {}
        for T in range(1, gen.MV_T_MAX + 1):
            mx = torch.from_numpy(gen.matvec_x(30, T)).to(dev)
            my = torch.empty((T, rows), device=dev)
            gm = torch.cuda.CUDAGraph()
            stream.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(stream):
                with torch.cuda.graph(gm, stream=stream):
                    for k in list(range(n_mv)) * (4 * ROT):
                        rc = hcr.hcr_matvec_bf16(mw[k].data_ptr(), rows, cols, T, mx.data_ptr(), my.data_ptr(),
                                                 stream.cuda_stream)
                        assert rc == hcr.HCR_OK
            torch.cuda.current_stream().wait_stream(stream)
            reps = max(args.per_t_reps, 1)
            us = timed(gm, reps, 2) * 1000.0 / (reps * 4 * ROT * n_mv)
            b = rows * cols * 2 + T * cols * 4 + T * rows * 4
            mv_T_us[T] = round(us, 3)
            mv_T_gbps[T] = round(b / us / 1e3, 1)
            log(f"bench: matvec T={T} {us:.3f} us/call  {mv_T_gbps[T]:.0f} GB/s")
            del gm
        best = max(mv_T_gbps.values())
        matvec = {"shape": [rows, cols], "copies": n_mv, "per_T_us": mv_T_us, "per_T_algorithmic_GBps": mv_T_gbps,
                  "roofline": {"bound": "hbm", "achieved": round(sum(mv_T_gbps.values()) / len(mv_T_gbps), 1),
                               "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                               "frac": round(sum(mv_T_gbps.values()) / len(mv_T_gbps) / HBM_PEAK_GBPS, 4),
                               "best_frac": round(best / HBM_PEAK_GBPS, 4), "traffic": measured_matvec_traffic()},
                  "note": "y = W x, BF16 weights, 1..4 columns; graphs of 256 calls, 32 passes over the 8 rotated copies; "
                          "not part of the timed step"}
        del mw

    window = None
    if not args.no_window:
        # the verify window: 96 chained reads (out_i = x_{i+1}), distinct weight sets, T = 6, pending on
        n_win, t_win = 96, 6
        log(f"bench: generating the {n_win}-read verify window")
        cw = gen.verify_window(n_win, t_win)
        wreaders = [hcr.HCRead(torch.from_numpy(w.w_down.view(np.int16)).to(dev),
                               torch.from_numpy(w.w_up.view(np.int16)).to(dev),
                               torch.from_numpy(w.w_norm).to(dev)) for w in cw["weights"]]
        del cw["weights"]
        wpend = [torch.from_numpy(p_).to(dev) for p_ in cw["pending"]]
        wx0 = torch.from_numpy(cw["x0"]).to(dev)
        wouts = [torch.empty((t_win, S, D), device=dev) for _ in range(n_win)]
        wmeans = [torch.empty((t_win, D), device=dev) for _ in range(n_win)]
        gw = torch.cuda.CUDAGraph()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            with torch.cuda.graph(gw, stream=stream):
                xx = wx0
                for i, r in enumerate(wreaders):
                    r.read(xx, wpend[i], None, out=wouts[i], mean=wmeans[i])
                    xx = wouts[i]
        torch.cuda.current_stream().wait_stream(stream)
        reps = 50
        wms = timed(gw, reps, 3) / reps
        hashes["verify_window"] = {"out_last": sha256_of(wouts[-1]), "mean_last": sha256_of(wmeans[-1]),
                                   "means_all": sha256_of(*wmeans)}
        wbytes = n_win * algorithmic_bytes(t_win, pending=True)
        window = {"reads": n_win, "T": t_win, "pending": True, "us_per_window": round(wms * 1000, 2),
                  "us_per_read": round(wms * 1000 / n_win, 3),
                  "algorithmic_GBps": round(wbytes / (wms * 1e-3) / 1e9, 1),
                  "note": "one HIP graph of the 96-read residual chain, distinct BF16 weight sets (1.26 GB)"}
        log(f"bench: window {window['us_per_window']} us ({window['us_per_read']} us/read, "
            f"{window['algorithmic_GBps']} GB/s)")
        # the same window twice in one graph (the chain carried on through the same 96 sets): a replay of it
        # takes 2 W + b, one of the one-window graph W + b, so W and the replay boundary b follow
        g2 = torch.cuda.CUDAGraph()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g2, stream=stream):
                xx = wx0
                for i in range(2 * n_win):
                    wreaders[i % n_win].read(xx, wpend[i % n_win], None, out=wouts[i % n_win], mean=wmeans[i % n_win])
                    xx = wouts[i % n_win]
        torch.cuda.current_stream().wait_stream(stream)
        w2ms = timed(g2, reps // 2, 2) / (reps // 2)
        wms1 = timed(gw, reps, 2) / reps  # the one-window graph again, beside it
        del g2
        window["us_per_window_without_replay_boundary"] = round((w2ms - wms1) * 1000, 2)
        window["graph_replay_boundary_us"] = round((2 * wms1 - w2ms) * 1000, 2)
        window["replay_boundary_note"] = ("a graph of the window twice (192 chained reads) against the one-window "
                                          "graph, timed beside it: W = t2 - t1, boundary = 2 t1 - t2 (the runtime's "
                                          "cost of one graph replay, counted once in us_per_window)")
        log(f"bench: window without the replay boundary {window['us_per_window_without_replay_boundary']} us "
            f"(boundary {window['graph_replay_boundary_us']} us)")
        # the same chain with its weights resident in the MALL (16 sets, 210 MB, reused in turn): the bound
        # that prefetching the next read's weights into the MALL could reach
        del gw
        gh = torch.cuda.CUDAGraph()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            with torch.cuda.graph(gh, stream=stream):
                xx = wx0
                for i in range(n_win):
                    wreaders[i % 16].read(xx, wpend[i], None, out=wouts[i], mean=wmeans[i])
                    xx = wouts[i]
        torch.cuda.current_stream().wait_stream(stream)
        hms = timed(gh, reps, 3) / reps
        window["mall_resident_us_per_window"] = round(hms * 1000, 2)
        window["mall_resident_note"] = ("the same chain over 16 weight sets (210 MB, resident in the 256 MB MALL): "
                                        "the bound of prefetching the next read's weights into the MALL")
        log(f"bench: window with MALL-resident weights {window['mall_resident_us_per_window']} us")
        del gh
        # the same 96 reads (weights, pending write, T = 6) without the chain: every read takes x0, so the
        # chain's cost over independent reads is the difference
        gi = torch.cuda.CUDAGraph()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            with torch.cuda.graph(gi, stream=stream):
                for i, r in enumerate(wreaders):
                    r.read(wx0, wpend[i], None, out=wouts[i], mean=wmeans[i])
        torch.cuda.current_stream().wait_stream(stream)
        ims = timed(gi, reps, 3) / reps
        window["unchained_us_per_window"] = round(ims * 1000, 2)
        window["unchained_note"] = ("the same 96 reads (weights, pending write, T = 6) with x0 as every read's x: "
                                    "no residual chain")
        log(f"bench: the same reads unchained {window['unchained_us_per_window']} us")
        del gi

    line = {
        "metric": METRIC, "value": round(us_per_read, 3), "unit": "µs", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "cold HC read T sweep: 4 streams x 2560, R = 320, 32 rotated BF16 weight sets "
                               "(419 MB), T = 1..8, one read per set and T per step, HIP graph replay",
                   "reads_per_step": reads_per_step, "weight_sets": len(readers),
                   "arithmetic": "bf16 weights; fp32 accumulation (down: FMA on widened weights; up: "
                                 "v_mfma_f32_16x16x32_bf16 with lo "
                                 "split into bf16 high + low)",
                   "per_T_us": {T: v for T, v in per_T_us.items() if T <= TMAX},
                   "per_T_algorithmic_GBps": {T: v for T, v in per_T_gbps.items() if T <= TMAX},
                   "wide_windows_T9_16": {"per_T_us": {T: v for T, v in per_T_us.items() if T > TMAX},
                                          "per_T_algorithmic_GBps": {T: v for T, v in per_T_gbps.items()
                                                                     if T > TMAX},
                                          "note": "same cold rotation, not part of the timed step"},
                   "cold_cache_check_us_per_read": cold_check, "calibration": calibration,
                   "full_epilogue": full_epilogue,
                   "verify_window": window, "q8_0": q8, "matvec_bf16": matvec,
                   "output_sha256": hashes, "replay_equals_direct": bool(replay_equals_direct),
                   "output_sha256_note": "sha256 of the bytes of out and of mean after each graph (the last read: "
                                         "the last weight set); replay_equals_direct: the same reads made directly "
                                         "gave the same bytes"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": "the read (hc_down + hc_up_mfma dispatches), event-timed per read over the "
                               "timed region; "
                               "traffic = counter-measured HBM bytes per read (mean over T = 1..8)"},
    }
    if not args.no_cpu_baseline:
        log("bench: timing the FP64 reference on the host")
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
