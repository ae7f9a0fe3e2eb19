"""Benchmark of the StagQ batch-one GEMV on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--mode graph|stream|eager]
    python bench.py --sweep          every matrix of every workload
    python bench.py --read-sweep     plain-read launch shapes at the headline byte counts

Workload: the Llama-3.1-8B gate/up projection, W 14336 x 4096 (rows = output
channels), Student-t (nu = 4) weights scaled to std 0.02, group 128, base +
2 planes (2/3/4-bit prefixes), side record 0.1 % of the weights, x ~ N(0, 1)
fp16, batch one.  Weights are synthetic (seeded) and encoded by the library's
host encoder; nothing is read from disk.

The packed image is replicated (63 copies, over 1 GB at 2 bits) so that no
launch finds its bytes in the 256 MB Infinity Cache: every launch streams its
weights from HBM.  In graph mode (the default) one HIP graph per precision
holds one GEMV on every copy, and one step replays the three graphs (2, 3, 4
bits): 3 x 63 GEMVs.  A spin kernel queued ahead of the timed region keeps
the GPU busy while the host submits the replays, and timing events between
the replays, on the stream the kernels run on, give every replay's mean time
per launch.  --mode stream issues one GEMV per precision per step back to back
from Python; --mode eager brackets every launch with events.  Prints one JSON
line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, AMD public specification
METRIC = "µs per batch-1 GEMV and effective HBM GB/s (% of peak) at 2/3/4 bits"
A100_STAGQ_US = {2: 23.7, 3: 28.9, 4: 32.8}   # the paper's Table 8, 8B gate/up, A100 40 GB, g = 32
KERNEL_SRC = os.path.join(ROOT, "precision_weight_only_amd", "csrc", "stagq_device.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_14336x4096_traffic.md")


def kernel_source_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def read_traffic():
    """HBM bytes per launch measured by rocprofv3 counters (FETCH_SIZE, WRITE_SIZE),
    valid only while the kernel source is the one they were taken on."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    if not m or m.group(1) != kernel_source_hash():
        return None
    out = {}
    for b, val in re.findall(r"traffic_bytes_per_launch\[(\d)\]:\s*([0-9.eE+]+)", text):
        out[int(b)] = float(val)
    return out or None


def cpu_baseline(rows_sample: int = 1024, target_s: float = 10.0):
    """The oracle's float64 decode + matvec on the host, on a row sample of the
    same workload (oracle-encoded), repeated for about target_s seconds with
    the host's BLAS threads, then again on one thread (reported in the sample
    text)."""
    import oracle
    from workloads import WORKLOADS, synth_matrix
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:
        blas = 1
    wl = WORKLOADS["mlp"]
    w, x = synth_matrix(rows_sample, 4096, wl.dist, 0)
    te = time.perf_counter()
    F = oracle.encode(w, wl.group, wl.nbits, wl.frac, wl.ratio_T)
    t_encode = time.perf_counter() - te
    G = 4096 // wl.group
    nbytes = {M: rows_sample * 4096 * M // 8 + rows_sample * G * 4 + (rows_sample + 1) * 4 + F.nnz * 8
              + 4096 * 2 + rows_sample * 4 for M in wl.bits}
    round_bytes = sum(nbytes.values())

    def timed(seconds):
        t0 = time.perf_counter()
        rounds = []
        while time.perf_counter() - t0 < seconds or len(rounds) < 3:
            r0 = time.perf_counter()
            for M in wl.bits:
                oracle.gemv(F, x, M)
            rounds.append(time.perf_counter() - r0)
        return len(rounds) * round_bytes / sum(rounds) / 1e9, len(rounds), sum(rounds), float(np.median(rounds))

    gbs, done, dt, med = timed(target_s)
    one = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1, user_api="blas"):
            one = timed(target_s / 2)
    except Exception:
        pass
    one_txt = (f"; on 1 thread {one[0]:.4f} GB/s ({one[1]} rounds, median round {one[3] * 1e3:.1f} ms)"
               if one else "")
    return {
        "value": round(gbs, 4), "unit": "GB/s", "cores": int(blas), "kind": "oracle",
        "sample": f"{rows_sample}x4096 rows of the same Student-t workload (oracle-encoded), "
                  f"float64 decode (Eq. 9) + side record + matvec at bits 2,3,4, {done} rounds in {dt:.1f} s, "
                  f"median round {med * 1e3:.1f} ms; elementwise NumPy on 1 thread, BLAS matvec on {blas} "
                  f"threads{one_txt}; the one-time oracle encode of the sample (not in the rate) "
                  f"took {t_encode:.2f} s; host has {os.cpu_count()} logical CPUs",
    }


INFINITY_CACHE_BYTES = 256 << 20   # MI355X last-level (Infinity) cache


def rotation_copies(rot_mb: int, bytes_per_launch: int, minimum: int = 2) -> int:
    """Image copies a timed run cycles through: enough that the bytes all copies
    give the lowest precision read exceed rot_mb MB, which must be at least four
    times the Infinity Cache, so no launch finds its bytes there (the FETCH_SIZE
    counters count cache hits too; the rotation is what makes them HBM bytes)."""
    if rot_mb * (1 << 20) < 4 * INFINITY_CACHE_BYTES:
        raise ValueError(f"--rot-mb {rot_mb} is below 4 x the {INFINITY_CACHE_BYTES >> 20} MB Infinity Cache")
    n = max(minimum, -(-rot_mb * (1 << 20) // bytes_per_launch))
    assert n * bytes_per_launch >= 4 * INFINITY_CACHE_BYTES
    return n


def busy_gpu(ms: float = 2.0) -> None:
    """Queue a spin kernel of about ms milliseconds on the current stream, so the
    launches queued behind it (while it spins) start back to back instead of
    waiting for the host to submit them."""
    import torch
    try:
        torch.cuda._sleep(int(ms * 1e6))
    except Exception:                    # no spin kernel in this build: a few large fills
        buf = torch.empty(64 << 20, dtype=torch.float32, device="cuda")
        for _ in range(max(1, int(ms * 4))):
            buf.fill_(1.0)


def graph_time(launch, n_copies, K, bits_seq):
    """Mean microseconds per launch over about K launches: one HIP graph holds
    n_copies launches (launch i on copy i with precision bits_seq[i % len]),
    replayed ceil(K / n_copies) times behind a spin kernel, with timing events
    around the replays on the stream the kernels run on."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n_copies):
            launch(i, bits_seq[i % len(bits_seq)])
    g.replay()
    torch.cuda.synchronize()
    reps = max(1, -(-K // n_copies))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    busy_gpu()
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * n_copies)


def eager_time(launch, n_copies, K, bits_seq):
    """Mean microseconds per launch of K launches issued from Python (launch i
    on copy i % n_copies, precision bits_seq[i % len]), one event pair around
    them: a run that rocprofv3 counter collection can split per dispatch."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(K):
        launch(i % n_copies, bits_seq[i % len(bits_seq)])
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / K


def cpu_baseline_sweep(args):
    """The oracle (float64 decode by Eq. 9, side record, BLAS matvec) timed per
    configuration shape and precision on the host: median of 3 calls with the
    host's BLAS threads and one call on a single thread.  Fields come from the
    oracle's own encoder (not timed).  One JSON line."""
    import oracle
    from workloads import WORKLOADS, synth_matrix
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        blas = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:
        threadpool_limits, blas = None, 1
    cpu = ""
    try:
        cpu = next(ln.split(":", 1)[1].strip() for ln in open("/proc/cpuinfo") if ln.startswith("model name"))
    except Exception:
        pass
    picks = [("tiny", "W"), ("attn", "qkvo"), ("layer_sweep", "k"), ("mlp", "gate_up"), ("mlp", "down"),
             ("phi4_mlp", "gate_up"), ("phi4_mlp", "down"), ("layer_sweep", "lm_head")]
    if args.workloads:
        picks = [p for p in picks if p[0] in args.workloads.split(",")]
    out = []
    for wname, mname in picks:
        wl = WORKLOADS[wname]
        mat = [m for m in wl.matrices if m.name == mname][0]
        w, x = synth_matrix(mat.rows, mat.cols, wl.dist, mat.seed)
        t0 = time.perf_counter()
        F = oracle.encode(w, wl.group, wl.nbits, wl.frac, wl.ratio_T)
        t_enc = time.perf_counter() - t0
        del w
        for M in wl.bits:
            runs = []
            for _ in range(3):
                r0 = time.perf_counter()
                oracle.gemv(F, x, M)
                runs.append(time.perf_counter() - r0)
            one = None
            if threadpool_limits is not None:
                with threadpool_limits(limits=1, user_api="blas"):
                    r0 = time.perf_counter()
                    oracle.gemv(F, x, M)
                    one = time.perf_counter() - r0
            row = {"workload": wname, "matrix": mname, "rows": mat.rows, "cols": mat.cols, "bits": M,
                   "us_all_threads": round(float(np.median(runs)) * 1e6, 1),
                   "us_one_thread": round(one * 1e6, 1) if one else None, "encode_s": round(t_enc, 2)}
            out.append(row)
            print(f"[oracle] {wname}/{mname} {mat.rows}x{mat.cols} bits={M}: {row['us_all_threads']} us "
                  f"({row['us_one_thread']} us on 1 thread)", file=sys.stderr, flush=True)
        del F
    print(json.dumps({"oracle_sweep": out, "blas_threads": int(blas), "cpu_count": os.cpu_count(),
                      "affinity": len(os.sched_getaffinity(0)), "cpu_model": cpu}), flush=True)


def codebook_fields(fields):
    """Timing workload for codebook metadata at full size: two uniform 16-entry
    codebooks over the range of the encoder's pairs (log2 s and lo/s) and per
    group the nearest index; lo, s become the pairs the indices select.  (The
    per-group Eq. 5 choice is the oracle's and is parity-tested on smaller
    shapes; the GEMV's cost does not depend on which index a group holds.)"""
    lo = fields["lo"].astype(np.float64)
    s = fields["s"].astype(np.float64)
    pos = s > 0
    L, P = np.log2(s[pos]), lo[pos] / s[pos]
    t = np.arange(16) / 15.0
    cs = (L.min() + t * (L.max() - L.min())).astype(np.float16)
    cr = (P.min() + t * (P.max() - P.min())).astype(np.float16)
    ts = np.exp2(cs.astype(np.float64)).astype(np.float16)
    i = np.abs(np.log2(np.where(pos, s, 1.0))[..., None] - cs.astype(np.float64)).argmin(-1)
    sv = ts[i].astype(np.float64)
    j = np.abs((lo / sv)[..., None] - cr.astype(np.float64)).argmin(-1)
    out = dict(fields)
    out.update(idx=(i * 16 + j).astype(np.uint8), cb_log2s=cs, cb_ratio=cr, s=ts[i],
               lo=(cr.astype(np.float64)[j] * sv).astype(np.float16))
    return out


def read_ceiling(bytes_alg, args):
    """Streaming-read ceiling per precision: a plain read of the same byte
    count (stagq_stream_read), K launches in one graph cycling through fresh
    windows of a pool larger than --rot-mb, timed like the GEMV."""
    import torch
    import precision_weight_only_amd as pwo
    out = {}
    pool_bytes = (max(args.rot_mb, 256) << 20) + (max(bytes_alg.values()) + 4096)
    pool = torch.empty(pool_bytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for M, b in bytes_alg.items():
        win = (b + 4095) // 4096 * 4096
        nwin = max(2, (pool_bytes - 4096) // win)

        def launch(i, _M, b=b, win=win, nwin=nwin):
            pwo.stream_read(pool, (i % nwin) * win, b, sink)

        for i in range(args.warmup):
            launch(i, M)
        torch.cuda.synchronize()
        us = graph_time(launch, nwin, args.steps, [M])
        out[M] = {"us": round(us, 3), "bytes": int(b), "gbps": round(b / us / 1e3, 1),
                  "pct_peak": round(100 * b / us / 1e3 / PEAK_HBM_GBS, 2)}
    del pool
    return out


def read_sweep(args):
    """Plain reads (stagq_stream_read_shape) of the headline GEMV's byte counts at
    2, 3, 4 bits and of the LM head's at 2 and 4 bits, over threads per
    workgroup x 16-byte loads per thread in flight x workgroups (0 = one pass,
    else a persistent grid of that many), each timed like the GEMV: one graph
    of launches on fresh windows of a 1.5 GB pool, replayed behind a spin
    kernel.  One JSON line: every shape's microseconds and the best per size."""
    import torch
    import precision_weight_only_amd as pwo
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    def alg_bytes(R, C, M, g=128, frac=0.001):   # as stagq_query reports for a CSR image with fp16 pairs
        nnz = int(np.floor(frac * R * C + 0.5))
        return R * C * M // 8 + R * (C // g) * 4 + nnz * 8 + (R + 1) * 4 + C * 2 + R * 4
    sizes = {"gemv_2bit": alg_bytes(14336, 4096, 2), "gemv_3bit": alg_bytes(14336, 4096, 3),
             "gemv_4bit": alg_bytes(14336, 4096, 4), "lm_head_2bit": alg_bytes(128256, 4096, 2),
             "lm_head_4bit": alg_bytes(128256, 4096, 4)}
    pool_bytes = 1536 << 20
    pool = torch.empty(pool_bytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    rows, best = [], {}
    for name, b in sizes.items():
        win = (b + 4095) // 4096 * 4096
        nwin = max(2, min(64, pool_bytes // win))
        for threads in (256, 512, 1024):
            for loads in (1, 2, 4, 8, 16):
                for grid in (0, cus, 2 * cus, 4 * cus, 8 * cus):
                    def launch(i, _M, b=b, win=win, nwin=nwin, t=threads, l=loads, g=grid):
                        pwo.stream_read_shape(pool, (i % nwin) * win, b, sink, t, l, g)
                    us = graph_time(launch, nwin, max(args.steps, 2 * nwin), [0])
                    one_pass = -(-b // (threads * loads * 16))
                    r = {"size": name, "bytes": b, "threads": threads, "loads": loads,
                         "grid": min(grid, one_pass) if grid else one_pass, "persistent": bool(grid and grid < one_pass),
                         "us": round(us, 3), "pct_peak": round(100 * b / us / 1e3 / PEAK_HBM_GBS, 2)}
                    rows.append(r)
                    if name not in best or us < best[name]["us"]:
                        best[name] = r
        print(f"[read-sweep] {name}: best {best[name]}", file=sys.stderr, flush=True)
    print(json.dumps({"read_sweep": rows, "best": best, "cus": cus}), flush=True)


def sweep(args):
    """Every matrix of the attention, MLP, Phi-4 and layer-sweep workloads at each
    precision (one graph of K launches per precision, rotating image copies),
    plus the layer sweep's per-call precision switching 2, 3, 4, 2, ...; one JSON line."""
    import torch
    import precision_weight_only_amd as pwo
    from workloads import WORKLOADS, synth_matrix
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    rows = []
    timer = graph_time if args.mode == "graph" else eager_time
    names = ("attn", "mlp", "mlp_rows", "phi4_mlp", "layer_sweep")
    if args.workloads:
        names = tuple(n for n in names if n in args.workloads.split(","))
    for wname in names:
        wl = WORKLOADS[wname]
        for mat in wl.matrices:
            w, x = synth_matrix(mat.rows, mat.cols, wl.dist, mat.seed)
            K = int(np.floor(wl.frac * mat.rows * mat.cols + 0.5))
            fields = pwo.encode(w, wl.group, wl.nbits, K, wl.ratio_T, post_per_row=wl.post_per_row)
            del w
            base = pwo.StagQMatrix.pack(fields, device=dev)
            slm = pwo.StagQMatrix.pack(fields, device=dev, side_slots=-1) if wl.post_per_row and not args.plain else None
            cbm = pwo.StagQMatrix.pack(codebook_fields(fields), device=dev) if wname == "mlp" and not args.plain else None
            del fields
            n_copies = rotation_copies(args.rot_mb, base.bytes_read[min(wl.bits)])
            copies = [base] + [base.replicate() for _ in range(n_copies - 1)]
            xd = torch.from_numpy(x.view(np.int16)).view(torch.float16).to(dev)
            ys = [torch.empty(mat.rows, dtype=torch.float32, device=dev) for _ in range(n_copies)]

            def launch(c, M):
                copies[c].gemv(xd, M, y=ys[c])

            for i in range(args.warmup):
                launch(i % n_copies, wl.bits[i % len(wl.bits)])
            torch.cuda.synchronize()
            entry = {"workload": wname, "matrix": mat.name, "rows": mat.rows, "cols": mat.cols,
                     "nnz": int(base.nnz), "copies": n_copies, "bits": {}}
            for M in wl.bits:
                us = timer(launch, n_copies, args.steps, [M])
                b = base.bytes_read[M]
                entry["bits"][str(M)] = {"us": round(us, 3), "bytes": int(b), "gbps": round(b / us / 1e3, 1),
                                         "pct_peak": round(100 * b / us / 1e3 / PEAK_HBM_GBS, 2),
                                         "launch": base.plan(M)}
            if wname == "mlp" and not args.plain:
                # the same GEMVs with the inverse AWQ scale applied to x (stagq_gemv_scaled)
                sc = torch.from_numpy(np.full(mat.cols, 0.5, np.float16).view(np.int16)).view(torch.float16).to(dev)

                def launch_sc(c, M):
                    copies[c].gemv(xd, M, y=ys[c], x_scale=sc)

                for M in wl.bits:
                    us = timer(launch_sc, n_copies, args.steps, [M])
                    entry["bits"][str(M)]["awq_scaled_us"] = round(us, 3)
                # the same GEMVs with an fp16 result (stagq_gemv_f16)
                y16 = [torch.empty(mat.rows, dtype=torch.float16, device=dev) for _ in range(n_copies)]

                def launch_h(c, M):
                    copies[c].gemv(xd, M, y=y16[c])

                for M in wl.bits:
                    us = timer(launch_h, n_copies, args.steps, [M])
                    entry["bits"][str(M)]["fp16_out_us"] = round(us, 3)
                del y16
                # the same GEMVs on codebook metadata (1 byte per group + 256 pairs)
                cbc = [cbm] + [cbm.replicate() for _ in range(n_copies - 1)]

                def launch_cb(c, M):
                    cbc[c].gemv(xd, M, y=ys[c])

                for M in wl.bits:
                    us = timer(launch_cb, n_copies, args.steps, [M])
                    b = cbm.bytes_read[M]
                    entry["bits"][str(M)]["codebook"] = {"us": round(us, 3), "bytes": int(b),
                                                         "pct_peak": round(100 * b / us / 1e3 / PEAK_HBM_GBS, 2)}
                del cbc, cbm
            if slm is not None:
                # the same fields with the side record in fixed per-row slots
                slc = [slm] + [slm.replicate() for _ in range(n_copies - 1)]

                def launch_sl(c, M):
                    slc[c].gemv(xd, M, y=ys[c])

                for M in wl.bits:
                    us = timer(launch_sl, n_copies, args.steps, [M])
                    b = slm.bytes_read[M]
                    entry["bits"][str(M)]["slots"] = {"us": round(us, 3), "bytes": int(b), "W": slm.side_slots,
                                                      "pct_peak": round(100 * b / us / 1e3 / PEAK_HBM_GBS, 2)}
                del slc
            del slm
            if wname == "layer_sweep" and not args.plain:
                us = timer(launch, n_copies, args.steps, list(wl.bits))
                b = sum(base.bytes_read[M] for M in wl.bits) / len(wl.bits)
                entry["switched_2_3_4"] = {"us_per_call": round(us, 3), "gbps": round(b / us / 1e3, 1)}
            rows.append(entry)
            print(f"[sweep] {wname}/{mat.name} {mat.rows}x{mat.cols}: " +
                  " ".join(f"{M}b {v['us']}us {v['pct_peak']}%" +
                           (f" (awq {v['awq_scaled_us']}us)" if "awq_scaled_us" in v else "") +
                           (f" (fp16 out {v['fp16_out_us']}us)" if "fp16_out_us" in v else "") +
                           (f" (codebook {v['codebook']['us']}us)" if "codebook" in v else "") +
                           (f" (slots W={v['slots']['W']} {v['slots']['us']}us)" if "slots" in v else "")
                           for M, v in entry["bits"].items()),
                  file=sys.stderr, flush=True)
            del copies, base, ys
            torch.cuda.empty_cache()
    print(json.dumps({"metric": METRIC, "sweep": rows, "steps": args.steps, "warmup": args.warmup,
                      "mode": args.mode, "data": "synthetic"}), flush=True)


HEADLINE = ("mlp", "gate_up")      # the Llama-3.1-8B gate/up projection, 14336 x 4096


def make_line(args, mat, wl, dur, bytes_alg, wall, launches_per_step, n_copies, ceiling, plans, nnz,
              image_bytes):
    """The JSON line: per-precision timing (dur[M] = microseconds per launch,
    one value per timed replay or launch), the whole-job rate and the roofline
    of the dominant launch (the 4-bit GEMV, which moves the most bytes)."""
    bits = list(wl.bits)
    K = args.steps
    per_bits = {}
    for M in bits:
        d = np.array(dur[M], dtype=np.float64)
        mean = float(d.mean())
        per_bits[str(M)] = {
            "us_mean": round(mean, 3), "us_median": round(float(np.median(d)), 3),
            "us_p10": round(float(np.percentile(d, 10)), 3), "us_p90": round(float(np.percentile(d, 90)), 3),
            "bytes": int(bytes_alg[M]),
            "gbps": round(bytes_alg[M] / (mean * 1e-6) / 1e9, 1),
            "pct_peak": round(100.0 * bytes_alg[M] / (mean * 1e-6) / 1e9 / PEAK_HBM_GBS, 2),
            "a100_stagq_us": A100_STAGQ_US[M],
            "read_ceiling": ceiling.get(M),
            "launch": plans.get(M),
        }
    step_bytes = sum(bytes_alg.values()) * launches_per_step
    value = step_bytes * K / wall / 1e9
    traffic = read_traffic()
    dom = max(bits)
    ach = per_bits[str(dom)]["gbps"]
    roofline = {
        "bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
        "frac": round(ach / PEAK_HBM_GBS, 4),
        "traffic": (traffic or {}).get(dom),
        "kernel": f"the {dom}-bit GEMV launch (gemv_kernel, M = {dom})",
        "by_bits": {str(M): {"achieved": per_bits[str(M)]["gbps"],
                             "frac": round(per_bits[str(M)]["gbps"] / PEAK_HBM_GBS, 4),
                             "traffic": (traffic or {}).get(M),
                             "read_ceiling_gbps": (ceiling.get(M) or {}).get("gbps")} for M in bits},
    }
    step = (f"one GEMV at each of 2, 3, 4 bits on each of the {n_copies} image copies "
            f"({3 * launches_per_step} GEMVs), as three HIP graph replays" if launches_per_step > 1 else
            "one GEMV at each of 2, 3, 4 bits, each on its own image copy")
    return {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(wall / K * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic",
        "config": {"workload": f"Llama-3.1-8B gate/up GEMV {mat.rows}x{mat.cols}, Student-t(4) std 0.02, "
                               f"g={wl.group}, base + {wl.nbits - 2} planes, side record {100 * wl.frac:g}%, batch 1",
                   "rows": mat.rows, "cols": mat.cols, "group": wl.group, "nbits": wl.nbits, "bits": bits,
                   "side_record_nnz": nnz, "image_bytes": image_bytes,
                   "rotation_copies": n_copies, "mode": args.mode, "gemvs_per_step": 3 * launches_per_step,
                   "step": step},
        "per_bits": per_bits,
        "roofline": roofline,
        "kernel_source_sha256_16": kernel_source_hash(),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--mode", choices=("graph", "stream", "eager"), default="graph",
                    help="graph: K launches per precision captured in one HIP graph; stream: the "
                         "same K launches issued back to back with one event pair around them; "
                         "eager: an event pair around every launch")
    ap.add_argument("--rot-mb", type=int, default=1024,
                    help="bytes (MB) the rotated image copies hold at the lowest precision read: "
                         "every precision cycles through all copies, so at least this much is "
                         "streamed between two reads of one copy (4x the 256 MB Infinity Cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="time every matrix of every workload instead of the headline line")
    ap.add_argument("--workloads", default="",
                    help="--sweep / --oracle-sweep: comma-separated workload names to run (default all)")
    ap.add_argument("--plain", action="store_true",
                    help="--sweep: only the plain GEMV per matrix (no AWQ, fp16-output, codebook, slot "
                         "or switched-precision variants)")
    ap.add_argument("--oracle-sweep", action="store_true",
                    help="time the CPU oracle per configuration shape and precision (host only)")
    ap.add_argument("--read-sweep", action="store_true",
                    help="time plain reads of the headline byte counts and of the LM head's over a "
                         "grid of launch shapes (threads, loads in flight, workgroups)")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="also run 5 device-to-device copies of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: the GEMV runs on one GPU only; --gpus must be 1 (the GEMV path has "
              "no multi-GPU leg).", file=sys.stderr)
        sys.exit(2)

    if args.oracle_sweep:
        cpu_baseline_sweep(args)
        return

    import torch
    import precision_weight_only_amd as pwo
    from workloads import WORKLOADS, synth_matrix

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.sweep:
        sweep(args)
        return
    if args.read_sweep:
        read_sweep(args)
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = WORKLOADS[HEADLINE[0]]
    mat = [m for m in wl.matrices if m.name == HEADLINE[1]][0]
    R, Cc = mat.rows, mat.cols
    bits = list(wl.bits)

    t0 = time.time()
    w, x = synth_matrix(R, Cc, wl.dist, mat.seed)
    side_budget = int(np.floor(wl.frac * R * Cc + 0.5))
    fields = pwo.encode(w, wl.group, wl.nbits, side_budget, wl.ratio_T)
    base = pwo.StagQMatrix.pack(fields, device=dev)
    # Enough copies that the lowest precision's reads of all of them exceed
    # the rotation size, and every precision cycles through all of them.
    n_copies = rotation_copies(args.rot_mb, base.bytes_read[min(bits)], minimum=6)
    copies = [base] + [base.replicate() for _ in range(n_copies - 1)]
    xd = torch.from_numpy(x.view(np.int16)).view(torch.float16).to(dev)
    ys = [torch.empty(R, dtype=torch.float32, device=dev) for _ in range(n_copies)]
    setup_s = time.time() - t0
    stream = torch.cuda.current_stream()

    def launch(i, M):
        c = i % n_copies
        copies[c].gemv(xd, M, y=ys[c])

    if args.calib_copy_mb:
        # A plain copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters.
        src = torch.ones(args.calib_copy_mb << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # warmup (also loads the code objects)
    for s in range(args.warmup):
        for j, M in enumerate(bits):
            launch(3 * s + j, M)
    torch.cuda.synchronize()

    K = args.steps
    # launch ids per precision: each precision cycles through every copy
    order = {M: [j * K + s for s in range(K)] for j, M in enumerate(bits)}
    dur = {M: [] for M in bits}
    launches_per_step = 1          # GEMVs per precision in one step

    if args.mode == "graph":
        # One HIP graph per precision holds one launch on every image copy
        # (n_copies launches); a step replays the three graphs, precisions
        # interleaved (2, 3, 4), so a step is n_copies GEMVs at each precision
        # and every graph is as long whatever K is.  A spin kernel ahead of the
        # first timing event keeps the GPU busy while the host submits the
        # replays, so no launch waits for the host; timing events between the
        # replays, on the stream the kernels run on, give each replay's mean
        # microseconds per launch.
        graphs = {}
        for M in bits:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for c in range(n_copies):
                    launch(c, M)
            graphs[M] = g
            g.replay()
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            for M in bits:
                graphs[M].replay()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(K * len(bits) + 1)]
        torch.cuda.synchronize()
        busy_gpu()
        t_start = time.perf_counter()
        evs[0].record()
        n = 0
        for s in range(K):
            for M in bits:
                graphs[M].replay()
                n += 1
                evs[n].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_start
        for j, M in enumerate(bits):
            dur[M] = [evs[s * len(bits) + j].elapsed_time(evs[s * len(bits) + j + 1]) * 1e3 / n_copies
                      for s in range(K)]                                  # microseconds per launch
        launches_per_step = n_copies
    elif args.mode == "stream":
        # The K launches of a precision issued back to back, events around them.
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(bits) + 1)]
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        evs[0].record()
        for j, M in enumerate(bits):
            for i in order[M]:
                launch(i, M)
            evs[j + 1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_start
        for j, M in enumerate(bits):
            dur[M] = [evs[j].elapsed_time(evs[j + 1]) * 1e3 / K] * K
    else:
        # Eager launches with a timing event pair around every launch.
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(3 * K)]
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for s in range(K):
            for j, M in enumerate(bits):
                i = order[M][s]
                ev[i][0].record()
                launch(i, M)
                ev[i][1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_start
        for j, M in enumerate(bits):
            dur[M] = [ev[i][0].elapsed_time(ev[i][1]) * 1e3 for i in order[M]]

    bytes_alg = {M: base.bytes_read[M] for M in bits}
    ceiling = read_ceiling(bytes_alg, args) if args.mode == "graph" else {}
    out = make_line(args, mat, wl, dur, bytes_alg, wall, launches_per_step, n_copies, ceiling,
                    {M: base.plan(M) for M in bits}, int(base.nnz), int(base.image_bytes))
    out["setup_s"] = round(setup_s, 2)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
