"""Throughput of the QAM-W codec on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step = the whole codec path over one matrix already resident in HBM:
qamw_build_plan (search plan for the codebook, on a second stream) beside
qamw_calibrate_prepare (s, sigma, row norms), then qamw_encode_indices
(rotation, nearest centroid, packing) -> qamw_decode (fp32 output).  The same work is then timed as separate entry points (qamw_calibrate,
qamw_encode_prepare, qamw_encode_indices) for per-kernel figures.  The default workload is the 4096 x 11008 bf16
down-projection-shaped matrix (Student-t(5) entries, std 0.02; K = 2048,
Hadamard block 256).  Prints one JSON line.

value         weights per second of the whole step (Gweights/s), the step
              replayed as a HIP graph with inputs resident in HBM
cold_step     the same replays after a 1 GiB read each (L2 and MALL cold)
roofline      the dominant kernel (encode_lds_kernel, all of
              qamw_encode_indices with a plan): algorithmic HBM bytes (W read
              + packed write) / its mean launch time from HIP events on the
              launch stream (10 launches in a HIP graph, mean per launch),
              against 8 TB/s; traffic from the committed
              counter passes when they match the kernel sources
valu_view     the exhaustive search (no plan) against the fp32 vector peak,
              and the planned search's speedup over it in those units
decode_cold   decode alone after a 1 GiB read, next to a plain fill of the
              same output bytes under the same protocol (also for 16 bits):
              one eager launch, and per launch of a graph of 8 decodes over
              distinct buffers (no launch latency, every byte from/to HBM)
c4_sweep      the 5120 x 13824 bf16 matrix at K = 256 / 1024 / 2048 / 4096
              and alpha = 0 / 0.5: plan, calibrate + encode, decode per variant
c5_stack      the 7B-shaped stack (32 layers x q, k, v, o, gate, up, down):
              calibrate + encode every matrix, then decode every matrix
parity        sampled rows of the step's outputs against the fp64 oracle
              (near ties, mismatches, row-norm bits, decode error)
cpu_baseline  the fp64 NumPy oracle on a 640-row sample of the same workload
              (calibrate + encode + decode), split over the host's cores, and
              on 64 rows in one thread
decode_matmul the fused decoded-weight matmul Y = X W^^T on the packed matrix
              for T tokens, against decode-to-bf16 + torch.matmul (not part
              of the step)
polar         the polar-code baseline encode (qamw_encode_polar, 8 amplitude
              levels x 32 phases = 8 bits per pair) on the same matrix with
              the step's s and sigma (not part of the step)
learned_codebook  Lloyd rounds of the codebook on the matrix's own normalised
              pairs (qamw_learn_codebook: plan, encode, update per round) from
              the Gaussian codebook: distortion per round, time per round,
              reconstruction error before and after (not part of the step)
alpha_sweep   channel RMS of synthetic activations X (qamw_channel_rms), then
              for alpha in 0 .. 1: calibrate, encode, decode and the layer-
              output error ||X dW^T||^2 (qamw_output_error, bf16 MFMA); the
              times of the two metric kernels (not part of the step)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads  # noqa: E402

PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
KERNEL_SOURCES = [os.path.join(ROOT, "vector_codebook_codec_amd", "csrc", f)
                  for f in ("encode.hip", "encode_window.h", "qamw_device.h", "qamw_internal.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "encode_lds_kernel_4096x11008_traffic.txt")


def workload_entries(name: str) -> str:
    """The weight and channel-RMS distributions of a named workload."""
    if name.startswith("c1_"):
        return "N(0, 0.02^2), r~LogNormal(0,0.5)"
    if name.startswith("c2_"):
        return "N(0, 0.02^2) with 1% of columns x8, r~LogNormal(0,1)"
    if name.startswith("c3"):
        return "Student-t(5) std 0.02, r~LogNormal(0,1.2)"
    if name.startswith("c4_"):
        return "N(0, 0.015^2), r~LogNormal(0,1)"
    return "Student-t(5) std 0.02, r~LogNormal(0,1)"


def measured_traffic(workload):
    """Encode-kernel HBM bytes per launch from the committed counter passes,
    or None when they were taken on other kernel sources or another workload."""
    import hashlib

    try:
        kv = {}
        for line in open(TRAFFIC_FILE):
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
        sha = hashlib.sha256(b"".join(open(f, "rb").read() for f in KERNEL_SOURCES)).hexdigest()
    except OSError:
        return None
    if kv.get("source_sha256") != sha or kv.get("workload") != workload:
        return None
    return 1024.0 * (float(kv["fetch_kib"]) * float(kv["fetch_scale"]) +
                     float(kv["write_kib"]) * float(kv["write_scale"]))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c3t_4096x11008")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--parity-rows", type=int, default=64,
                    help="rows of the step's output checked against the oracle (0 to skip)")
    ap.add_argument("--cold-steps", type=int, default=10,
                    help="steps timed after a 1 GiB read each (0 to skip)")
    ap.add_argument("--sweep-c4", type=int, default=1,
                    help="time the 5120 x 13824 K / alpha sweep (0 to skip)")
    ap.add_argument("--stack-layers", type=int, default=32,
                    help="layers of the 7B-shaped stack timed end to end (0 to skip)")
    ap.add_argument("--cold-decode-reps", type=int, default=10,
                    help="decode-only reps timed after overwriting a 1 GiB buffer")
    ap.add_argument("--exhaustive-reps", type=int, default=5,
                    help="encodes without a search plan timed after the steps (0 to skip)")
    ap.add_argument("--matmul-tokens", type=int, nargs="*", default=[1, 16, 64],
                    help="token counts T of the fused decoded-weight matmul measurement")
    ap.add_argument("--matmul-reps", type=int, default=10)
    ap.add_argument("--sweep-tokens", type=int, default=1024,
                    help="synthetic activation rows for the channel-RMS / output-error alpha sweep (0 to skip)")
    ap.add_argument("--learn-iters", type=int, default=3,
                    help="Lloyd rounds of the codebook refinement on the matrix's own pairs (0 to skip)")
    ap.add_argument("--polar-reps", type=int, default=10,
                    help="polar-code encodes (8 amplitudes x 32 phases) timed after the steps (0 to skip)")
    ap.add_argument("--copy-reference", type=int, default=0,
                    help="also run N copies of a 1 GiB buffer (counter calibration)")
    return ap.parse_args()


def _oracle_rows(task):
    """One worker's share of an oracle run: encode (and decode) rows of W with
    the given calibration; returns what the caller asked for."""
    from oracle import qamw_ref as O

    Wr, s, sig, b, seed, C, d, want = task
    enc = O.encode(Wr, s, sig, b, seed, C)
    out = {"idx": enc["idx"], "zt": enc["zt"], "rho_hat_bits": enc["rho_hat_bits"]}
    if want == "decode":
        out["dec"] = O.decode(enc["packed"], enc["rho_hat_bits"], s, sig, b, seed, C, d)
    return out


def _oracle_decode(task):
    from oracle import qamw_ref as O

    packed, rn, s, sig, b, seed, C, d = task
    return O.decode(packed, rn, s, sig, b, seed, C, d)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, C, pool, workers, rows=640, rows_1t=64):
    """The oracle as it stands on a sample of the workload's rows: calibrate
    over the sample (one process), then encode and decode the sample split
    over `workers` processes; and the same on a smaller sample in one thread,
    for the per-core rate."""
    from threadpoolctl import threadpool_limits
    from oracle import qamw_ref as O

    def run(nrows, nproc):
        Wf = wl.W_f32()[:nrows]
        t0 = time.perf_counter()
        s, sig, _ = O.calibrate(Wf, wl.r, wl.alpha, wl.block, wl.sign_seed)
        if nproc > 1:
            chunks = np.array_split(np.arange(nrows), nproc)
            pool.map(_oracle_rows, [(Wf[c], s, sig, wl.block, wl.sign_seed, C, wl.d, "decode") for c in chunks])
        else:
            _oracle_rows((Wf, s, sig, wl.block, wl.sign_seed, C, wl.d, "decode"))
        return time.perf_counter() - t0

    dt = run(rows, workers)
    with threadpool_limits(limits=1):
        dt1 = run(rows_1t, 1)
    n, n1 = rows * wl.d, rows_1t * wl.d
    return {"value": n / dt / 1e9, "unit": "Gweights/s", "cores": workers, "kind": "oracle",
            "sample": f"rows 0..{rows - 1} of {wl.name} ({n} weights): calibrate over the sample (one process), "
                      f"encode and decode split over {workers} processes; fp64 NumPy, {dt:.2f} s",
            "cpu_model": cpu_model(),
            "one_thread": {"value": n1 / dt1 / 1e9, "rows": rows_1t, "seconds": dt1}}


def oracle_parity(wl, C, pool, workers, s, sigma, packed, rn, dec_rows, rows):
    """Sampled rows of the GPU's step checked against the oracle with the
    GPU's s and sigma: indices that differ (near ties within 1e-6 |z~|^2 of
    the oracle's distance, and mismatches beyond that), row-norm bits, and the
    fp32 decode's largest absolute error against the oracle's decode of the
    GPU's packed rows."""
    from oracle import qamw_ref as O

    Wf = wl.W_f32()[rows]
    K = C.shape[0]
    chunks = np.array_split(np.arange(len(rows)), workers)
    res = pool.map(_oracle_rows, [(Wf[c], s, sigma, wl.block, wl.sign_seed, C, wl.d, "encode") for c in chunks])
    dec = pool.map(_oracle_decode, [(packed[c], rn[c], s, sigma, wl.block, wl.sign_seed, C, wl.d) for c in chunks])
    idx_o = np.concatenate([r["idx"] for r in res])
    zt = np.concatenate([r["zt"] for r in res]).reshape(-1, 2)
    rn_o = np.concatenate([r["rho_hat_bits"] for r in res])
    idx_g = O.unpack(packed, K, wl.d)
    ok = O.accept_index(zt, C, idx_o.reshape(-1), idx_g.reshape(-1))
    differ = idx_o.reshape(-1) != idx_g.reshape(-1)
    err = float(np.max(np.abs(dec_rows.astype(np.float64) - np.concatenate(dec))))
    return {"rows": len(rows), "pairs": int(idx_g.size), "near_ties": int((differ & ok).sum()),
            "mismatches": int((~ok).sum()), "rownorm_bits_differ": int((rn_o != rn).sum()),
            "decode_max_abs_err": err,
            "note": "GPU words of sampled rows vs the oracle with the GPU's s and sigma; a differing index "
                    "is a near tie when its fp64 squared distance is within 1e-6 |z~|^2 of the oracle's, "
                    "otherwise a mismatch; decode error of the fp32 step output against the oracle's decode"}


def sweep_c4(q, dev, torch):
    """The 5120 x 13824 codebook-size sweep (K = 256, 1024, 2048, 4096 at
    alpha = 0 and 1/2; block 128): per variant the step (plan, calibrate +
    encode, fp32 decode) timed eagerly with HIP events, median of 3."""
    base = workloads.get("c4_5120x13824_K256_a0")
    W = torch.from_numpy(base.W.view(np.int16)).to(dev).view(torch.bfloat16)
    r = torch.from_numpy(base.r).to(dev)
    N, d, b = base.N, base.d, base.block
    out = torch.empty((N, d), dtype=torch.float32, device=dev)
    res = {}
    for K in (256, 1024, 2048, 4096):
        Ct = torch.from_numpy(q.load_codebook(K)).to(dev)
        rw = q.qamw_packed_row_words(d, K)
        packed = torch.empty((N, rw), dtype=torch.int32, device=dev)
        rn = torch.empty(N, dtype=torch.int16, device=dev)
        s = torch.empty(d, dtype=torch.float32, device=dev)
        sig = torch.empty(d // 2, dtype=torch.float32, device=dev)
        plan = torch.empty(q.qamw_plan_bytes(K), dtype=torch.uint8, device=dev)
        ws = torch.empty(q.qamw_calibrate_encode_workspace_bytes(N, d), dtype=torch.uint8, device=dev)
        for alpha in (0.0, 0.5):
            times = []
            for rep in range(4):
                ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
                ev[0].record()
                q.qamw_build_plan(Ct, plan)
                ev[1].record()
                q.qamw_calibrate_encode(W, r, alpha, b, 0, Ct, plan, s, sig, packed, rn, ws)
                ev[2].record()
                q.qamw_decode(packed, rn, d, s, sig, b, 0, Ct, out=out)
                ev[3].record()
                torch.cuda.synchronize()
                if rep:
                    times.append([ev[i].elapsed_time(ev[i + 1]) for i in range(3)])
            pl, ce, de = (float(np.median([t[i] for t in times])) for i in range(3))
            dec_bytes = N * d * 4 + N * rw * 4 + N * 2
            res[f"K{K}_a{alpha:g}"] = {
                "build_plan_ms": pl, "calibrate_encode_ms": ce, "decode_ms": de,
                "encode_gweights_s": N * d / ((pl + ce) * 1e-3) / 1e9,
                "decode_gweights_s": N * d / (de * 1e-3) / 1e9,
                "decode_frac_hbm": dec_bytes / (de * 1e-3) / 1e9 / PEAK_HBM_GBS,
                "step_gweights_s": N * d / ((pl + ce + de) * 1e-3) / 1e9}
        print(f"c4 sweep K={K}: {res[f'K{K}_a0']['step_gweights_s']:.1f} / {res[f'K{K}_a0.5']['step_gweights_s']:.1f} "
              "Gweights/s (alpha 0 / 0.5)", file=sys.stderr, flush=True)
    return {"workload": "5120x13824 bf16 N(0, 0.015^2), r ~ LogNormal(0, 1), block 128, fp32 decode; "
                        "per variant: build_plan + calibrate_encode + decode",
            "by_variant": res}


def stack_c5(q, dev, torch, layers):
    """The 7B-shaped linear stack end to end: `layers` x {q, k, v, o 4096 x
    4096; gate, up 11008 x 4096; down 4096 x 11008} bf16, Student-t(5) entries
    of std 0.02 and r ~ LogNormal(0, 1) per matrix, alpha 1/2, block 128,
    K = 2048 (one plan).  The matrices are generated on the GPU (torch's
    generator seeded per matrix; the same distribution as the host recipe, not
    the same numbers) before timing; then every matrix is calibrated and
    encoded, and then every one decoded to fp32, each phase timed as a whole
    with HIP events."""
    shapes = [("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
              ("gate", 11008, 4096), ("up", 11008, 4096), ("down", 4096, 11008)]
    K, b, alpha = 2048, 128, 0.5
    Ct = torch.from_numpy(q.load_codebook(K)).to(dev)
    plan = q.qamw_build_plan(Ct)
    mats = []
    for layer in range(layers):
        for p_i, (name, N, d) in enumerate(shapes):
            g = torch.Generator(device=dev)
            g.manual_seed(5000 + 8 * layer + p_i)
            z = torch.randn((N, d), generator=g, device=dev)
            chi2 = torch.zeros((N, d), device=dev)
            for _ in range(5):                  # chi-square with 5 degrees of freedom
                chi2.add_(torch.randn((N, d), generator=g, device=dev).square_())
            W = (z / torch.sqrt(chi2 / 5.0) * (0.02 / np.sqrt(5.0 / 3.0))).to(torch.bfloat16)
            del z, chi2
            r = torch.exp(torch.randn(d, generator=g, device=dev))
            rw = q.qamw_packed_row_words(d, K)
            mats.append(dict(W=W, r=r, N=N, d=d, packed=torch.empty((N, rw), dtype=torch.int32, device=dev),
                             rn=torch.empty(N, dtype=torch.int16, device=dev),
                             s=torch.empty(d, dtype=torch.float32, device=dev),
                             sig=torch.empty(d // 2, dtype=torch.float32, device=dev)))
    ws = torch.empty(max(q.qamw_calibrate_encode_workspace_bytes(m["N"], m["d"]) for m in mats),
                     dtype=torch.uint8, device=dev)
    out = torch.empty(max(m["N"] * m["d"] for m in mats), dtype=torch.float32, device=dev)

    def encode_all():
        for m in mats:
            q.qamw_calibrate_encode(m["W"], m["r"], alpha, b, 0, Ct, plan, m["s"], m["sig"], m["packed"], m["rn"], ws)

    def decode_all():
        for m in mats:
            q.qamw_decode(m["packed"], m["rn"], m["d"], m["s"], m["sig"], b, 0, Ct,
                          out=out[:m["N"] * m["d"]].view(m["N"], m["d"]))

    encode_all()
    decode_all()
    torch.cuda.synchronize()
    t = []
    for _ in range(3):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record()
        encode_all()
        ev[1].record()
        decode_all()
        ev[2].record()
        torch.cuda.synchronize()
        t.append((ev[0].elapsed_time(ev[1]), ev[1].elapsed_time(ev[2])))
    enc_ms = float(np.median([x[0] for x in t]))
    dec_ms = float(np.median([x[1] for x in t]))
    weights = sum(m["N"] * m["d"] for m in mats)
    res = {"matrices": len(mats), "weights": weights, "encode_ms": enc_ms, "decode_ms": dec_ms,
           "encode_gweights_s": weights / (enc_ms * 1e-3) / 1e9, "decode_gweights_s": weights / (dec_ms * 1e-3) / 1e9,
           "end_to_end_gweights_s": weights / ((enc_ms + dec_ms) * 1e-3) / 1e9,
           "note": "calibrate_encode of every matrix with one plan, then decode of every matrix to fp32; "
                   "host launch gaps between the calls included"}
    print(f"7B stack ({len(mats)} matrices): encode {enc_ms:.2f} ms, decode {dec_ms:.2f} ms", file=sys.stderr,
          flush=True)
    del mats
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the codec shards by rows or by matrix, but no multi-GPU path is built)", file=sys.stderr)
        sys.exit(2)

    # oracle worker processes are forked before anything touches the GPU
    pool, workers = None, 1
    if not args.no_cpu_baseline or args.parity_rows > 0:
        import multiprocessing as mp

        workers = max(1, min(16, len(os.sched_getaffinity(0))))
        pool = mp.get_context("fork").Pool(workers)

    import torch
    import vector_codebook_codec_amd as q

    dev = torch.device("cuda:0")
    wl = workloads.get(args.workload)
    C = q.load_codebook(wl.K)
    N, d, K, b = wl.N, wl.d, wl.K, wl.block
    if wl.wdtype == "bf16":
        W = torch.from_numpy(wl.W.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        W = torch.from_numpy(wl.W).to(dev)
    r = torch.from_numpy(wl.r).to(dev)
    Ct = torch.from_numpy(C).to(dev)
    s = torch.empty(d, dtype=torch.float32, device=dev)
    sigma = torch.empty(d // 2, dtype=torch.float32, device=dev)
    rw = q.qamw_packed_row_words(d, K)
    packed = torch.empty((N, rw), dtype=torch.int32, device=dev)
    rn = torch.empty(N, dtype=torch.int16, device=dev)
    out = torch.empty((N, d), dtype=torch.float32, device=dev)
    ws_cal = torch.empty(q.qamw_calibrate_workspace_bytes(N, d, b), dtype=torch.uint8, device=dev)
    ws_enc = torch.empty(max(256, q.qamw_encode_workspace_bytes(N, d)), dtype=torch.uint8, device=dev)
    plan = torch.empty(q.qamw_plan_bytes(K), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    ev = lambda: torch.cuda.Event(enable_timing=True)

    ws_ce = torch.empty(q.qamw_calibrate_encode_workspace_bytes(N, d), dtype=torch.uint8, device=dev)

    # The plan (a function of the codebook only) is built on a second stream
    # while the calibration pass runs; that stream then waits for the
    # calibration and runs the encode and the decode (of the capture orders
    # measured, this one lets a HIP graph of the step join the two branches
    # soonest), and the step's stream waits for it at the end.
    plan_stream = torch.cuda.Stream()

    def step(marks=None, st=None):
        cur = torch.cuda.current_stream() if st is None else st

        def mark(i, on=None):
            if marks is not None:
                marks[i].record(cur if on is None else on)
        mark(0)
        plan_stream.wait_stream(cur)
        with torch.cuda.stream(plan_stream):
            mark(4, plan_stream)
            q.qamw_build_plan(Ct, plan)
            mark(5, plan_stream)
        q.qamw_calibrate_prepare(W, r, wl.alpha, b, wl.sign_seed, s, sigma, rn, ws_ce, stream=cur)
        mark(1)
        plan_stream.wait_stream(cur)
        with torch.cuda.stream(plan_stream):
            q.qamw_encode_indices(W, b, Ct, ws_ce, plan=plan, packed=packed, stream=plan_stream)
            mark(2, plan_stream)
            q.qamw_decode(packed, rn, d, s, sigma, b, wl.sign_seed, Ct, out=out, stream=plan_stream)
            mark(3, plan_stream)
        cur.wait_stream(plan_stream)

    # The step is timed as replays of a HIP graph that holds one step's
    # launches (every kernel runs on every replay; only the host-side argument
    # checks and launch calls are done once, at capture).  The same step
    # launched eagerly is timed too, for the per-entry split and as
    # `eager_ms_per_step`.
    for i in range(max(1, args.warmup)):   # at least one eager step: the replays' reference
        step()
    torch.cuda.synchronize()
    ref_out = [t.clone() for t in (s, sigma, packed, rn, out)]
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(st=None)                   # warm the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step(st=None)                   # launches go to the capture stream
    torch.cuda.synchronize()
    for i in range(args.warmup):
        graph.replay()
        torch.cuda.synchronize()
        # deterministic: every replay reproduces the eager step bit for bit
        if not all(torch.equal(a, b_) for a, b_ in zip(ref_out, (s, sigma, packed, rn, out))):
            raise RuntimeError("graph replay of the step differs from the eager step")
        print(f"warmup step {i + 1}/{args.warmup} done", file=sys.stderr, flush=True)

    t0 = time.perf_counter()
    for i in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    print(f"timed {args.steps} steps (graph replays) in {wall:.4f} s", file=sys.stderr, flush=True)
    if not all(torch.equal(a, b_) for a, b_ in zip(ref_out, (s, sigma, packed, rn, out))):
        raise RuntimeError("graph replay of the step differs from the eager step")
    step_ms = wall * 1e3 / args.steps

    # the same replays with cold caches: a 1 GiB read before each one leaves
    # L2 and the Infinity Cache holding other, clean data
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    flush_sum = torch.empty((), dtype=torch.float32, device=dev)
    cold_steps = []
    for _ in range(args.cold_steps):
        torch.sum(flush, dim=0, out=flush_sum)
        torch.cuda.synchronize()
        a_ev, z_ev = ev(), ev()
        a_ev.record()
        graph.replay()
        z_ev.record()
        torch.cuda.synchronize()
        cold_steps.append(a_ev.elapsed_time(z_ev))
    cold_step_ms = float(np.median(cold_steps)) if cold_steps else None

    marks = [[ev() for _ in range(6)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(marks[i])
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    seg = lambda mk, i, j=None: float(np.mean([m[i].elapsed_time(m[i + 1 if j is None else j]) for m in mk]))
    cal_step_ms, idx_step_ms, dec_ms = (seg(marks, i) for i in range(3))
    plan_ms = seg(marks, 4, 5)                # on the second stream, overlapping the calibration
    enc_ms = seg(marks, 0, 2)                 # step start to the end of the encode

    # the same work as separate entry points, for per-kernel times: the roofline's
    # kernel (encode_lds_kernel, all of qamw_encode_indices) is timed here on its own
    packed_c = torch.empty_like(packed)
    rn_c = torch.empty_like(rn)
    s_c = torch.empty_like(s)
    sigma_c = torch.empty_like(sigma)
    cmarks = [[ev() for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        m = cmarks[i]
        m[0].record(stream)
        q.qamw_calibrate(W, r, wl.alpha, b, wl.sign_seed, s_c, sigma_c, ws_cal, stream)
        m[1].record(stream)
        q.qamw_encode_prepare(W, s_c, sigma_c, b, wl.sign_seed, rn_c, ws_enc, stream)
        m[2].record(stream)
        q.qamw_encode_indices(W, b, Ct, ws_enc, plan, packed_c, stream)
        m[3].record(stream)
    torch.cuda.synchronize()
    cal_ms, prep_ms, idx_ms_eager = (seg(cmarks, i) for i in range(3))
    if not (torch.equal(packed_c, packed) and torch.equal(rn_c, rn) and torch.equal(s_c, s)
            and torch.equal(sigma_c, sigma)):
        raise RuntimeError("qamw_calibrate_encode and the separate entry points disagree")

    # The roofline kernel's launch time: 10 back-to-back qamw_encode_indices
    # launches captured in a HIP graph, replayed between HIP events on the
    # replay stream (the per-launch event pairs above also count each
    # launch's start latency); mean per launch over the replays.
    roof_launches = 10
    roof_graph = torch.cuda.CUDAGraph()
    rs = torch.cuda.Stream()
    rs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(rs):
        q.qamw_encode_indices(W, b, Ct, ws_enc, plan, packed_c)
    torch.cuda.current_stream().wait_stream(rs)
    torch.cuda.synchronize()
    with torch.cuda.graph(roof_graph):
        for _ in range(roof_launches):
            q.qamw_encode_indices(W, b, Ct, ws_enc, plan, packed_c)
    roof_graph.replay()
    torch.cuda.synchronize()
    roof = []
    for _ in range(max(3, args.steps // 4)):
        a_ev, z_ev = ev(), ev()
        a_ev.record()
        roof_graph.replay()
        z_ev.record()
        torch.cuda.synchronize()
        roof.append(a_ev.elapsed_time(z_ev) / roof_launches)
    idx_ms = float(np.mean(roof))
    if not torch.equal(packed_c, packed):
        raise RuntimeError("graph replays of qamw_encode_indices differ from the step's encode")

    # the exhaustive search (no plan) for comparison; same indices, bit for bit
    packed_x = torch.empty_like(packed)
    exh = []
    for _ in range(args.exhaustive_reps):
        a, z = ev(), ev()
        a.record(stream)
        q.qamw_encode_indices(W, b, Ct, ws_enc, None, packed_x, stream)
        z.record(stream)
        torch.cuda.synchronize()
        exh.append(a.elapsed_time(z))
    if exh and not torch.equal(packed_x, packed):
        raise RuntimeError("planned and exhaustive encodes disagree")
    exh_ms = float(np.median(exh)) if exh else None

    # decode alone, with the caches (L2, MALL) holding other, clean data: a
    # 1 GiB read before each rep (a write would leave dirty lines whose
    # write-back the timed kernel would pay for)
    cold = []
    for _ in range(args.cold_decode_reps):
        torch.sum(flush, dim=0, out=flush_sum)
        torch.cuda.synchronize()
        a, z = ev(), ev()
        a.record(stream)
        q.qamw_decode(packed, rn, d, s, sigma, b, wl.sign_seed, Ct, out=out, stream=stream)
        z.record(stream)
        torch.cuda.synchronize()
        cold.append(a.elapsed_time(z))
    dec_cold_ms = float(np.median(cold)) if cold else None

    # a plain writer of the decode's output bytes under the same protocol
    # (torch's fill of the fp32 and of a 16-bit output): what a kernel that
    # only writes those bytes reaches on this device
    def cold_fill(t, reps):
        t.fill_(0.0)                    # pages touched once before timing
        ts = []
        for _ in range(reps):
            torch.sum(flush, dim=0, out=flush_sum)
            torch.cuda.synchronize()
            a, z = ev(), ev()
            a.record(stream)
            t.fill_(0.0)
            z.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(z))
        return float(np.median(ts)) if ts else None
    fill_buf = torch.empty_like(out)      # not `out`: it holds the step's decode
    fill32_ms = cold_fill(fill_buf, args.cold_decode_reps)

    # The same two without the launch latency of a single eager launch: a
    # HIP graph of 8 decodes (or fills), each over its own copy of the packed
    # matrix and its own output (1.7 GB in all, far more than the 256 MB
    # Infinity Cache, so every launch reads and writes HBM), replayed after
    # the 1 GiB read; per launch = graph time / 8.
    n_dc = 8
    dc_pk = [packed.clone() for _ in range(n_dc)] if args.cold_decode_reps else []

    def graph_cold(outs, reps, fill):
        gst = torch.cuda.Stream()
        gst.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(gst):
            def body():
                for i, o in enumerate(outs):
                    if fill:
                        o.fill_(1.0)
                    else:
                        q.qamw_decode(dc_pk[i], rn, d, s, sigma, b, wl.sign_seed, Ct, out=o, stream=gst)
            body()                      # pages touched once before capture
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=gst):
                body()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            torch.sum(flush, dim=0, out=flush_sum)
            torch.cuda.synchronize()
            a, z = ev(), ev()
            a.record()                  # a graph replays on the current stream
            gr.replay()
            z.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(z) / len(outs))
        return float(np.median(ts)) if ts else None

    dec_graph_cold_ms = fill32_graph_ms = None
    if args.cold_decode_reps:
        dc_out = [torch.empty_like(out) for _ in range(n_dc)]
        dec_graph_cold_ms = graph_cold(dc_out, args.cold_decode_reps, False)
        if not all(torch.equal(o, out) for o in dc_out):
            raise RuntimeError("graph-replayed decodes differ from the step's decode")
        fill32_graph_ms = graph_cold(dc_out, args.cold_decode_reps, True)
        del dc_out

    # decode to 16-bit outputs (the fused decode -> fp16 / bf16 of the
    # 11008 x 4096 configuration's transpose), warm and cold
    dec16 = {}
    for name, tdt in (("f16", torch.float16), ("bf16", torch.bfloat16)):
        out16 = torch.empty((N, d), dtype=tdt, device=dev)
        run16 = lambda: q.qamw_decode(packed, rn, d, s, sigma, b, wl.sign_seed, Ct, out=out16, stream=stream)
        run16()
        torch.cuda.synchronize()
        # against the fp32 decode rounded (RNE) to 16 bits: the kernel rounds the
        # last product straight to fp16 (one rounding), so at exact fp16 ties of
        # the fp32 value the two may differ by one unit in the last place
        # (-0 and +0 are the same value: an exact zero scaled by a negative
        # factor is -0 in fp32, and +0 where the scale is fused with the
        # conversion, which adds +0)
        ref16 = out.to(tdt)
        got_b, ref_b = out16.view(torch.int16).int(), ref16.view(torch.int16).int()
        n_signed_zero = int(((got_b != ref_b) & (out16 == 0) & (ref16 == 0)).sum())
        got_b = torch.where(got_b == -32768, torch.zeros_like(got_b), got_b)
        ref_b = torch.where(ref_b == -32768, torch.zeros_like(ref_b), ref_b)
        dbits = (got_b - ref_b).abs()
        if int(dbits.max()) > 1:
            bad = torch.nonzero(dbits > 1)[:4].tolist()
            raise RuntimeError(f"{name} decode differs from the rounded fp32 decode by more than one ulp at "
                               + ", ".join(f"{i}: {float(out[i[0], i[1]])!r} -> {float(out16[i[0], i[1]])!r}"
                                           for i in bad))
        n_ulp = int((dbits != 0).sum())
        warm16, cold16 = [], []
        for rep in range(2 * max(1, args.cold_decode_reps)):
            is_cold = rep % 2 == 1
            if is_cold:
                torch.sum(flush, dim=0, out=flush_sum)
            torch.cuda.synchronize()
            a, z = ev(), ev()
            a.record(stream)
            run16()
            z.record(stream)
            torch.cuda.synchronize()
            (cold16 if is_cold else warm16).append(a.elapsed_time(z))
        nb16 = N * d * 2 + N * rw * 4 + N * 2
        fill16_ms = cold_fill(fill_buf.view(-1).view(tdt)[:N * d], args.cold_decode_reps)
        g16 = f16g = None
        if args.cold_decode_reps:
            outs16 = [torch.empty((N, d), dtype=tdt, device=dev) for _ in range(n_dc)]
            g16 = graph_cold(outs16, args.cold_decode_reps, False)
            if not all(torch.equal(o, out16) for o in outs16):
                raise RuntimeError(f"graph-replayed {name} decodes differ")
            f16g = graph_cold(outs16, args.cold_decode_reps, True)
            del outs16
        dec16[name] = {"warm_ms": float(np.median(warm16)), "cold_ms": float(np.median(cold16)),
                       "algorithmic_bytes": nb16, "one_ulp_from_rounded_f32": n_ulp, "signed_zero_differences": n_signed_zero,
                       "frac_hbm_cold": nb16 / (np.median(cold16) * 1e-3) / 1e9 / PEAK_HBM_GBS,
                       "plain_fill_cold_ms": fill16_ms,
                       "plain_fill_frac_hbm_cold": None if fill16_ms is None else
                           N * d * 2 / (fill16_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                       "graph_cold_ms": g16,
                       "frac_hbm_graph_cold": None if g16 is None else nb16 / (g16 * 1e-3) / 1e9 / PEAK_HBM_GBS,
                       "plain_fill_graph_cold_ms": f16g,
                       "plain_fill_frac_hbm_graph_cold": None if f16g is None else
                           N * d * 2 / (f16g * 1e-3) / 1e9 / PEAK_HBM_GBS}
        del out16

    # fused decoded-weight matmul Y = X W^^T for T tokens (not part of the step).
    # Cold: the graph cycles through 12 copies of the packed matrix (372 MB, more
    # than the 256 MB Infinity Cache), so each call's weights come from HBM, as
    # in a model whose layers stream through.
    mm = {}
    n_copies = 12
    pk_copies = [packed.clone() for _ in range(n_copies)] if args.matmul_tokens else []
    for T in args.matmul_tokens:
        X = torch.randn((T, d), device=dev, dtype=torch.float32).to(torch.bfloat16)
        Xr = torch.empty((T, d), dtype=torch.bfloat16, device=dev)
        Y = torch.empty((T, N), dtype=torch.float32, device=dev)
        Wbf = torch.empty((N, d), dtype=torch.bfloat16, device=dev)

        def fused(st):
            q.qamw_rotate_activations(X, s, b, wl.sign_seed, Xr, st)
            q.qamw_decode_matmul(Xr, packed, rn, sigma, Ct, out=Y, stream=st)

        def unfused(st):
            q.qamw_decode(packed, rn, d, s, sigma, b, wl.sign_seed, Ct, out=Wbf, stream=st)
            torch.matmul(X, Wbf.t())

        # GPU time per call: 20 calls captured in a HIP graph and replayed, so
        # that host launch gaps (comparable to these kernels) are not counted
        inner = 20
        res_t = {}
        fused(stream)
        torch.cuda.synchronize()
        Y_eager = Y.clone()
        for name, fn in (("fused", fused), ("unfused", unfused)):
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                for _ in range(3):
                    fn(None)
            torch.cuda.current_stream().wait_stream(side)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(inner):
                    fn(None)
            times = []
            for _ in range(max(1, args.matmul_reps)):
                a, z = ev(), ev()
                a.record()
                g.replay()
                z.record()
                torch.cuda.synchronize()
                times.append(a.elapsed_time(z) / inner)
            res_t[name] = float(np.median(times))
            if name == "fused" and not torch.equal(Y, Y_eager):
                raise RuntimeError("graph replays of the fused matmul differ from the eager result")
        def cold_fused(st, pk):
            q.qamw_rotate_activations(X, s, b, wl.sign_seed, Xr, st)
            q.qamw_decode_matmul(Xr, pk, rn, sigma, Ct, out=Y, stream=st)

        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            cold_fused(None, pk_copies[0])
        torch.cuda.current_stream().wait_stream(side)
        gc = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gc):
            for pk in pk_copies:
                cold_fused(None, pk)
        gc.replay()
        torch.cuda.synchronize()
        tc = []
        for _ in range(max(1, args.matmul_reps)):
            a, z = ev(), ev()
            a.record()
            gc.replay()
            z.record()
            torch.cuda.synchronize()
            tc.append(a.elapsed_time(z) / n_copies)
        res_t["fused_cold"] = float(np.median(tc))
        if not torch.equal(Y, Y_eager):
            raise RuntimeError("the fused matmul over a copy of the packed matrix differs")
        # algorithmic bytes of the fused path: packed + row norms + sigma + X read + Xr write/read + Y write
        mm_bytes = N * rw * 4 + N * 2 + d * 2 + T * d * 2 * 3 + T * N * 4
        mm[str(T)] = {"fused_us": res_t["fused"] * 1e3, "unfused_us": res_t["unfused"] * 1e3,
                      "fused_cold_us": res_t["fused_cold"] * 1e3,
                      "frac_hbm_cold": mm_bytes / (res_t["fused_cold"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
                      "algorithmic_bytes": mm_bytes,
                      "GB_s": mm_bytes / (res_t["fused"] * 1e-3) / 1e9,
                      "frac_hbm": mm_bytes / (res_t["fused"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
                      "tflops": 2.0 * T * N * d / (res_t["fused"] * 1e-3) / 1e12}
        print(f"decode_matmul T={T}: fused {res_t['fused'] * 1e3:.1f} us (cold {res_t['fused_cold'] * 1e3:.1f}), "
              f"decode-to-bf16 + torch.matmul {res_t['unfused'] * 1e3:.1f} us",
              file=sys.stderr, flush=True)

    # polar-code baseline encode at 8 bits per pair (not part of the step)
    polar = None
    if args.polar_reps > 0:
        Ka, Kp = 8, 32
        lv, dr, _ = q.load_polar(Ka, Kp)
        lv_t, dr_t = torch.from_numpy(lv).to(dev), torch.from_numpy(dr).to(dev)
        rw_p = q.qamw_packed_row_words(d, Ka * Kp)
        packed_p = torch.empty((N, rw_p), dtype=torch.int32, device=dev)
        rn_p = torch.empty(N, dtype=torch.int16, device=dev)
        for _ in range(2):
            q.qamw_encode_polar(W, s, sigma, b, wl.sign_seed, lv_t, dr_t, packed_p, rn_p, ws_enc, stream)
        torch.cuda.synchronize()
        pt = []
        for _ in range(args.polar_reps):
            a, z = ev(), ev()
            a.record(stream)
            q.qamw_encode_polar(W, s, sigma, b, wl.sign_seed, lv_t, dr_t, packed_p, rn_p, ws_enc, stream)
            z.record(stream)
            torch.cuda.synchronize()
            pt.append(a.elapsed_time(z))
        p_ms = float(np.median(pt))
        in_b = 2 if wl.wdtype == "bf16" else 4
        p_bytes = 2 * N * d * in_b + N * rw_p * 4 + N * 2     # W read twice (prepare, quantise) + packed + norms
        polar = {"Ka": Ka, "Kp": Kp, "bits_per_index": q.qamw_index_bits(Ka * Kp), "ms": p_ms,
                 "gweights_s": N * d / (p_ms * 1e-3) / 1e9, "algorithmic_bytes": p_bytes,
                 "frac_hbm": p_bytes / (p_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                 "note": "qamw_encode_polar = encode_prepare_kernel + encode_polar_kernel"}
        print(f"polar encode {Ka}x{Kp}: {p_ms * 1e3:.1f} us", file=sys.stderr, flush=True)

    # codebook refinement on the matrix's own pairs (not part of the step)
    learned = None
    if args.learn_iters > 0:
        it = args.learn_iters
        ws_l = torch.empty(q.qamw_lloyd_workspace_bytes(K), dtype=torch.uint8, device=dev)
        C_l = torch.empty_like(Ct)
        dist_l = torch.empty(it, dtype=torch.float64, device=dev)
        packed_l = torch.empty_like(packed)
        plan_l = torch.empty_like(plan)
        q.qamw_calibrate_encode(W, r, wl.alpha, b, wl.sign_seed, Ct, plan, s, sigma, packed, rn, ws_ce, stream)
        q.qamw_learn_codebook(W, b, ws_ce, Ct, it, C_l, dist_l, plan_l, packed_l, ws_l, stream)
        torch.cuda.synchronize()
        a, z = ev(), ev()
        a.record(stream)
        q.qamw_learn_codebook(W, b, ws_ce, Ct, it, C_l, dist_l, plan_l, packed_l, ws_l, stream)
        z.record(stream)
        torch.cuda.synchronize()
        learn_ms = a.elapsed_time(z)
        Wf = W.float()
        q.qamw_decode(packed, rn, d, s, sigma, b, wl.sign_seed, Ct, out=out, stream=stream)
        e0 = float(torch.linalg.norm(out - Wf) / torch.linalg.norm(Wf))
        q.qamw_build_plan(C_l, plan_l, stream)
        q.qamw_encode(W, s, sigma, b, wl.sign_seed, C_l, plan=plan_l, packed=packed_l, stream=stream)
        q.qamw_decode(packed_l, rn, d, s, sigma, b, wl.sign_seed, C_l, out=out, stream=stream)
        e1 = float(torch.linalg.norm(out - Wf) / torch.linalg.norm(Wf))
        learned = {"rounds": it, "distortion_by_round": [float(v) for v in dist_l.cpu()],
                   "ms_per_round": learn_ms / it, "relative_error_gaussian_codebook": e0,
                   "relative_error_learned_codebook": e1}
        print(f"learned codebook: {learned}", file=sys.stderr, flush=True)

    # channel RMS from activations and the output error over alpha (not part of the step)
    sweep = None
    if args.sweep_tokens > 0:
        Tt = args.sweep_tokens
        Xs = torch.from_numpy(workloads.activations(Tt, wl.r, seed=2024)).to(dev).to(torch.bfloat16)
        ws_rms = torch.empty(max(256, q.qamw_channel_rms_workspace_bytes(Tt, d)), dtype=torch.uint8, device=dev)
        ws_oe = torch.empty(max(256, q.qamw_output_error_workspace_bytes(Tt, N, d)), dtype=torch.uint8, device=dev)
        r_x = torch.empty(d, dtype=torch.float32, device=dev)
        e_out = torch.empty(1, dtype=torch.float64, device=dev)
        s_a = torch.empty_like(s)
        sig_a = torch.empty_like(sigma)
        packed_a = torch.empty_like(packed)
        rn_a = torch.empty_like(rn)

        def timed(fn, reps=5):
            fn()
            torch.cuda.synchronize()
            ts = []
            for _ in range(reps):
                a, z = ev(), ev()
                a.record(stream)
                fn()
                z.record(stream)
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(z))
            return float(np.median(ts))

        rms_ms = timed(lambda: q.qamw_channel_rms(Xs, r_x, ws_rms, stream))
        errs = {}
        for alpha in (0.0, 0.25, 0.5, 0.75, 1.0):
            q.qamw_calibrate(W, r_x, alpha, b, wl.sign_seed, s_a, sig_a, ws_cal, stream)
            q.qamw_encode(W, s_a, sig_a, b, wl.sign_seed, Ct, packed=packed_a, rownorm_f16=rn_a,
                          workspace=ws_enc, stream=stream, plan=plan)
            q.qamw_decode(packed_a, rn_a, d, s_a, sig_a, b, wl.sign_seed, Ct, out=out, stream=stream)
            q.qamw_output_error(Xs, W, out, e_out, ws_oe, stream)
            errs[str(alpha)] = float(e_out.cpu()[0])
        oe_ms = timed(lambda: q.qamw_output_error(Xs, W, out, e_out, ws_oe, stream))
        oe_flops = 2.0 * Tt * N * d
        rms_bytes = Tt * d * 2 + d * 4
        sweep = {"tokens": Tt, "activations": "X[t][j] = r_j g, g ~ N(0, 1), bf16; r = the workload's channel RMS",
                 "output_error_by_alpha": errs, "best_alpha": min(errs, key=errs.get),
                 "channel_rms_us": rms_ms * 1e3,
                 "channel_rms_frac_hbm": rms_bytes / (rms_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                 "output_error_us": oe_ms * 1e3,
                 "output_error_tflops": oe_flops / (oe_ms * 1e-3) / 1e12,
                 "output_error_frac_bf16_mfma": oe_flops / (oe_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
        print(f"alpha sweep: {errs}; channel_rms {rms_ms * 1e3:.1f} us, output_error {oe_ms * 1e3:.1f} us",
              file=sys.stderr, flush=True)

    for _ in range(args.copy_reference):
        flush2 = torch.empty_like(flush)
        flush2.copy_(flush)
        torch.cuda.synchronize()

    B = q.qamw_index_bits(K)
    P = N * d // 2
    in_bytes = 2 if wl.wdtype == "bf16" else 4
    enc_bytes = N * d * in_bytes + N * rw * 4             # W read + packed write (qamw_encode_indices)
    enc_gbs = enc_bytes / (idx_ms * 1e-3) / 1e9
    exh_flops = P * K * 4.0                               # exhaustive search: K evaluations x 4 flops per pair
    dec_bytes = N * d * 4 + N * rw * 4 + N * 2            # fp32 out + packed + row norms
    weights = N * d
    res = {
        "metric": "QAM-W encode & decode Gweights/s at 4096x11008; % VALU peak / % HBM BW",
        "value": weights / (step_ms * 1e-3) / 1e9,
        "unit": "Gweights/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "eager_ms_per_step": eager_ms,
        "cold_step": None if cold_step_ms is None else {
            "ms": cold_step_ms, "gweights_s": weights / (cold_step_ms * 1e-3) / 1e9,
            "note": "the step's graph replayed after a 1 GiB read each time (L2 and Infinity Cache cold)"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: {N}x{d} {wl.wdtype} {workload_entries(wl.name)}, "
                               f"alpha={wl.alpha}, block={b}, K={K}, fp32 decode",
                   "N": N, "d": d, "K": K, "block": b, "bits_per_index": B, "in_dtype": wl.wdtype,
                   "out_dtype": "f32"},
        "roofline": {"bound": "hbm",
                     "kernel": ("encode_lds_kernel" if K <= 2048 else "encode_plan_kernel")
                               + " (qamw_encode_indices with a search plan)",
                     "achieved": enc_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": enc_gbs / PEAK_HBM_GBS,
                     "traffic": measured_traffic(wl.name),
                     "algorithmic": f"W read {N * d * in_bytes} B + packed write {N * rw * 4} B "
                                    f"= {enc_bytes} B per launch ({in_bytes} + {B}/16 B per weight)"},
        "valu_view": {
            "exhaustive_equivalent_flops": exh_flops,
            "exhaustive_encode_indices_ms": exh_ms,
            "exhaustive_frac_of_fp32_peak": None if exh_ms is None else
                exh_flops / (exh_ms * 1e-3) / 1e12 / PEAK_FP32_TFLOPS,
            "planned_speedup_vs_exhaustive_at_fp32_peak": exh_flops / (idx_ms * 1e-3) / 1e12 / PEAK_FP32_TFLOPS,
            "step_encode_speedup_vs_exhaustive_at_fp32_peak":
                exh_flops / (enc_ms * 1e-3) / 1e12 / PEAK_FP32_TFLOPS,
            "note": "the exhaustive search (no plan) against the fp32 vector peak, counting pairs x K x 4 "
                    "flops; the planned search gives the same indices scoring a few candidates per pair, so "
                    "its rate in those units is a speedup over an exhaustive search at the fp32 peak, not a "
                    "utilisation (its own bound is HBM, see roofline)"},
        "per_entry_ms": {"build_plan": plan_ms, "calibrate_prepare": cal_step_ms, "encode_indices": idx_step_ms,
                         "decode": dec_ms, "encode_total": enc_ms,
                         "note": "eager launches; build_plan runs on a second stream beside calibrate_prepare, "
                                 "and that stream then runs encode_indices and decode; encode_total is the step's "
                                 "start to the end of its encode"},
        "separate_entry_ms": {"calibrate": cal_ms, "encode_prepare": prep_ms, "encode_indices": idx_ms_eager,
                              "encode_indices_graph": idx_ms,
                              "note": "the step's calibrate_encode as separate calls (same results, bit for "
                                      "bit); encode_prepare repeats the row-norm pass"},
        "encode_gweights_s": weights / (enc_ms * 1e-3) / 1e9,
        "decode_gweights_s": weights / (dec_ms * 1e-3) / 1e9,
        "decode_16bit": dec16,
        "decode_cold": None if dec_cold_ms is None else {
            "ms": dec_cold_ms, "algorithmic_bytes": dec_bytes,
            "GB_s": dec_bytes / (dec_cold_ms * 1e-3) / 1e9,
            "frac_hbm": dec_bytes / (dec_cold_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "plain_fill_cold_ms": fill32_ms,
            "plain_fill_frac_hbm_cold": None if fill32_ms is None else
                N * d * 4 / (fill32_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "graph_cold_ms": dec_graph_cold_ms,
            "frac_hbm_graph_cold": None if dec_graph_cold_ms is None else
                dec_bytes / (dec_graph_cold_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "plain_fill_graph_cold_ms": fill32_graph_ms,
            "plain_fill_frac_hbm_graph_cold": None if fill32_graph_ms is None else
                N * d * 4 / (fill32_graph_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "note": "1 GiB read before each rep; ms: one eager launch (its launch latency included); "
                    "graph_cold_ms: per launch of a HIP graph of 8 decodes, each over its own copy of the "
                    "packed matrix and its own output (1.7 GB, all from and to HBM); plain_fill: torch's fill "
                    "of the same outputs under the same two protocols"},
        "achieved_bpw": B / 2 + 16.0 / d,
        "decode_matmul": {"note": "Y = X W^^T over the packed matrix (qamw_rotate_activations + "
                                  "qamw_decode_matmul) vs qamw_decode to bf16 + torch.matmul; per T",
                          "by_tokens": mm},
        "polar": polar,
        "alpha_sweep": sweep,
        "learned_codebook": learned,
    }
    if args.sweep_c4:
        res["c4_sweep"] = sweep_c4(q, dev, torch)
    if args.stack_layers > 0:
        res["c5_stack"] = stack_c5(q, dev, torch, args.stack_layers)
    if args.parity_rows > 0:
        print(f"checking {args.parity_rows} sampled rows against the oracle", file=sys.stderr, flush=True)
        prow = np.unique(np.linspace(0, N - 1, args.parity_rows).astype(np.int64))
        res["parity"] = oracle_parity(wl, C, pool, workers, ref_out[0].cpu().numpy(), ref_out[1].cpu().numpy(),
                                      ref_out[2].cpu().numpy().view(np.uint32)[prow],
                                      ref_out[3].cpu().numpy().view(np.uint16)[prow],
                                      ref_out[4].cpu().numpy()[prow], prow)
        print(f"parity: {res['parity']}", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        print("timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(wl, C, pool, workers)
    if pool is not None:
        pool.close()
        pool.join()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
