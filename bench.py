#!/usr/bin/env python3
"""Benchmark of the KDA hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  * chunked prefill (metadata, intra-chunk and state/output kernels) of the
    Kimi-Linear-shaped workload: 16 sequences with lengths U{512..4096}
    (seed 4: T = 38,632 tokens), Hk = Hv = 32, K = V = 128, bf16 q/k/v,
    realistic per-channel gates, fp32 state pool of 32 slots updated in place;
  * one-token recurrent decode of 4096 requests, Hk = Hv = 32, K = V = 128,
    bf16 q/k/v, fp32 state pool of 4160 slots updated in place.
Inputs are generated on the host (seeded), copied to HBM before timing, and
stay resident.  After the timed steps the same workloads are passed through
the fused-gate entry points (raw bf16 gate and beta inputs, activation inside
the kernels) and reported under "fused_gate", and a multi-token verify decode
(1024 requests x 4 tokens with a per-step state cache) is timed and reported
under "spec_decode".  Prints one JSON line.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--no-cpu-baseline]

Other workloads, each timed on its own: --part prefill with --prefill-workload
long (one 32,768-token sequence) or --prefill-lengths L1,L2,..; --part decode
with --decode-batch B and --spec-batch B (small batches).

The traffic records under profiles/ (HBM bytes counted by rocprofv3) are
written by ``--traffic-record``, from counter runs of this script.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFLOPS = 2516.6    # MI355X dense fp16/bf16 MFMA, TFLOP/s

METRIC = "KDA prefill tokens/s + MFMA util; decode states/s + HBM GB/s vs peak"
DECODE_KERNEL = "kda::decode_kernel<128, 128, kda::bf16, float, false, false, true>"
DECODE_SRC = os.path.join(ROOT, "gated_delta_rule_51_amd", "csrc", "kda_decode.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_b4096_traffic.json")
PREFILL_SRC = os.path.join(ROOT, "gated_delta_rule_51_amd", "csrc", "kda_prefill.hip")
PREFILL_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_16seq_traffic.json")


def _sha(path):
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(path=TRAFFIC_FILE, src=DECODE_SRC):
    """The rocprofv3 FETCH_SIZE / WRITE_SIZE record under profiles/ (HBM bytes
    per launch, scaled by a plain copy of known size), or None when the
    kernel source changed since the counters were taken."""
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != _sha(src):
        return None
    return rec


def prefill_work(cu, hk, hv, dk, dv, chunk=64, gate_bytes=4):
    """Algorithmic flops and bytes of one prefill call.

    flops per (token, value head): 6 K V (W S0, K~^T U, (Q G) S0) + C (3K + 2V)
    (A, W, M and Ut, M U; triangles counted half).  Bytes: q, k (shared by the
    Hv/Hk value heads of a key head), v, g (per channel), beta, o per
    token-head, plus h0 read and ht written per (sequence, head) in fp32.
    ``gate_bytes`` is the size of one g / beta element: 4 for fp32 g and beta,
    2 for the raw bf16 inputs of the fused-gate entry point (which also reads
    A_log and dt_bias, 8 bytes per (head, channel), once)."""
    T = int(cu[-1])
    N = len(cu) - 1
    flops = T * hv * (6 * dk * dv + chunk * (3 * dk + 2 * dv))
    per_tok = 2 * dk * 2 * hk / hv + 2 * dv + gate_bytes * (dk + 1) + 2 * dv
    nbytes = T * hv * per_tok + N * hv * 2 * 4 * dk * dv + (8 * hv * dk if gate_bytes != 4 else 0)
    return flops, nbytes


def decode_work(B, hk, hv, dk, dv, gate_bytes=4):
    """Bytes per (request, head): fp32 state read + write, q, k, v, g, beta, o
    (g and beta elements of ``gate_bytes`` each, as for prefill_work)."""
    per = 2 * 4 * dk * dv + (2 * dk * 2 * hk / hv + 2 * dv + gate_bytes * (dk + 1) + 2 * dv)
    return B * hv * per + (8 * hv * dk if gate_bytes != 4 else 0)


def multi_decode_work(lengths, hk, hv, dk, dv, pitch, update_pool, gate_bytes=2):
    """Bytes of one multi-token decode call: per (request, head) the fp32 state
    read once, one fp32 state written per cached step (min(L, pitch) of them),
    the pool row written back if update_pool; per (token, head) q, k, v, g,
    beta, o as for decode_work; A_log and dt_bias once."""
    state = 4 * dk * dv
    tokens = sum(lengths)
    per_tok = 2 * dk * 2 * hk / hv + 2 * dv + gate_bytes * (dk + 1) + 2 * dv
    steps = sum(min(L, pitch) for L in lengths)
    busy = sum(1 for L in lengths if L > 0)
    return hv * (busy * state * (2 if update_pool else 1) + steps * state + tokens * per_tok) + 8 * hv * dk


def cpu_baseline(pre, dec, reps=5, nreq=1024):
    """The fp64 oracle on the host cores, on a bounded sample of the same
    workload: the full prefill batch (all 16 sequences, all heads; median of
    ``reps`` runs) and the first ``nreq`` of the 4096 decode requests (median of
    3 runs).  The inputs are converted to the oracle's array types before
    the clock starts, so each time covers the oracle's computation only."""
    from oracle import oracle as O
    O.build(force=False)
    threads = O.max_threads()
    f32 = lambda x: x.float().contiguous().numpy()
    f64 = lambda x: x.double().contiguous().numpy()
    slots = O.map_slot(pre.indices.numpy(), pre.pool.shape[0])
    h0 = pre.pool[slots]
    P = (f32(pre.q), f32(pre.k), f32(pre.v), f64(pre.g), f64(pre.beta), pre.cu_seqlens.numpy())
    h0n = f32(h0)
    tps = []
    for _ in range(reps):
        t = time.perf_counter()
        O.prefill(*P, h0=h0n)
        tps.append(time.perf_counter() - t)
    tp = statistics.median(tps)
    T = int(pre.cu_seqlens[-1])
    nreq = min(nreq, dec.q.shape[0])
    dslots = O.map_slot(dec.indices.numpy()[:nreq], dec.pool.shape[0])
    D = (f32(dec.q[:nreq]), f32(dec.k[:nreq]), f32(dec.v[:nreq]), f64(dec.g[:nreq]), f64(dec.beta[:nreq]))
    pool = f32(dec.pool[dslots])
    tds = []
    for _ in range(3):
        t = time.perf_counter()
        O.decode(*D, pool)
        tds.append(time.perf_counter() - t)
    td = statistics.median(tds)
    hv = dec.v.shape[1]
    # one thread, on the first `h1` heads of every sequence (heads are
    # independent units of equal cost), scaled to all heads
    h1 = 4
    sel = lambda x: x[:, :h1]
    P1 = (f32(sel(pre.q)), f32(sel(pre.k)), f32(sel(pre.v)), f64(sel(pre.g)), f64(sel(pre.beta)),
          pre.cu_seqlens.numpy())
    h01 = f32(sel(h0))
    t = time.perf_counter()
    O.prefill(*P1, h0=h01, nthreads=1)
    t1 = (time.perf_counter() - t) * hv / h1
    return {
        "value": T / tp, "unit": "tokens/s", "cores": threads, "kind": "oracle",
        "sample": "fp64 C oracle (OpenMP over sequence-head units): full prefill batch "
                  "(%d tokens x 32 heads), median of %d runs = %.2f s; decode: first %d of %d "
                  "requests, median of 3 runs = %.3f s; one thread: the first %d heads of the "
                  "prefill batch, scaled to 32 heads; inputs converted before timing"
                  % (T, reps, tp, nreq, dec.q.shape[0], td, h1),
        "decode_states_per_s": nreq * hv / td,
        "one_thread_value": T / t1,
        "cpu_model": cpu_model(),
        "host_cpus": os.cpu_count(),
        "affinity_cpus": len(os.sched_getaffinity(0)),
    }


# Kernels whose counters the traffic records hold (names as rocprofv3 prints them).
FUSED_DECODE_KERNEL = "kda::decode_kernel<128, 128, kda::bf16, float, false, true, true>"
MULTI_DECODE_KERNEL = "kda::multi_decode_kernel<128, 128, kda::bf16, float, false, true>"
# (The prefill kernels sit in an unnamed namespace inside kda::.)
PREFILL_KERNELS = (("intra", "intra_kernel<128, 128, kda::bf16, false, false>"),
                   ("intra_fused_gate", "intra_kernel<128, 128, kda::bf16, false, true>"),
                   ("state", "state_kernel<128, 128, 64, 2, kda::bf16, float>"),
                   ("meta", "meta_kernel"))


def _pmc_values(d, counter):
    """{kernel name: [value per dispatch]} of one counter from the
    counter_collection.csv files of a rocprofv3 --pmc output directory."""
    import csv
    import glob
    out = {}
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    if not out:
        raise SystemExit("no %s values under %s" % (counter, d))
    return out


def _mean_of(vals, name):
    """Mean over the dispatches of the one kernel whose name contains name."""
    hits = [v for k, v in vals.items() if name in k]
    if len(hits) != 1:
        raise SystemExit("%d kernels named %s" % (len(hits), name))
    return sum(hits[0]) / len(hits[0]), len(hits[0])


def traffic_record(part, fetch_dir, write_dir, path=None):
    """Write profiles/<part> traffic JSON from two rocprofv3 --pmc runs of
    this script (FETCH_SIZE, then WRITE_SIZE, in KiB per dispatch) made with
    --copy-calibration-gib 4: both counters are scaled by what they read for
    that plain 4 GiB copy, and the record carries the hash of the kernel
    source, so that the bench reports it only while the source is unchanged."""
    F, Wr = _pmc_values(fetch_dir, "FETCH_SIZE"), _pmc_values(write_dir, "WRITE_SIZE")
    cf = max(v for k, vs in F.items() if "copyBuffer" in k for v in vs)
    cw = max(v for k, vs in Wr.items() if "copyBuffer" in k for v in vs)
    ref_kib = 4 * 1024 * 1024
    fs, ws = ref_kib / cf, ref_kib / cw
    rec_cmd = ("python3 bench.py --traffic-record %s --fetch-dir <out FETCH_SIZE> --write-dir <out WRITE_SIZE>"
               % part)
    cmds = ["cd /tmp && rocprofv3 --pmc %s --output-format csv -d <out %s> -o run -- python3 <repo>/bench.py "
            "--part %s --steps 1 --warmup 0 --no-cpu-baseline --copy-calibration-gib 4 --fused-gate-steps 2 "
            "--spec-steps 2" % (c, c, part) for c in ("FETCH_SIZE", "WRITE_SIZE")] + [rec_cmd]
    common = {"copy_reference": "one 4 GiB device-to-device copy (rocclr copyBuffer) in the same process",
              "copy_fetch_size_kib": cf, "copy_write_size_kib": cw, "fetch_scale": fs, "write_scale": ws}
    both = lambda f, w: (f * fs + w * ws) * 1024
    if part == "decode":
        f, _ = _mean_of(F, DECODE_KERNEL)
        w, _ = _mean_of(Wr, DECODE_KERNEL)
        ff, _ = _mean_of(F, FUSED_DECODE_KERNEL)
        fw, _ = _mean_of(Wr, FUSED_DECODE_KERNEL)
        mf, _ = _mean_of(F, MULTI_DECODE_KERNEL)
        mw, _ = _mean_of(Wr, MULTI_DECODE_KERNEL)
        rec = {"kernel": DECODE_KERNEL,
               "workload": "decode B=4096, Hk=Hv=32, K=V=128, bf16 q/k/v, fp32 pool 4160 slots",
               "fetch_size_kib": f, "write_size_kib": w, **common,
               "traffic_bytes_per_launch": both(f, w),
               "algorithmic_bytes_per_launch": decode_work(4096, 32, 32, 128, 128),
               "fused_gate_kernel": FUSED_DECODE_KERNEL,
               "fused_gate_fetch_size_kib_mean": ff, "fused_gate_write_size_kib_mean": fw,
               "fused_gate_traffic_bytes_per_launch": both(ff, fw),
               "fused_gate_algorithmic_bytes_per_launch": decode_work(4096, 32, 32, 128, 128, gate_bytes=2),
               "multi_decode_kernel": MULTI_DECODE_KERNEL,
               "multi_decode_workload": "verify: 1024 requests x 4 tokens, Hv=32, K=V=128, fused gate, fp32 pool "
                                        "read-only, fp32 cache pitch 8",
               "multi_decode_fetch_size_kib_mean": mf, "multi_decode_write_size_kib_mean": mw,
               "multi_decode_traffic_bytes_per_launch": both(mf, mw),
               "multi_decode_algorithmic_bytes_per_launch": multi_decode_work([4] * 1024, 32, 32, 128, 128, 8,
                                                                              False),
               "kernel_source_sha256_16": _sha(DECODE_SRC), "commands": cmds}
        path = path or TRAFFIC_FILE
    else:
        import kda_workloads as W
        cu = W.kimi_prefill_16seq().cu_seqlens.tolist()
        kern = {}
        for nm, key in PREFILL_KERNELS:
            f, calls = _mean_of(F, key)
            w, _ = _mean_of(Wr, key)
            kern[nm] = {"kernel": "kda::" + key, "calls": calls, "fetch_size_kib_mean": f, "write_size_kib_mean": w,
                        "read_bytes": f * fs * 1024, "written_bytes": w * ws * 1024}
        tot = lambda names: sum(kern[n]["read_bytes"] + kern[n]["written_bytes"] for n in names)
        rec = {"workload": "prefill: 16 sequences, lengths U{512..4096} (T=%d), Hk=Hv=32, K=V=128, bf16 q/k/v, "
                           "fp32 g and beta, fp32 pool of 32 slots" % cu[-1],
               **common, "kernels": kern,
               "traffic_bytes_per_call": tot(["meta", "intra", "state"]),
               "algorithmic_bytes_per_call": prefill_work(cu, 32, 32, 128, 128)[1],
               "fused_gate_traffic_bytes_per_call": tot(["meta", "intra_fused_gate", "state"]),
               "fused_gate_algorithmic_bytes_per_call": prefill_work(cu, 32, 32, 128, 128, gate_bytes=2)[1],
               "kernel_source_sha256_16": _sha(PREFILL_SRC), "commands": cmds}
        path = path or PREFILL_TRAFFIC_FILE
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print("wrote %s" % path)
    return rec


def cpu_model():
    """The host CPU's model name, from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def workload_name(part, long_prompt, T, B=4096, lengths=None):
    if lengths:
        return ("KDA chunked prefill: %d sequences of lengths %s (T=%d), Hk=Hv=32, K=V=128, bf16 q/k/v, "
                "realistic per-channel gates, fp32 pool %d slots" % (len(lengths), lengths, T, len(lengths) + 1))
    pre = ("KDA chunked prefill: 1 sequence of %d tokens, Hk=Hv=32, K=V=128, bf16 q/k/v, realistic "
           "per-channel gates, fp32 pool 2 slots" % T if long_prompt else
           "KDA chunked prefill: 16 seqs, lengths U{512..4096} (T=%d), Hk=Hv=32, K=V=128, bf16 q/k/v, "
           "realistic per-channel gates, fp32 pool 32 slots" % T)
    dec = "recurrent decode: B=%d, Hk=Hv=32, K=V=128, fp32 pool %d slots" % (B, B + 64)
    return {"both": pre + "; + " + dec, "prefill": pre, "decode": dec}[part]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--spec-steps", type=int, default=10,
                    help="after the timed steps, time this many multi-token verify decodes "
                         "(--spec-batch requests x 4 tokens, cache pitch 8; 0: skip)")
    ap.add_argument("--fused-gate-steps", type=int, default=10,
                    help="after the timed steps, time this many passes through the fused-gate "
                         "entry points (0: skip)")
    ap.add_argument("--decode-batch", type=int, default=4096,
                    help="requests of the one-token decode (pool of batch + 64 slots)")
    ap.add_argument("--spec-batch", type=int, default=1024,
                    help="requests of the verify decode (4 tokens each; pool of batch + 64 slots)")
    ap.add_argument("--part", choices=["both", "prefill", "decode"], default="both",
                    help="time one part only (for profiling runs)")
    ap.add_argument("--prefill-lengths", default=None,
                    help="comma-separated sequence lengths for a prefill of their own (32 heads, "
                         "K=V=128, bf16, realistic gates, fp32 pool), with --part prefill")
    ap.add_argument("--prefill-workload", choices=["16seq", "long"], default="16seq",
                    help="16seq: 16 sequences of 512-4096 tokens (the step's prefill); long: one "
                         "sequence of 32,768 tokens, 32 heads (a measurement of its own)")
    ap.add_argument("--copy-calibration-gib", type=float, default=0.0,
                    help="run one plain device copy of this size first (a known-size "
                         "reference for FETCH_SIZE / WRITE_SIZE counter runs)")
    ap.add_argument("--traffic-record", choices=["prefill", "decode"],
                    help="no timing: write that part's traffic record under profiles/ from two "
                         "rocprofv3 --pmc runs (--fetch-dir, --write-dir) and exit")
    ap.add_argument("--fetch-dir", help="rocprofv3 -d directory of the FETCH_SIZE run")
    ap.add_argument("--write-dir", help="rocprofv3 -d directory of the WRITE_SIZE run")
    args = ap.parse_args()
    long_prompt = args.prefill_workload == "long"
    if (long_prompt or args.prefill_lengths) and args.part != "prefill":
        ap.error("--prefill-workload long and --prefill-lengths are timed on their own: add --part prefill")
    lengths = [int(x) for x in args.prefill_lengths.split(",")] if args.prefill_lengths else None
    if args.traffic_record:
        if not (args.fetch_dir and args.write_dir):
            ap.error("--traffic-record needs --fetch-dir and --write-dir")
        traffic_record(args.traffic_record, args.fetch_dir, args.write_dir)
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: (sequence, head) and (request, head) units are "
              "independent, so more GPUs would each run this same path on their own heads or "
              "sequences with no cross-GPU step to time; use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import kda_workloads as W
    import gated_delta_rule_51_amd as kda

    kda.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    do_pre = args.part in ("both", "prefill")
    do_dec = args.part in ("both", "decode")
    if not do_pre:
        pre = None
    elif lengths:
        pre = W.make_prefill(12, lengths, 32, 32, 128, 128, gate="realistic", pool_slots=len(lengths) + 1)
    else:
        pre = W.long_prompt_32k() if long_prompt else W.kimi_prefill_16seq()
    dec = W.decode_b4096(batch=args.decode_batch, num_slots=args.decode_batch + 64) if do_dec else None
    names = ("q", "k", "v", "g", "beta", "gx", "A_log", "dt_bias", "bx", "pool", "indices")
    P = {n: getattr(pre, n).to(dev) for n in names + ("cu_seqlens",)} if do_pre else {}
    D = {n: getattr(dec, n).to(dev) for n in names} if do_dec else {}
    torch.cuda.synchronize()

    if args.copy_calibration_gib > 0:
        nel = int(args.copy_calibration_gib * (1 << 30)) // 4
        src = torch.ones(nel, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step(evs=None):
        if evs is not None:
            evs[0].record()
        if do_pre:
            kda.chunk_prefill(P["q"], P["k"], P["v"], P["g"], P["beta"], P["cu_seqlens"],
                              initial_state=P["pool"], state_indices=P["indices"])
        if evs is not None:
            evs[1].record()
        if do_dec:
            kda.recurrent_decode(D["q"], D["k"], D["v"], D["g"], D["beta"], D["pool"], D["indices"])
        if evs is not None:
            evs[2].record()

    def fused_step(evs):
        """The same pass through the fused-gate entry points (raw bf16 gate and
        beta inputs activated inside the kernels)."""
        evs[0].record()
        if do_pre:
            kda.chunk_prefill_fused_gate(P["q"], P["k"], P["v"], P["gx"], P["A_log"], P["dt_bias"], P["bx"],
                                         P["cu_seqlens"], initial_state=P["pool"], state_indices=P["indices"])
        evs[1].record()
        if do_dec:
            kda.recurrent_decode_fused_gate(D["q"], D["k"], D["v"], D["gx"], D["A_log"], D["dt_bias"],
                                            D["bx"], D["pool"], D["indices"])
        evs[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre_t = [e[0].elapsed_time(e[1]) for e in evs]
    dec_t = [e[1].elapsed_time(e[2]) for e in evs]
    pre_ms, dec_ms = sum(pre_t) / args.steps, sum(dec_t) / args.steps

    # fused-gate variant, timed after the step loop (not part of the step)
    fsteps = args.fused_gate_steps
    fused_pre_ms = fused_dec_ms = None
    if fsteps > 0:
        fev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(fsteps + 1)]
        for e in fev:   # the first pass is a warm-up
            fused_step(e)
        torch.cuda.synchronize()
        fused_pre_ms = sum(e[0].elapsed_time(e[1]) for e in fev[1:]) / fsteps
        fused_dec_ms = sum(e[1].elapsed_time(e[2]) for e in fev[1:]) / fsteps
    finite = all(bool(torch.isfinite(X["pool"]).all().item()) for X in (P, D) if X)

    # multi-token verify decode (speculative decoding), timed on its own
    spec = None
    if args.spec_steps > 0 and do_dec:
        m = W.spec_decode_b1024(batch=args.spec_batch, num_slots=args.spec_batch + 64)
        t = m.tok
        S = {n: getattr(t, n).to(dev) for n in ("q", "k", "v", "gx", "A_log", "dt_bias", "bx", "cu_seqlens")}
        spool, sidx = m.pool.to(dev), m.indices.to(dev)
        hv_, dv_, dk_ = t.v.shape[1], t.v.shape[2], t.q.shape[2]
        cache = torch.empty(t.num_seqs, m.cache_pitch, hv_, dv_, dk_, dtype=spool.dtype, device=dev)

        def verify():
            kda.recurrent_decode_multi_fused_gate(S["q"], S["k"], S["v"], S["gx"], S["A_log"], S["dt_bias"],
                                                  S["bx"], S["cu_seqlens"], spool, sidx,
                                                  intermediate_states=cache, update_pool=False)
        # Warm-up: the first calls into the freshly allocated 16 GiB step cache
        # run up to ~15% slower (measured per launch under the tracer: 2.16,
        # 2.09, 2.19, 2.07, 2.00, 1.98, 1.92, then 1.87-1.90 ms); a serving loop
        # reuses one cache allocation.
        for _ in range(5):
            verify()
        torch.cuda.synchronize()
        sev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.spec_steps)]
        for e in sev:
            e[0].record()
            verify()
            e[1].record()
        torch.cuda.synchronize()
        spec_ms = sum(e[0].elapsed_time(e[1]) for e in sev) / args.spec_steps
        lens = (t.cu_seqlens[1:] - t.cu_seqlens[:-1]).tolist()
        sb = multi_decode_work(lens, t.q.shape[1], hv_, dk_, dv_, m.cache_pitch, False)
        spec = {"workload": "multi-token verify decode: %d requests x 4 tokens, Hk=Hv=32, K=V=128, bf16 io, "
                            "fused gate, fp32 pool %d slots read-only, fp32 step cache pitch 8"
                            % (args.spec_batch, args.spec_batch + 64),
                "steps": args.spec_steps, "ms": spec_ms,
                "tokens_per_s": sum(lens) / (spec_ms * 1e-3),
                "alg_bytes_per_launch": sb, "alg_gbs": sb / (spec_ms * 1e-3) / 1e9,
                "hbm_frac_alg": sb / (spec_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        del cache, spool

    hk, hv, dk, dv = 32, 32, 128, 128
    cu = pre.cu_seqlens.tolist() if do_pre else [0]
    T = cu[-1]
    pf, pb = prefill_work(cu, hk, hv, dk, dv)
    B = dec.q.shape[0] if do_dec else 0
    db = decode_work(B, hk, hv, dk, dv)

    prefill = {"ms": pre_ms, "ms_median": statistics.median(pre_t),
               "tokens_per_s": T / (pre_ms * 1e-3) if do_pre else None,
               "tokens": T, "alg_tflops": pf / (pre_ms * 1e-3) / 1e12 if do_pre else None,
               "alg_gbs": pb / (pre_ms * 1e-3) / 1e9 if do_pre else None}
    if do_pre:
        prefill["mfma_frac_alg"] = prefill["alg_tflops"] / MFMA_F16_PEAK_TFLOPS
        prefill["hbm_frac_alg"] = prefill["alg_gbs"] / HBM_PEAK_GBS
        prefill["roofline_frac"] = max(pf / (MFMA_F16_PEAK_TFLOPS * 1e12), pb / (HBM_PEAK_GBS * 1e9)) / (pre_ms * 1e-3)
    decode = {"ms": dec_ms, "ms_median": statistics.median(dec_t),
              "states_per_s": B * hv / (dec_ms * 1e-3) if do_dec else None,
              "requests_per_s": B / (dec_ms * 1e-3) if do_dec else None,
              "alg_gbs": db / (dec_ms * 1e-3) / 1e9 if do_dec else None}
    if do_dec:
        decode["hbm_frac_alg"] = decode["alg_gbs"] / HBM_PEAK_GBS
    fused = None
    if fsteps > 0:
        io_b = 2   # bf16 raw gate and beta inputs
        _, fpb = prefill_work(cu, hk, hv, dk, dv, gate_bytes=io_b)
        fdb = decode_work(B, hk, hv, dk, dv, gate_bytes=io_b)
        fused = {"steps": fsteps}
        if do_pre:
            fused["prefill"] = {"ms": fused_pre_ms, "tokens_per_s": T / (fused_pre_ms * 1e-3),
                                "alg_gbs": fpb / (fused_pre_ms * 1e-3) / 1e9,
                                "alg_tflops": pf / (fused_pre_ms * 1e-3) / 1e12}
        if do_dec:
            fused["decode"] = {"ms": fused_dec_ms, "states_per_s": B * hv / (fused_dec_ms * 1e-3),
                               "alg_gbs": fdb / (fused_dec_ms * 1e-3) / 1e9,
                               "hbm_frac_alg": fdb / (fused_dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}

    # dominant kernel: the decode kernel (one launch per step, timed by the
    # events that bracket it on the stream it runs on)
    if do_pre:
        # (the record covers the 16-sequence workload only)
        ptr = None if (long_prompt or lengths) else measured_traffic(PREFILL_TRAFFIC_FILE, PREFILL_SRC)
        # counted HBM bytes of one prefill call (meta, intra and state kernels)
        # and their ratio to the algorithmic bytes
        prefill["traffic"] = ptr.get("traffic_bytes_per_call") if ptr else None
        prefill["traffic_over_alg"] = prefill["traffic"] / pb if prefill["traffic"] else None
    if do_dec:
        # (the record covers the 4096-request workload only)
        dtr = measured_traffic() if B == 4096 else None
        roof = {"kernel": DECODE_KERNEL, "bound": "hbm",
                "achieved": decode["alg_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": decode["alg_gbs"] / HBM_PEAK_GBS,
                "traffic": dtr.get("traffic_bytes_per_launch") if dtr else None,
                "alg_bytes_per_launch": db}
    else:
        roof = {"kernel": "prefill (meta + intra + state)", "bound": "hbm",
                "achieved": prefill["alg_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": prefill["alg_gbs"] / HBM_PEAK_GBS, "traffic": None,
                "alg_bytes_per_launch": pb}

    out = {
        "metric": METRIC,
        "value": prefill["tokens_per_s"] if do_pre else decode["states_per_s"],
        "unit": "tokens/s" if do_pre else "states/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic",
        "config": {"workload": workload_name(args.part, long_prompt, T, B, lengths),
                   "global_batch": len(cu) - 1, "seq_len": T, "parallelism": "single-gpu"},
        "prefill": prefill, "decode": decode, "roofline": roof, "finite": finite,
        "fused_gate": fused, "spec_decode": spec,
    }
    if not args.no_cpu_baseline and do_pre and do_dec:
        out["cpu_baseline"] = cpu_baseline(pre, dec)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
