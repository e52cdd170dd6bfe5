#!/usr/bin/env python3
"""Headline benchmark: batched homomorphic rotation (hybrid key switching) on
one MI355X.

Workload (the HRot throughput recipe): N = 2^16, L = 24 ciphertext primes of
54 bits, K = 8 special primes of 60 bits, dnum = 3, level 23; a batch of 32
ciphertexts, each rotated by its own offset (32 distinct offsets drawn from
[1, 32767]) with its own Galois key.  One step = one ckks_rotate call on the
batch.  Ciphertext and key words are seeded uniform residues: the rotation
performs exactly the same operations on them as on real encryptions and keys
(in RLWE both look uniform), and no scheme arithmetic is needed to make them.

Also reported: the batched NTT (16 polynomials x 24 limbs x 2^16 words) in
GB/s against the HBM peak, the roofline of the dominant kernel measured with
HIP events on the library's stream during the timed region, and the CPU
oracle timed on a bounded sample of the same batch.

Prints ONE JSON line on stdout.
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "HRot (hybrid key-switch) ops/s at N=2^16,L=24,dnum=3; NTT GB/s vs HBM peak"
HBM_PEAK_GBPS = 8000.0
BYTES_PER_HROT = 150_994_944  # ciphertext in (24 MiB) + key (96 MiB) + ciphertext out (24 MiB)
# modmul-class operations per HRot at level 23: 83.9M butterflies (160 limb
# transforms), 44.0M ModUp, 16.8M inner product, 32.5M ModDown
OPS_PER_HROT = 177_200_000
# Derived ALU peak in modmul-class operations per second: 256 CUs x 4 SIMDs x
# 16 lanes x 2.4 GHz = 39.32 T 32-bit lane-operations/s, at 16 lane-operations
# per 64-bit modmul-class operation (the measured lazy butterfly is 2.3 T/s).
# It decides a kernel's bound; the measured R_mm gives the ALU fractions.
ALU_PEAK_OPS = 256 * 4 * 16 * 2.4e9 / 16
# limbs of 2^16 words each kernel family reads or writes per ciphertext at
# level 23 (its own I/O, intermediates included)
# ciphertexts per launch of the dominant kernel (the key switch's chunk)
DOMINANT_ITEMS_PER_LAUNCH = 4
KERNEL_IO_LIMBS = {
    # per ciphertext limb: 2 converted limbs (the other digits) + 1 input limb
    # (its own digit) + 3 x 2 key limbs + 2 ModDown limbs + 1 limb of tau_g(c0)
    # read, 2 output limbs written: 24 x (2 + 1 + 6 + 2 + 1 + 2)
    "comb_ip": 48 + 24 + 144 + 48 + 24 + 48,
}


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


# Sources the dominant kernel is compiled from: HBM traffic taken with
# rocprofv3 counters is reported only while these are unchanged.
KERNEL_SOURCES = ["keyswitch.hip", "rowpass.h", "ntt_core.h", "arith.h", "internal.h", "kernels.h", "automorph.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "comb_ip_c3_traffic.txt")


def kernel_sources_sha256():
    import hashlib

    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "private_rns_ckks_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary (FETCH_SIZE and WRITE_SIZE, each scaled by the same counter's
    reading for a copy of known size), or None when the kernel's sources have
    changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            kv = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith("#"))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("sources_sha256") != kernel_sources_sha256():
        return None
    try:
        return int(float(kv["fetch_bytes_per_launch"]) + float(kv["write_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def copy_probe(lib):
    """The library's plain device copy of 1 GiB (include/ckks_probe.h, probe
    "copy"; 16 launches): the reference reading for the FETCH_SIZE /
    WRITE_SIZE counters, each launch reading and writing 2^30 B."""
    lib.ckks_probe_rate("copy", copy_bytes=1 << 30)


def cpu_baseline(cfg, q, p, cts, gs, keys, target_s, got):
    """The CPU oracle on a bounded sample of the batch (same words), and the
    parity of the GPU's output words for the items the sample computed."""
    import numpy as np

    import oracle

    P = oracle.Params(cfg["log_n"], q, p, cfg["dnum"])
    level = cfg["L"] - 1
    t0 = time.perf_counter()
    ref0 = oracle.rotate_batch(P, level, cts[:1], gs[:1], keys[:1])
    t1 = time.perf_counter() - t0
    checked = {0: int(np.count_nonzero(ref0[0] != got[0]))}
    # items 1..B-1 of the batch, cycled until about target_s of work
    k = max(1, int(round(target_s / max(t1, 1e-3))))
    B = len(gs)
    done, dt = 0, 0.0
    while done < k:
        lo = 1 + done % (B - 1)
        hi = min(B, lo + (k - done))
        t0 = time.perf_counter()
        ref = oracle.rotate_batch(P, level, cts[lo:hi], gs[lo:hi], keys[lo:hi])
        dt += time.perf_counter() - t0
        for i in range(lo, hi):
            checked[i] = int(np.count_nonzero(ref[i - lo] != got[i]))
        done += hi - lo
    cores = oracle.num_threads()
    # one-thread figure on one rotation of the sample
    oracle.set_num_threads(1)
    t0 = time.perf_counter()
    oracle.rotate_batch(P, level, cts[1:2], gs[1:2], keys[1:2])
    t_one = time.perf_counter() - t0
    oracle.set_num_threads(cores)
    parity = {
        "status": "bit-exact" if not any(checked.values()) else "MISMATCH",
        "items_checked": sorted(checked),
        "words_checked": len(checked) * int(got[0].size),
        "mismatched_words": int(sum(checked.values())),
        "against": "CPU oracle (oracle/ckks_oracle.c), same input words, every word of each checked item",
    }
    return {
        "value": k / dt,
        "unit": "HRot/s",
        "cores": cores,
        "kind": "oracle",
        "sample": "%d rotations of the C3 batch (items 1..%d cycled), same words as the GPU run, "
                  "plain __int128 %% oracle with OpenMP over limbs/coefficients; %.1f s" % (k, B - 1, dt),
        "value_1thread": round(1.0 / t_one, 4),
        "cpu_model": cpu_model(),
    }, parity


def cpu_model():
    """Host CPU model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-ntt", action="store_true")
    ap.add_argument("--no-workloads", action="store_true", help="skip the C4 / C5 timings")
    ap.add_argument("--copy-probe", action="store_true",
                    help="first copy 1 GiB with the library's probe copy kernel (reference for HBM byte counters)")
    ap.add_argument("--ntt-only", action="store_true",
                    help="time only the C2 batched NTT and print its figures (for profiling the transform)")
    ap.add_argument("--serial", action="store_true",
                    help="run the batch's chunks one after another on one stream (CKKS_LANES=1): kernels do not "
                         "overlap, for per-kernel counters")
    ap.add_argument("--no-calibration", action="store_true",
                    help="skip the calibration probes (the ALU ceiling and copy rate are then not reported)")
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="print a per-kernel markdown table from the rocprofv3 CSV output under DIR (kernel trace "
                         "and counter collection runs) and exit")
    ap.add_argument("--traffic-out", metavar="FILE",
                    help="with --summarize-counters: also write the dominant kernel's scaled FETCH_SIZE / "
                         "WRITE_SIZE bytes per launch to FILE (read back by later runs while its sources match)")
    ap.add_argument("--traffic-command", default="",
                    help="the counter command recorded in the --traffic-out file")
    ap.add_argument("--probe", action="store_true",
                    help="measure the device calibration probes (instruction and modular-primitive rates, copy "
                         "rate by size) and print them as one JSON line")
    args = ap.parse_args()
    if args.summarize_counters:
        print(summarize_counters(args.summarize_counters, args.traffic_out, args.traffic_command))
        return 0
    if args.serial:
        os.environ["CKKS_LANES"] = "1"  # read by the library at its first batched call
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(a rotation batch would shard by ciphertext, with no exchange between GPUs). "
              "Run with --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import ckks_synth as S
    import private_rns_ckks_amd as lib

    cfg = S.CONFIGS["C3"]
    N, L, K, dnum = 1 << cfg["log_n"], cfg["L"], cfg["K"], cfg["dnum"]
    level, B = L - 1, cfg["batch"]
    torch.cuda.set_device(0)
    if args.copy_probe:
        copy_probe(lib)
    if args.probe:
        print(json.dumps({"probe": calibration(lib, copy_sizes_mib=PROBE_COPY_MIB)}), flush=True)
        return 0
    if args.ntt_only:
        print(json.dumps({"ntt": ntt_bench(lib, S, torch, np, args)}), flush=True)
        return 0
    q = lib.ckks_find_primes(cfg["log_n"], cfg["q_bits"], L)
    p = lib.ckks_find_primes(cfg["log_n"], cfg["p_bits"], K)
    ctx = lib.Context(cfg["log_n"], q, p, dnum, device=0)

    seed = 3
    log("generating inputs")
    cts = S.uniform_limbs(S.stream(seed, "bench/ct"), q, N, lead=(B, 2))
    offsets = S.distinct_offsets(S.stream(seed, "bench/offsets"), B, *cfg["offset_range"])
    gs = [pow(5, int(k), 2 * N) for k in offsets]
    keys_h = [S.uniform_limbs(S.stream(seed, "bench/evk/%d" % b), q + p, N, lead=(dnum, 2)) for b in range(B)]
    d_ct = torch.from_numpy(cts.view(np.int64)).cuda()
    d_keys = [torch.from_numpy(k.view(np.int64)).cuda() for k in keys_h]
    d_out = torch.empty_like(d_ct)
    stream = torch.cuda.current_stream()

    def step():
        lib.ckks_rotate(ctx, d_ct, d_out, B, level, gs, d_keys, 0, stream)

    for _ in range(args.warmup):
        step()
    # headline: K steps, each bracketed by HIP events on the call's stream, no
    # tracing; the reported step time is the median, the total is kept too
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    ms_median = step_ms[len(step_ms) // 2]
    ms_mean = sum(step_ms) / len(step_ms)
    value = B / (ms_median / 1e3)
    log("HRot/s %.1f  (median %.3f ms, mean %.3f ms per batch of %d)" % (value, ms_median, ms_mean, B))

    # device ceilings measured on this GPU: the library's lazy forward
    # butterfly rate is the modmul-class operation rate R_mm
    cal = None if args.no_calibration else calibration(lib, copy_sizes_mib=(128, 1024))
    r_mm = cal["butterfly_ct"] * 1e12 if cal else None
    copy_gbps = cal["copy_GBps"]["1024"] if cal else None

    # dominant kernel: a second pass of K steps with HIP events around each of
    # its launches (recorded by the library on the stream it launches on)
    trace = lib.KernelTrace(ctx, lib.DOMINANT_KERNEL)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kstat = trace.read()
    trace.close()
    roof = None
    if kstat["launches"]:
        avg_s = kstat["total_ms"] / kstat["launches"] / 1e3
        items_per_launch = B * args.steps / kstat["launches"]
        alg_bytes = items_per_launch * BYTES_PER_HROT      # algorithmic bytes per HRot x HRots per launch
        ops = kstat["alg_units"] / kstat["launches"]       # modmul-class operations per launch
        hbm_gbps = alg_bytes / avg_s / 1e9
        alu_frac = ops / avg_s / r_mm if r_mm else None
        hbm_bound = alg_bytes / (HBM_PEAK_GBPS * 1e9) >= ops / ALU_PEAK_OPS
        roof = {
            "kernel": kstat["name"],
            "bound": "hbm" if hbm_bound else "alu",
            "achieved": round(hbm_gbps, 2) if hbm_bound else round(ops / avg_s / 1e12, 4),
            "peak": HBM_PEAK_GBPS if hbm_bound else round(ALU_PEAK_OPS / 1e12, 4),
            "unit": "GB/s" if hbm_bound else "T modmul-class ops/s",
            "frac": round(hbm_gbps / HBM_PEAK_GBPS, 4) if hbm_bound else round(ops / avg_s / ALU_PEAK_OPS, 4),
            "traffic": measured_traffic(),
            "items_per_launch": items_per_launch,
            "alg_bytes_per_launch": int(alg_bytes),
            "kernel_io_bytes_per_launch": int(items_per_launch * KERNEL_IO_LIMBS[kstat["name"]] * N * 8),
            "alg_ops_per_launch": int(ops),
            "alu_frac": round(alu_frac, 4) if alu_frac is not None else None,
            "avg_launch_us": round(avg_s * 1e6, 2),
            "launches": kstat["launches"],
            "note": "achieved = %d B per HRot x %g HRots per launch / average launch time, from a second pass of "
                    "%d steps with HIP events around each launch (the headline pass runs untraced); chunks run "
                    "on two streams at once, so a launch's time includes co-running kernels of the other stream"
                    % (BYTES_PER_HROT, items_per_launch, args.steps),
        }

    ntt = None
    if not args.no_ntt:
        ntt = ntt_bench(lib, S, torch, np, args)
        for d in ("fwd", "inv"):
            ntt[d + "_copy_frac"] = round(ntt[d + "_GBps"] / copy_gbps, 4) if copy_gbps else None

    workloads = None
    if not args.no_workloads:
        workloads = workload_bench(lib, S, torch, ctx, q, p, stream)
        workloads.update(c1_bench(lib, S, torch, np, stream))

    cpu = parity = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        got = d_out.cpu().numpy().view(np.uint64)
        cpu, parity = cpu_baseline(cfg, q, p, cts, gs, keys_h, args.cpu_seconds, got)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "HRot/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_median, 4),
        "ms_per_step_mean": round(ms_mean, 4),
        "timed_wall_s": round(wall, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u64",
        "data": "synthetic",
        "config": {
            "workload": "HRot batch: N=2^16, L=24 x 54-bit + K=8 x 60-bit primes, dnum=3, level 23, "
                        "32 ciphertexts with distinct offsets in [1,32767] and one Galois key each",
            "batch": B, "N": N, "L": L, "K": K, "dnum": dnum, "level": level,
        },
        "roofline": roof,
        "hbm_roofline_frac": round(value * BYTES_PER_HROT / 1e9 / HBM_PEAK_GBPS, 4),
        "alu_roofline_frac": round(value * OPS_PER_HROT / r_mm, 4) if r_mm else None,
        "r_mm_Tops": round(r_mm / 1e12, 4) if r_mm else None,
        "copy_GBps": copy_gbps,
        "hbm_frac_vs_copy": round(value * BYTES_PER_HROT / 1e9 / copy_gbps, 4) if copy_gbps else None,
        "calibration": cal,
        "parity": parity,
        "ntt": ntt,
        "workloads": workloads,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    ctx.close()
    return 0


def summarize_counters(root, traffic_out=None, command=""):
    """Markdown table per kernel from the rocprofv3 CSVs under root: every
    *_kernel_stats.csv (durations) and *_counter_collection.csv (counters,
    summed per dispatch and averaged over the kernel's dispatches).  FETCH_SIZE
    and WRITE_SIZE are scaled by the factors that make the library's probe
    copy kernel (bench.py --copy-probe: 1 GiB read and written) read and write
    its own size, and reported in MB per dispatch.  With traffic_out, the
    dominant kernel's scaled bytes per dispatch are also written there, in the
    form measured_traffic() reads, tagged with the hash of its sources."""
    import csv
    import glob
    from collections import defaultdict

    dur = {}
    for f in glob.glob(os.path.join(root, "**", "*kernel_stats.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            dur[r["Name"]] = (int(r["Calls"]), float(r["AverageNs"]) / 1e3)
    per = defaultdict(lambda: defaultdict(float))  # (kernel, counter) -> dispatch -> value
    for f in glob.glob(os.path.join(root, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            per[(r["Kernel_Name"], r["Counter_Name"])][(f, r["Dispatch_Id"])] += float(r["Counter_Value"])
    avg = {k: sum(v.values()) / len(v) for k, v in per.items()}
    kernels = sorted({k for k, _ in avg} | set(dur), key=lambda k: -dur.get(k, (0, 0))[0] * dur.get(k, (0, 0))[1])
    copy = next((k for k, _ in avg if "copy_kernel" in k), "copy_kernel")
    fscale = wscale = 1.0
    # the copy probe copies 1 GiB: 1048576 KiB read and written
    if (copy, "FETCH_SIZE") in avg:
        fscale = 1048576.0 / avg[(copy, "FETCH_SIZE")]
    if (copy, "WRITE_SIZE") in avg:
        wscale = 1048576.0 / avg[(copy, "WRITE_SIZE")]
    names = sorted({c for _, c in avg})
    head = ("| Kernel | Calls | Average (us) | " + " | ".join(names) +
            " | HBM read per dispatch (MB) | HBM written per dispatch (MB) |")
    lines = [head, "|" + "---|" * (head.count("|") - 1)]
    for k in kernels:
        calls, us = dur.get(k, (0, float("nan")))
        vals = ["%.4g" % avg[(k, c)] if (k, c) in avg else "" for c in names]
        rd = "%.1f" % (avg[(k, "FETCH_SIZE")] * fscale * 1024 / 1e6) if (k, "FETCH_SIZE") in avg else ""
        wr = "%.1f" % (avg[(k, "WRITE_SIZE")] * wscale * 1024 / 1e6) if (k, "WRITE_SIZE") in avg else ""
        lines.append("| `%s` | %d | %.1f | %s | %s | %s |" % (k[:90], calls, us, " | ".join(vals), rd, wr))
    lines.append("")
    lines.append("FETCH_SIZE scale %.4f, WRITE_SIZE scale %.4f (from %s)" % (fscale, wscale, copy))
    if traffic_out:
        import private_rns_ckks_amd as lib

        dom = next(k for k in kernels if lib.DOMINANT_KERNEL + "_kernel" in k)
        f_b = avg[(dom, "FETCH_SIZE")] * fscale * 1024
        w_b = avg[(dom, "WRITE_SIZE")] * wscale * 1024
        n_f = len(per[(dom, "FETCH_SIZE")])
        items = DOMINANT_ITEMS_PER_LAUNCH
        kio = items * KERNEL_IO_LIMBS[lib.DOMINANT_KERNEL] * (1 << 16) * 8
        kname = re.sub(r"\(anonymous namespace\)::|^void |ckks::", "", dom).split("(")[0]
        with open(traffic_out, "w") as f:
            f.write("# HBM traffic per launch of %s on the HRot batch (N=2^16, L=24 + K=8, dnum=3,\n" % kname)
            f.write("# level 23, 32 ciphertexts; launches of %d ciphertexts), %d dispatches averaged.\n" % (items, n_f))
            f.write("# Command (MI355X, repository root; FETCH_SIZE and WRITE_SIZE each in its own run):\n")
            f.write("#   %s\n" % command)
            f.write("# Scale: the probe copy of 1 GiB reads FETCH_SIZE x %.4f and writes WRITE_SIZE x %.4f\n"
                    % (fscale, wscale))
            f.write("# of its size, so the counters are multiplied by those factors.  Kernel I/O bytes\n")
            f.write("# per launch: %d items x %d limbs x 2^16 words x 8 B (every limb the kernel reads\n"
                    % (items, KERNEL_IO_LIMBS[lib.DOMINANT_KERNEL]))
            f.write("# or writes, once); algorithmic bytes per launch: %d HRots x %d B (ciphertext in,\n"
                    % (items, BYTES_PER_HROT))
            f.write("# key, ciphertext out).  bench.py reports traffic while the sources hash to\n")
            f.write("# sources_sha256.\n")
            f.write("sources_sha256: %s\n" % kernel_sources_sha256())
            f.write("fetch_bytes_per_launch: %d\n" % round(f_b))
            f.write("write_bytes_per_launch: %d\n" % round(w_b))
            f.write("kernel_io_bytes_per_launch: %d\n" % kio)
            f.write("algorithmic_bytes_per_launch: %d\n" % (items * BYTES_PER_HROT))
    return "\n".join(lines)


PROBE_COPY_MIB = (16, 32, 64, 128, 192, 256, 384, 512, 1024, 2048)


def calibration(lib, copy_sizes_mib=(1024,)):
    """Measured device ceilings (include/ckks_probe.h): every ALU probe in
    lane-operations per second, and the copy rate (bytes read + written per
    second) at each size in MiB."""
    out = {}
    for name in lib.ckks_probe_list():
        if name == "copy":
            continue
        rate, _ = lib.ckks_probe_rate(name)
        out[name] = round(rate / 1e12, 4)
    out["unit"] = "T lane-ops/s"
    out["copy_GBps"] = {str(m): round(lib.ckks_probe_rate("copy", copy_bytes=m << 20)[0] / 1e9, 1)
                        for m in copy_sizes_mib}
    return out


def uniform_dev(torch, moduli, N, lead):
    """Uniform residues generated on the device: [*lead][len(moduli)][N] int64 words, limb i below moduli[i]."""
    out = torch.empty(tuple(lead) + (len(moduli), N), dtype=torch.int64, device="cuda")
    for i, m in enumerate(moduli):
        out[..., i, :].random_(0, int(m))
    return out


def workload_bench(lib, S, torch, ctx, q, p, stream, reps=3):
    """Wall time of the other workload recipes on the same parameters:
    C4, the BSGS matrix-vector product (3 inputs at level 12, 12 outputs, 8 x 8
    steps, 15.7 GB of diagonals); C5, 48 ciphertext products with
    relinearisation and rescale followed by 15 rotate-and-sum steps; a
    degree-7 polynomial on the 48 ciphertexts; A x V, the BSGS product with
    576 ciphertext diagonals (7.9 GB)."""
    N = 1 << S.CONFIGS["C4"]["log_n"]
    dnum = S.CONFIGS["C4"]["dnum"]
    res = {}
    c4 = S.CONFIGS["C4"]
    level, n_in, n_out, n1, n2 = c4["level"], c4["n_in"], c4["n_out"], c4["n1"], c4["n2"]
    nq = level + 1
    x = uniform_dev(torch, q[:nq], N, (n_in, 2))
    diags = uniform_dev(torch, q[:nq], N, (n_out, n_in, n2, n1))
    kb = [uniform_dev(torch, q + p, N, (dnum, 2)) for _ in range(n1 - 1)]
    kg = [uniform_dev(torch, q + p, N, (dnum, 2)) for _ in range(n2 - 1)]
    gb = [pow(5, b, 2 * N) for b in range(1, n1)]
    gg = [pow(5, n1 * g, 2 * N) for g in range(1, n2)]
    y = torch.empty((n_out, 2, level, N), dtype=torch.int64, device="cuda")

    def run_c4():
        lib.ckks_ptmatvec(ctx, x, n_in, diags, n_out, n1, n2, gb, kb, gg, kg, y, level, 0, stream)

    res["c4_ptmatvec_ms"] = round(timed(torch, stream, run_c4, reps), 3)
    del x, diags, kb, kg, y
    torch.cuda.empty_cache()
    c5 = S.CONFIGS["C5"]
    B, level, steps = c5["batch"], S.CONFIGS["C5"]["L"] - 1, c5["rotsum_steps"]
    a = uniform_dev(torch, q, N, (B, 2))
    b = uniform_dev(torch, q, N, (B, 2))
    rlk = uniform_dev(torch, q + p, N, (dnum, 2))
    keys = [uniform_dev(torch, q + p, N, (dnum, 2)) for _ in range(steps)]
    gs = [pow(5, 1 << k, 2 * N) for k in range(steps)]
    bufs = [torch.empty((B, 2, level, N), dtype=torch.int64, device="cuda") for _ in range(2)]

    def run_c5():
        lib.ckks_mul_relin_rescale(ctx, a, b, rlk, bufs[0], B, level, 0, stream)
        for k in range(steps):
            lib.ckks_rotate(ctx, bufs[k % 2], bufs[(k + 1) % 2], B, level - 1, [gs[k]] * B, [keys[k]] * B,
                            lib.CKKS_ROT_ACCUMULATE, stream)

    res["c5_mul_rotsum_ms"] = round(timed(torch, stream, run_c5, reps), 3)
    # polynomial evaluation (degree 7, Horner) on the 48 ciphertexts at level 23
    coeffs = [1.0, 1.0, 0.5, 1 / 6, 1 / 24, 1 / 120, 1 / 720, 1 / 5040]
    pe_out = torch.empty((B, 2, level + 1 - 7, N), dtype=torch.int64, device="cuda")
    a_top = uniform_dev(torch, q, N, (B, 2))

    def run_pe():
        lib.ckks_poly_eval(ctx, a_top, B, level, 2.0 ** 54, coeffs, rlk, pe_out, stream)

    res["poly_eval_deg7_ms"] = round(timed(torch, stream, run_pe, reps), 3)
    # the same polynomial, and a degree-15 one, by the depth-efficient split
    # (depth 3 and 4; 5 and 10 ciphertext products per item, against 6 and 14 for Horner)
    c15 = [(-1) ** k / (k + 1) for k in range(16)]
    tree_out = {d: torch.empty((B, 2, level + 1 - lib.tree_depth(d), N), dtype=torch.int64, device="cuda")
                for d in (7, 15)}

    def run_tree7():
        lib.ckks_poly_eval_tree(ctx, a_top, B, level, 2.0 ** 54, coeffs, rlk, tree_out[7], stream)

    def run_tree15():
        lib.ckks_poly_eval_tree(ctx, a_top, B, level, 2.0 ** 54, c15, rlk, tree_out[15], stream)

    res["poly_eval_tree_deg7_ms"] = round(timed(torch, stream, run_tree7, reps), 3)
    res["poly_eval_tree_deg15_ms"] = round(timed(torch, stream, run_tree15, reps), 3)
    del a, b, a_top, keys, bufs, pe_out, tree_out
    torch.cuda.empty_cache()
    # attention output A x V with encrypted weights (ckks_ctmatvec)
    av = S.CONFIGS["AV"]
    level, n_in, n_out, n1, n2 = av["level"], av["n_in"], av["n_out"], av["n1"], av["n2"]
    nq = level + 1
    x = uniform_dev(torch, q[:nq], N, (n_in, 2))
    diags = uniform_dev(torch, q[:nq], N, (n_out, n_in, n2, n1, 2))
    kb = [uniform_dev(torch, q + p, N, (dnum, 2)) for _ in range(n1 - 1)]
    kg = [uniform_dev(torch, q + p, N, (dnum, 2)) for _ in range(n2 - 1)]
    gb = [pow(5, b, 2 * N) for b in range(1, n1)]
    gg = [pow(5, n1 * g, 2 * N) for g in range(1, n2)]
    y = torch.empty((n_out, 2, level, N), dtype=torch.int64, device="cuda")

    def run_av():
        lib.ckks_ctmatvec(ctx, x, n_in, diags, n_out, n1, n2, rlk, gb, kb, gg, kg, y, level, 0, stream)

    res["av_ctmatvec_ms"] = round(timed(torch, stream, run_av, reps), 3)
    del x, diags, kb, kg, y
    torch.cuda.empty_cache()
    res["note"] = "C4: one ckks_ptmatvec call; C5: ckks_mul_relin_rescale on 48 pairs + 15 accumulate rotations " \
                  "of the 48 products (768 key switches); poly_eval: degree-7 Horner evaluation on 48 ciphertexts " \
                  "at level 23 (6 products each, depth 7); poly_eval_tree: the same degree-7 polynomial and a " \
                  "degree-15 one by the depth-efficient split (depth 3 and 4); av: one ckks_ctmatvec call (A x V, 3 inputs, 3 outputs, 576 " \
                  "ciphertext diagonals at level 12, 24 relinearisations); c1: one ckks_rotate of a C1 " \
                  "ciphertext (N=2^12) by 1 and by 7, time per rotation over 20 reps; device-generated uniform " \
                  "words, %d timed reps" % reps
    log("C4 ptmatvec %.2f ms, C5 %.2f ms, poly_eval %.2f ms, A x V %.2f ms"
        % (res["c4_ptmatvec_ms"], res["c5_mul_rotsum_ms"], res["poly_eval_deg7_ms"], res["av_ctmatvec_ms"]))
    return res


def c1_bench(lib, S, torch, np, stream, reps=20):
    """The tiny configuration (N=2^12, 4 x 30-bit + 1 x 60-bit primes, dnum=4):
    one ciphertext rotated by 1 and by 7 in one call; time per rotation."""
    cfg = S.CONFIGS["C1"]
    N = 1 << cfg["log_n"]
    q = lib.ckks_find_primes(cfg["log_n"], cfg["q_bits"], cfg["L"])
    p = lib.ckks_find_primes(cfg["log_n"], cfg["p_bits"], cfg["K"])
    ctx = lib.Context(cfg["log_n"], q, p, cfg["dnum"], device=0)
    level = cfg["L"] - 1
    ks = list(cfg["rotations"])
    ct = uniform_dev(torch, q, N, (1, 2)).expand(len(ks), 2, len(q), N).contiguous()
    keys = [uniform_dev(torch, q + p, N, (cfg["dnum"], 2)) for _ in ks]
    gs = [pow(5, k, 2 * N) for k in ks]
    out = torch.empty_like(ct)

    def run():
        lib.ckks_rotate(ctx, ct, out, len(ks), level, gs, keys, 0, stream)

    t = timed(torch, stream, run, reps)
    ctx.close()
    return {"c1_rotate_us": round(t * 1e3 / len(ks), 2)}


def timed(torch, stream, fn, reps):
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def ntt_bench(lib, S, torch, np, args):
    """16 polynomials x 24 limbs x 2^16 words, forward and inverse, GB/s at 16 B per coefficient."""
    cfg = S.CONFIGS["C2"]
    N = 1 << cfg["log_n"]
    q = lib.ckks_find_primes(cfg["log_n"], cfg["q_bits"], cfg["L"])
    ctx = lib.Context(cfg["log_n"], q, [], 1, device=0)
    x = S.uniform_limbs(S.stream(2, "bench/ntt"), q, N, lead=(cfg["npoly"],))
    d = torch.from_numpy(x.view(np.int64)).cuda()
    stream = torch.cuda.current_stream()
    res = {}
    nbytes = cfg["npoly"] * cfg["L"] * N * 16
    for name, inv in (("fwd", 0), ("inv", 1)):
        for _ in range(3):
            lib.ckks_ntt(ctx, d, cfg["npoly"], 0, cfg["L"], inv, stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 20
        e0.record(stream)
        for _ in range(reps):
            lib.ckks_ntt(ctx, d, cfg["npoly"], 0, cfg["L"], inv, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / reps / 1e3
        res[name + "_GBps"] = round(nbytes / t / 1e9, 1)
        res[name + "_us"] = round(t * 1e6, 1)
        res[name + "_hbm_frac"] = round(nbytes / t / 1e9 / HBM_PEAK_GBPS, 4)
    res["shape"] = "16 x 24 x 2^16 u64, %d B per direction" % nbytes
    log("NTT fwd %.1f GB/s, inv %.1f GB/s" % (res["fwd_GBps"], res["inv_GBps"]))
    ctx.close()
    return res


if __name__ == "__main__":
    sys.exit(main())
