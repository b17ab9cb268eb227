"""Benchmark of the fused all-reduce + residual + RMSNorm epilogue on one MI355X.

One step = one call of the whole path (N-way fp32 reduce, residual add, RMSNorm) over one batch:
N = 8 bf16 partial sums of shape [m = 4096, hidden = 7168] (a tensor-parallel degree of 8 at a
7168-wide hidden state), a bf16 residual and a bf16 weight, synthetic values drawn as N(0, 0.5^2),
N(0, 1) and 1 + 0.1 N(0, 1). Inputs are resident in HBM when timing starts; two copies of every
buffer alternate between steps so that the working set (1.3 GB) exceeds the 256 MB Infinity Cache.

Prints one JSON line: the achieved HBM bandwidth on algorithmic bytes, 2 (N + 3) m hidden +
2 hidden per call, as `value` (GB/s), with the one-stage kernel's roofline, the per-call latency
of the decode shapes (m = 1..32, 2000 calls captured in one HIP graph, minimum over 80 replays,
as the aiter PR #3817 test plan times them) and the CPU oracle's rate on the same workload.

    python bench.py [--steps K] [--warmup W] [--m 4096] [--path 1]
    python bench.py --copy-calib    # a plain 1 GiB device copy, for scaling HBM byte counters
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published peak
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_onestage_n8_m4096_h7168.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "all_reduce_residual_way_amd", "csrc", f)
                  for f in ("kernels.h", "bf16x8.h", "wave_sum.h", "fused_ar.hip")]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--n", type=int, default=8)
    ap.add_argument("--m", type=int, default=4096)
    ap.add_argument("--hidden", type=int, default=7168)
    ap.add_argument("--eps", type=float, default=1e-6)
    ap.add_argument("--path", type=int, default=1, choices=(0, 1, 2))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-decode", action="store_true", help="skip the decode latency sweep")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum CPU time spent timing the oracle")
    ap.add_argument("--copy-calib", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (counter calibration)")
    return ap.parse_args()


def kernel_source_digest():
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the one-stage kernel from the committed counter summary, or None
    if there is none or the kernel sources changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    fields = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256") != kernel_source_digest():
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def algorithmic_bytes(n, m, hidden):
    # read n inputs and the residual, write residual_out and out: 2 (n + 3) m hidden; the weight
    # once: 2 hidden
    return 2 * (n + 3) * m * hidden + 2 * hidden


def copy_calibration(torch):
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(5):
        dst.copy_(src)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / 5
    print(json.dumps({"copy_calibration": {"bytes_read": nbytes, "bytes_written": nbytes,
                                           "launches": 5, "ms_per_copy": ms,
                                           "gbs": 2 * nbytes / ms / 1e6}}), flush=True)


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU's share of the fused epilogue on a single MI355X; "
              f"--gpus {args.gpus} (WORLD_SIZE={world}) is not supported: run it with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import all_reduce_residual_way_amd as fa
    from all_reduce_residual_way_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    fa.library()  # raises if the HIP library is not built
    torch.cuda.set_device(0)

    if args.copy_calib:
        copy_calibration(torch)
        return

    n, m, hidden, eps, path = args.n, args.m, args.hidden, args.eps, args.path
    log(f"generating n={n} m={m} hidden={hidden}")
    prob = synth.make_problem(n, m, hidden, seed=args.seed, eps=eps, name="bandwidth")

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()

    sets = []
    base = {"inputs": [to_dev(x) for x in prob.inputs], "residual": to_dev(prob.residual)}
    weight = to_dev(prob.weight)
    for copy in range(2):
        s = base if copy == 0 else {"inputs": [x.clone() for x in base["inputs"]],
                                    "residual": base["residual"].clone()}
        s["ro"] = torch.empty_like(s["residual"])
        s["out"] = torch.empty_like(s["residual"])
        s["ptrs"] = [x.data_ptr() for x in s["inputs"]]
        sets.append(s)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    handle = stream.cuda_stream
    lib = fa.library()
    ctypes_args = []
    import ctypes
    for s in sets:
        arr = (ctypes.c_void_p * n)(*s["ptrs"])
        ctypes_args.append(arr)

    def step(i, p):
        s = sets[i & 1]
        rc = lib.fused_ar_rmsnorm(ctypes_args[i & 1], n, s["residual"].data_ptr(),
                                  weight.data_ptr(), eps, m, hidden, s["ro"].data_ptr(),
                                  s["out"].data_ptr(), p, handle)
        if rc != 0:
            raise fa.FusedArError(rc, "fused_ar_rmsnorm")

    def timed(p, steps, warmup):
        for i in range(warmup):
            step(i, p)
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for i in range(steps):
            step(i, p)
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / steps

    bytes_alg = algorithmic_bytes(n, m, hidden)
    plan = fa.describe_launch(n, m, hidden, path)
    log(f"timing path {path}: {args.steps} steps after {args.warmup} warm-up")
    ms = timed(path, args.steps, args.warmup)
    gbs = bytes_alg / (ms * 1e-3) / 1e9

    # sampled parity of the timed configuration against the oracle (rows are independent)
    import oracle
    rows = np.array([0, 1, m // 2, m - 1])
    got_ro = sets[0]["ro"][rows].cpu().view(torch.int16).numpy().view(np.uint16)
    got_out = sets[0]["out"][rows].cpu().view(torch.int16).numpy().view(np.uint16)
    want_ro, want_out = oracle.fused([x[rows] for x in prob.inputs], prob.residual[rows],
                                     prob.weight, eps)
    ords = [np.where(b & 0x8000, -(b & 0x7FFF).astype(np.int32), b.astype(np.int32))
            for b in (got_out, want_out)]
    parity_ok = bool(np.array_equal(got_ro, want_ro) and np.abs(ords[0] - ords[1]).max() <= 1)

    other = {}
    for p in (1, 2):
        pms = ms if p == path else timed(p, max(args.steps // 2, 10), args.warmup)
        other[str(p)] = {"us_per_call": pms * 1e3,
                         "gbs_algorithmic": bytes_alg / (pms * 1e-3) / 1e9,
                         "kernels": [k["name"] for k in fa.describe_launch(n, m, hidden, p)["kernels"]]}

    decode = None
    if not args.no_decode:
        decode = {}
        dn, dh = 8, 7168
        for dm in (1, 2, 4, 8, 16, 32):
            log(f"decode latency m={dm}")
            dp = synth.make_problem(dn, dm, dh, seed=dm, name="decode")
            ins = [to_dev(x) for x in dp.inputs]
            res, w = to_dev(dp.residual), to_dev(dp.weight)
            ro, out = torch.empty_like(res), torch.empty_like(res)
            arr = (ctypes.c_void_p * dn)(*[x.data_ptr() for x in ins])
            for _ in range(3):
                lib.fused_ar_rmsnorm(arr, dn, res.data_ptr(), w.data_ptr(), 1e-6, dm, dh,
                                     ro.data_ptr(), out.data_ptr(), 1, handle)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                gh = torch.cuda.current_stream().cuda_stream
                for _ in range(2000):
                    rc = lib.fused_ar_rmsnorm(arr, dn, res.data_ptr(), w.data_ptr(), 1e-6, dm, dh,
                                              ro.data_ptr(), out.data_ptr(), 1, gh)
                    if rc != 0:
                        raise fa.FusedArError(rc, "fused_ar_rmsnorm (capture)")
            best = float("inf")
            for _ in range(80):
                start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                start.record()
                g.replay()
                end.record()
                torch.cuda.synchronize()
                best = min(best, start.elapsed_time(end))
            decode[str(dm)] = round(best / 2000 * 1e3, 3)  # us per call
            del g

    cpu = None
    if not args.no_cpu:
        log(f"timing the CPU oracle for at least {args.cpu_seconds:.0f} s")
        passes, t0 = 0, time.perf_counter()
        while True:
            oracle.fused(prob.inputs, prob.residual, prob.weight, eps)
            passes += 1
            elapsed = time.perf_counter() - t0
            if elapsed >= args.cpu_seconds:
                break
        cpu = {"value": round(passes * bytes_alg / elapsed / 1e9, 4), "unit": "GB/s", "cores": 1,
               "kind": "oracle",
               "sample": f"the whole timed workload (n={n}, m={m}, hidden={hidden}), {passes} "
                         f"pass(es) in {elapsed:.1f} s, single-threaded C oracle"}

    traffic = measured_traffic() if (n, m, hidden, path) == (8, 4096, 7168, 1) else None
    props = torch.cuda.get_device_properties(0)
    kname = plan["kernels"][0]["name"] if path == 1 else "stage2_norm"
    result = {
        "metric": "µs/call (m≤32) and achieved HBM GB/s (% of peak) at N=8, hidden=7168",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "storage_dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"fused reduce + residual + RMSNorm, N={n} bf16 partial sums "
                               f"[m={m}, hidden={hidden}], eps={eps}",
                   "n_inputs": n, "m": m, "hidden": hidden, "path": path,
                   "buffer_sets": 2, "launch": plan["kernels"]},
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": kname, "avg_launch_us": round(ms * 1e3, 3),
                     "algorithmic_bytes_per_launch": bytes_alg},
        "cpu_baseline": cpu,
        "paths": other,
        "decode_us_per_call": decode,
        "parity_sampled_rows_ok": parity_ok,
        "device": props.name,
        "cus": props.multi_processor_count,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
