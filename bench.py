"""Benchmark of the batch-invariant token-logprob path on one MI355X.

One step = one fused LM-head logprob call (leaf-tree contraction + fixed-order
log-softmax + gather) over one prefill chunk of 8192 tokens: hidden 4096,
vocabulary 151936, 8 leaves, bf16 inputs resident in HBM.  The printed JSON
line carries:

* value: whole-job tokens/s over the timed steps (HIP events on the stream the
  kernels run on, bracketed by device synchronisation);
* roofline: the fused kernel is bound by the matrix cores at this size; achieved
  = 2 M K V flops per call / the event-timed duration of one call;
* tree_gemm: the same contraction rate as TFLOP/s and fraction of the bf16
  dense peak;
* decode: one 128-row decode step of the same LM head (bound by streaming the
  1.245 GB weight from HBM), tokens/s and fraction of 8 TB/s;
* cpu_baseline: the fp64 CPU oracle timed on a bounded sample of rows of the
  same workload, on this host's cores (skipped with --no-cpu-baseline).

Inputs are seeded and synthetic (bf16 N(0,1) activations, N(0,0.02) weights);
sampled ids are uniform in [0, V) here (the kernel's cost does not depend on
their values).
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

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E peak


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_digest() -> str:
    """SHA-256 of the kernel source, to tell whether stored counters still apply."""
    import hashlib
    path = os.path.join(ROOT, "invariant_gemm_token_amd", "csrc", "tig_kernels.hip")
    return hashlib.sha256(open(path, "rb").read()).hexdigest()


def measured_traffic(name: str):
    """HBM-side bytes per launch of the fused kernel, from the committed counter summary.

    profiles/<name>_traffic.md holds `traffic_bytes_per_launch:` (FETCH_SIZE +
    WRITE_SIZE of one launch, each scaled by what the same counter reads for a
    1 GiB copy) and the `kernel_source_sha256:` it was measured on; if the
    kernel source has changed since, the figure no longer applies and None is
    returned.
    """
    path = os.path.join(ROOT, "profiles", f"{name}_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.split(":", 1)[0].strip() in ("traffic_bytes_per_launch", "kernel_source_sha256"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_source_sha256") != kernel_source_digest():
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=2048)
    ap.add_argument("--phase", choices=("all", "prefill", "decode"), default="all",
                    help="time only one configuration (for per-kernel profiles)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a 1 GiB device-to-device copy (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path is timed on a single MI355X "
              "(row sharding across GPUs needs no exchange; see the design notes).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import invariant_gemm_token_amd as tig
    import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    tig.load()
    dev = torch.device("cuda:0")
    cfg = wl.CONFIGS["lmhead"]
    M, K, V, L = cfg.n_seq * cfg.n_pos, cfg.K, cfg.N, cfg.leaves
    s = wl.streams(cfg.seed)
    t0 = time.time()
    H = wl.normal_bf16(s["H"], (M, K), 1.0)
    W = wl.normal_bf16(s["W"], (V, K), 0.02)
    ids = wl.uniform_ids(s["ids"], M, V)
    log(f"inputs generated in {time.time() - t0:.1f}s")

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    Hd, Wd, idd = to_dev(H), to_dev(W), torch.from_numpy(ids).to(dev)
    ws = torch.empty(tig.tig_logprob_workspace_bytes(M, K, V, L), dtype=torch.uint8, device=dev)
    lp = torch.empty(M, dtype=torch.float32, device=dev)
    lse = torch.empty(M, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    if args.copy_probe:
        # A plain copy of known size: its FETCH_SIZE / WRITE_SIZE calibrate the counters.
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step():
        tig.tig_logprob_gather(Hd, Wd, idd, lp, lse, L, ws)

    tok_s = ms_step = tflops = None
    flops = 2.0 * M * K * V
    if args.phase in ("all", "prefill"):
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        torch.cuda.synchronize()
        ev[0].record(stream)
        for i in range(args.steps):
            step()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        per_call = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
        total_ms = ev[0].elapsed_time(ev[-1])
        ms_step = total_ms / args.steps
        tok_s = M * args.steps / (total_ms / 1e3)
        avg_call_s = float(np.mean(per_call)) / 1e3
        tflops = flops / avg_call_s / 1e12
        log(f"prefill: {ms_step:.3f} ms/step, {tok_s:.4g} tok/s, {tflops:.1f} TFLOP/s "
            f"(min {min(per_call):.3f} ms, max {max(per_call):.3f} ms)")

    # decode: one step of 128 sequences against the same weights
    Md = cfg.n_seq
    Hdec, iddec = Hd[:Md].contiguous(), idd[:Md].contiguous()
    lpd = torch.empty(Md, dtype=torch.float32, device=dev)
    wsd = torch.empty(tig.tig_logprob_workspace_bytes(Md, K, V, L), dtype=torch.uint8, device=dev)

    def dstep():
        tig.tig_logprob_gather(Hdec, Wd, iddec, lpd, None, L, wsd)

    decode = None
    if args.phase in ("all", "decode"):
        for _ in range(args.warmup):
            dstep()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.decode_steps):
            dstep()
        e1.record(stream)
        torch.cuda.synchronize()
        dec_ms = e0.elapsed_time(e1) / args.decode_steps
        dec_bytes = 2.0 * K * V + 2.0 * Md * K + 8.0 * Md + 4.0 * Md
        dec_gbs = dec_bytes / (dec_ms / 1e3) / 1e9
        log(f"decode M={Md}: {dec_ms * 1e3:.1f} us/step, {dec_gbs:.0f} GB/s")
        decode = {"tokens": Md, "us_per_step": dec_ms * 1e3, "tokens_per_s": Md / (dec_ms / 1e3),
                  "achieved_GBs": dec_gbs, "peak_GBs": PEAK_HBM_GBS, "hbm_frac": dec_gbs / PEAK_HBM_GBS,
                  "algorithmic_bytes": dec_bytes}

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        try:
            from threadpoolctl import threadpool_info
            threads = max((i.get("num_threads", 1) for i in threadpool_info()
                           if i.get("user_api") == "blas"), default=os.cpu_count())
        except Exception:
            threads = os.cpu_count()
        rows = np.arange(args.cpu_rows)
        t0 = time.perf_counter()
        oracle.logprob_ref(H[rows], W, ids[rows])
        dt = time.perf_counter() - t0
        cpu = {"value": args.cpu_rows / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
               "sample": f"first {args.cpu_rows} of the {M} prefill rows, full vocabulary {V}, "
                         f"fp64 numpy (includes converting W to fp64), {dt:.1f}s"}
        log(f"cpu oracle: {cpu['value']:.3g} tok/s on {threads} threads")

    out = {
        "metric": "logprob tokens/s (LM head 4096x151936 bf16) + tree-GEMM TFLOP/s, % MFMA peak",
        "value": tok_s, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "lmhead_logprob_prefill", "hidden": K, "vocab": V, "tokens": M,
                   "leaves": L, "global_batch": M, "parallelism": "none"},
        "roofline": None if tflops is None else {
            "bound": "mfma", "achieved": tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": tflops / PEAK_BF16_TFLOPS, "traffic": measured_traffic("lmhead_prefill")},
        "tree_gemm": None if tflops is None else {
            "tflops": tflops, "mfma_frac": tflops / PEAK_BF16_TFLOPS,
            "shape": f"M={M} K={K} N={V} leaves={L}"},
        "decode": decode,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
