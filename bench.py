"""Benchmark of the batch-invariant token-logprob path on one MI355X.

One step = one fused LM-head logprob call (leaf-tree contraction + fixed-order
log-softmax + gather) over one prefill chunk of 8192 tokens: hidden 4096,
vocabulary 151936, 8 leaves, bf16 inputs resident in HBM.  The printed JSON
line carries:

* value: whole-job tokens/s over the timed steps (HIP events on the stream the
  kernels run on, bracketed by device synchronisation);
* roofline: the fused LM-head kernel is bound by the matrix cores at this
  size; achieved = 2 M K V flops per call / the event-timed duration of one
  call, against the bf16 dense peak; traffic = HBM-side bytes per launch from
  the committed counter summary, when it was taken on this kernel source;
* tree_gemm: the leaf-tree contraction entry point alone at the same shape
  (8192 x 4096 x 151936, 8 leaves; FP32 and bf16 output), TFLOP/s and
  fraction of the peak;
* clock: the GFX clock and board power sampled while the prefill runs in a
  loop, and the matrix-core peak at that clock (256 CUs x 4096 flop/clock);
* vendor_plain_gemm_context: torch.matmul (the vendor library's plain bf16
  GEMM, no leaf tree, no log-softmax) at the same shape, timed on the same
  box with its clock and power: context for what the board sustains, not
  part of the path;
* decode: one 128-row decode step of the same LM head (bound by streaming the
  1.245 GB weight from HBM), tokens/s and fraction of 8 TB/s;
* linear, moe, large: the other workloads of the path, each with its own
  roofline: the 4096 x 4096 linear layer at 4096 and 4097 rows (matrix
  cores), the MoE-shaped contraction (64 experts 2048 -> 1408, top-8 of 4096
  tokens, matrix cores), and the hidden-7168 / vocabulary-129280 LM head at
  16 leaves (16384-row prefill: matrix cores; 256-row decode: both);
* cpu_baseline: the fp64 CPU oracle timed on a bounded sample of rows of the
  headline workload, on this host's cores, plus the same oracle on every other
  workload (rows/s and fp64 GFLOP/s; skipped with --no-cpu-baseline).

Inputs are seeded and synthetic (workloads: bf16 N(0,1) activations,
N(0,0.02) weights, uniform sampled ids, top-8 routing of N(0,1) router
logits); a kernel's cost does not depend on the values.

The headline runs exactly --warmup untimed steps before its --steps timed ones.
Every other line first calls its kernel back to back for at least 200 ms, so
that it is not timed while the GPU clock comes back from an idle spell (input
generation, the CPU baseline).
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
AUX_WARM_MS = 200.0         # back-to-back calls before each line other than the headline
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 matrix-core peak


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
    ap.add_argument("--cpu-rows", type=int, default=8192)   # about 11 s of the fp64 oracle on 16 cores
    ap.add_argument("--cpu-rows-large", type=int, default=256)
    ap.add_argument("--no-extra", action="store_true", help="skip the linear / moe / large lines")
    ap.add_argument("--phase", choices=("all", "prefill", "decode", "tree"), default="all",
                    help="time only one LM-head configuration (for per-kernel profiles)")
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
    stream = torch.cuda.current_stream()

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def settle(fn, warm_ms):
        """Call fn back to back for at least warm_ms of wall time: after an idle spell
        (input generation, the CPU baseline) the GPU clock needs tens of ms to come back,
        and a short line timed right away measures part of that ramp."""
        import time
        if warm_ms <= 0:
            return
        t0 = time.perf_counter()
        while True:
            for _ in range(8):
                fn()
            torch.cuda.synchronize()
            if (time.perf_counter() - t0) * 1e3 >= warm_ms:
                return

    def timed(fn, steps, warmup, per_call=False, warm_ms=AUX_WARM_MS):
        """Mean ms per call over `steps` calls (events on the launch stream), and with
        per_call the time of each call (an event between calls: fine for long calls, an
        overhead of its own for short ones).  `warmup` calls, then at least warm_ms of
        calls, go first."""
        for _ in range(warmup):
            fn()
        settle(fn, warm_ms)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1 if per_call else 2)]
        ev[0].record(stream)
        for i in range(steps):
            fn()
            if per_call:
                ev[i + 1].record(stream)
        ev[-1].record(stream)
        torch.cuda.synchronize()
        per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)] if per_call else []
        return ev[0].elapsed_time(ev[-1]) / steps, per

    def device_timed(fn, steps, warmup, warm_ms=AUX_WARM_MS):
        """Device time per call of a short call: the calls are queued behind a sleep
        kernel, so the events bracket only GPU work, not the host's time to issue each
        call through the Python binding.  Returns (ms per call, ms per call as issued
        from the host, whether the queue stayed ahead of the GPU)."""
        import time
        for _ in range(warmup):
            fn()
        settle(fn, warm_ms)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        torch.cuda._sleep(int(4e6))   # a few ms of one spinning wave
        s1.record(stream)
        e0.record(stream)
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        t_issue = time.perf_counter() - t0
        e1.record(stream)
        torch.cuda.synchronize()
        dev_ms = e0.elapsed_time(e1) / steps
        # The GPU never waited for the host if issuing all calls took less time than
        # the sleep plus the calls themselves took on the GPU.
        ahead = t_issue * 1e3 < s0.elapsed_time(s1) + dev_ms * steps
        host_ms, _ = timed(fn, steps, 0, warm_ms=0)
        return dev_ms, host_ms, ahead

    def mfma_line(flops, ms):
        tf = flops / (ms / 1e3) / 1e12
        return {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": tf / PEAK_BF16_TFLOPS}

    def hbm_line(nbytes, ms):
        gbs = nbytes / (ms / 1e3) / 1e9
        return {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS}

    def sample_clock(fn, seconds):
        """Run fn in a loop for about `seconds` while sampling the GFX clocks and board power."""
        import subprocess
        import threading
        samples, stop = [], [False]

        def poll():
            while not stop[0]:
                try:
                    r = subprocess.run(["amd-smi", "metric", "-p", "-c", "--json"], capture_output=True, text=True,
                                       timeout=10)
                    d = json.loads(r.stdout)
                    g = (d["gpu_data"] if isinstance(d, dict) else d)[0]
                    clk = [v["clk"]["value"] for k, v in g["clock"].items()
                           if k.startswith("gfx_") and isinstance(v, dict) and isinstance(v.get("clk"), dict)
                           and isinstance(v["clk"].get("value"), (int, float))]
                    pw = g["power"]["socket_power"]["value"]
                    if clk and isinstance(pw, (int, float)):
                        samples.append((float(np.mean(clk)), float(pw)))
                except Exception:
                    pass
                time.sleep(0.2)

        th = threading.Thread(target=poll)
        th.start()
        t0 = time.time()
        while time.time() - t0 < seconds:
            fn()
            torch.cuda.synchronize()
        stop[0] = True
        th.join()
        # drop the first samples (clock still ramping)
        use = samples[2:] if len(samples) > 4 else samples
        if not use:
            return None
        mhz = float(np.median([c for c, _ in use]))
        return {"gfx_mhz_median": mhz, "power_w_median": float(np.median([p for _, p in use])), "samples": len(use),
                "peak_bf16_tflops_at_clock": 256 * 4096 * mhz * 1e6 / 1e12}

    # ---------------- headline: LM-head prefill ----------------
    cfg = wl.CONFIGS["lmhead"]
    M, K, V, L = cfg.n_seq * cfg.n_pos, cfg.K, cfg.N, cfg.leaves
    s = wl.streams(cfg.seed)
    t0 = time.time()
    H = wl.normal_bf16(s["H"], (M, K), 1.0)
    W = wl.normal_bf16(s["W"], (V, K), 0.02)
    ids = wl.uniform_ids(s["ids"], M, V)
    log(f"lm-head inputs generated in {time.time() - t0:.1f}s")
    Hd, Wd, idd = to_dev(H), to_dev(W), torch.from_numpy(ids).to(dev)
    ws = torch.empty(tig.tig_logprob_workspace_bytes(M, K, V, L), dtype=torch.uint8, device=dev)
    lp = torch.empty(M, dtype=torch.float32, device=dev)
    lse = torch.empty(M, dtype=torch.float32, device=dev)

    if args.copy_probe:
        # A plain copy of known size: its FETCH_SIZE / WRITE_SIZE calibrate the counters.
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    copy_gbs = None
    if args.phase == "all":
        # Attainable HBM rate on this machine: a 1 GiB device-to-device copy (bytes read + written).
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        copy_ms, _ = timed(lambda: dst.copy_(src), 10, 2, warm_ms=0)
        copy_gbs = 2.0 * (1 << 30) / (copy_ms / 1e3) / 1e9
        log(f"device copy: {copy_gbs:.0f} GB/s (read + write)")
        del src, dst

    tok_s = ms_step = tflops = None
    spread = None
    flops = 2.0 * M * K * V
    if args.phase in ("all", "prefill"):
        # The headline: exactly args.warmup untimed steps, then args.steps timed ones.
        ms_step, per_call = timed(lambda: tig.tig_logprob_gather(Hd, Wd, idd, lp, lse, L, ws),
                                  args.steps, args.warmup, per_call=True, warm_ms=0)
        tok_s = M / (ms_step / 1e3)
        tflops = flops / (float(np.mean(per_call)) / 1e3) / 1e12
        spread = {"min_ms": float(np.min(per_call)), "median_ms": float(np.median(per_call)),
                  "max_ms": float(np.max(per_call))}
        log(f"prefill: {ms_step:.3f} ms/step, {tok_s:.4g} tok/s, {tflops:.1f} TFLOP/s "
            f"(min {min(per_call):.3f} ms, max {max(per_call):.3f} ms)")

    clock = None
    tree = None
    vendor = None
    if args.phase == "all":
        clock = sample_clock(lambda: tig.tig_logprob_gather(Hd, Wd, idd, lp, lse, L, ws), 3.0)
        if clock is not None and tflops is not None:
            clock["prefill_frac_of_peak_at_clock"] = tflops / clock["peak_bf16_tflops_at_clock"]
            log(f"clock while the prefill runs: {clock['gfx_mhz_median']:.0f} MHz, {clock['power_w_median']:.0f} W; "
                f"peak at that clock {clock['peak_bf16_tflops_at_clock']:.0f} TFLOP/s")
        # Context, not the product path: the vendor's plain bf16 GEMM of the same shape (torch.matmul, no
        # leaf tree, no log-softmax, bf16 output), with the clock and power it runs at on this machine.
        try:
            Wt = Wd.t()
            Cb = torch.empty(M, V, dtype=torch.bfloat16, device=dev)
            ms_ref, _ = timed(lambda: torch.matmul(Hd, Wt, out=Cb), 5, 2)
            ref_clock = sample_clock(lambda: torch.matmul(Hd, Wt, out=Cb), 2.0)
            vendor = {"ms": ms_ref, "tflops": flops / (ms_ref / 1e3) / 1e12, "what": "torch.matmul bf16 out",
                      "clock": ref_clock}
            log(f"vendor plain GEMM (context): {ms_ref:.3f} ms, {vendor['tflops']:.0f} TFLOP/s")
            del Cb, Wt
        except Exception as e:   # the context line never fails the bench
            vendor = {"error": str(e)}
    if args.phase in ("all", "tree"):
        # The leaf-tree contraction entry point alone at the headline shape.
        tree = {"shape": f"M={M} K={K} N={V} leaves={L}"}
        for name, dt in (("fp32_out", torch.float32), ("bf16_out", torch.bfloat16)):
            if args.phase == "tree" and name == "bf16_out":
                continue
            Ct = torch.empty(M, V, dtype=dt, device=dev)
            ms_t, per_t = timed(lambda: tig.tig_tree_gemm(Hd, Wd, Ct, L), 5, 1, per_call=True)
            line = mfma_line(flops, ms_t)
            line["traffic"] = measured_traffic("tree_gemm_lmhead") if name == "fp32_out" else None
            tree[name] = {"ms": ms_t, "min_ms": float(np.min(per_t)), "tflops": line["achieved"],
                          "mfma_frac": line["frac"], "roofline": line,
                          "output_bytes": float(Ct.numel() * Ct.element_size())}
            log(f"tree_gemm {name}: {ms_t:.3f} ms, {line['achieved']:.0f} TFLOP/s")
            del Ct

    decode = None
    if args.phase in ("all", "decode"):
        Md = cfg.n_seq
        Hdec, iddec = Hd[:Md].contiguous(), idd[:Md].contiguous()
        lpd = torch.empty(Md, dtype=torch.float32, device=dev)
        wsd = torch.empty(tig.tig_logprob_workspace_bytes(Md, K, V, L), dtype=torch.uint8, device=dev)
        dec_ms, _ = timed(lambda: tig.tig_logprob_gather(Hdec, Wd, iddec, lpd, None, L, wsd),
                          args.decode_steps, args.warmup)
        dec_bytes = 2.0 * K * V + 2.0 * Md * K + 8.0 * Md + 4.0 * Md
        r = hbm_line(dec_bytes, dec_ms)
        r["traffic"] = measured_traffic("lmhead_decode")
        log(f"decode M={Md}: {dec_ms * 1e3:.1f} us/step, {r['achieved']:.0f} GB/s")
        decode = {"tokens": Md, "us_per_step": dec_ms * 1e3, "tokens_per_s": Md / (dec_ms / 1e3),
                  "achieved_GBs": r["achieved"], "peak_GBs": PEAK_HBM_GBS, "hbm_frac": r["frac"],
                  "algorithmic_bytes": dec_bytes, "roofline": r,
                  "frac_of_device_copy": None if copy_gbs is None else r["achieved"] / copy_gbs}

    # The LM-head contraction alone in block FP8 (W8A8) on the FP8 matrix cores:
    # W quantised once (128 x 128 blocks), the 8192 rows per token (1 x 128).
    fp8_lmhead = None
    if not args.no_extra and args.phase == "all":
        QW8, SW8 = tig.fp8_quantize(Wd, 128)
        QA8, SA8 = tig.fp8_quantize(Hd, 1)
        # re-quantising the BF16 master weights, as a training forward does every step
        ms_wq, _ = timed(lambda: tig.tig_fp8_quantize(Wd, QW8, SW8, 128), 5, 1)
        C8 = torch.empty(M, V, dtype=torch.float32, device=dev)
        ws8 = torch.empty(tig.tig_fp8_gemm_workspace_bytes(M, V, K), dtype=torch.uint8, device=dev)
        ms8, _ = timed(lambda: tig.tig_fp8_tree_gemm(QA8, SA8, QW8, SW8, C8, L, ws8), 5, 1)
        tf8 = 2.0 * M * K * V / (ms8 / 1e3) / 1e12
        fp8_lmhead = {"ms": ms8, "shape": f"M={M} K={K} N={V} leaves={L}",
                      "weight_quantize_ms": ms_wq, "weight_quantize": hbm_line(3.0 * V * K, ms_wq),
                      "roofline": {"bound": "mfma", "achieved": tf8, "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                                   "frac": tf8 / PEAK_FP8_TFLOPS}}
        log(f"fp8 lm-head gemm: {ms8:.2f} ms, {tf8:.0f} TFLOP/s")
        del QW8, SW8, QA8, SA8, C8, ws8

    cpu = None
    do_cpu = not args.no_cpu_baseline and args.phase == "all"
    if do_cpu:
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
                         f"fp64 numpy (includes converting W to fp64), {dt:.1f}s",
               "host_cores": os.cpu_count(), "blas_threads": int(threads),
               "configs": {"lmhead": {"rows": args.cpu_rows, "s": dt, "rows_per_s": args.cpu_rows / dt,
                                      "fp64_gflops": 2.0 * args.cpu_rows * K * V / dt / 1e9}}}
        log(f"cpu oracle: {cpu['value']:.3g} tok/s on {threads} threads ({os.cpu_count()} host cores)")

        def cpu_line(name, nrows, flop, fn):
            t1 = time.perf_counter()
            fn()
            d = time.perf_counter() - t1
            cpu["configs"][name] = {"rows": nrows, "s": d, "rows_per_s": nrows / d, "fp64_gflops": flop / d / 1e9}
            log(f"cpu oracle {name}: {nrows / d:.3g} rows/s, {flop / d / 1e9:.1f} fp64 GFLOP/s ({d:.1f}s)")

        c = wl.CONFIGS["tiny"]
        st = wl.streams(c.seed)
        Ht, Wt = wl.normal_bf16(st["H"], (64, c.K), 1.0), wl.normal_bf16(st["W"], (c.N, c.K), 0.02)
        it = wl.uniform_ids(st["ids"], 64, c.N)
        cpu_line("tiny", 64, 2.0 * 64 * c.K * c.N, lambda: oracle.logprob_ref(Ht, Wt, it))
    del H, W
    del Hd, Wd, idd, ws

    # ---------------- the other workloads of the path ----------------
    linear = moe = large = topk = None
    if not args.no_extra and args.phase == "all":
        c = wl.CONFIGS["linear"]
        sl = wl.streams(c.seed)
        Ah, Wlh = wl.normal_bf16(sl["H"], (4097, c.K), 1.0), wl.normal_bf16(sl["W"], (c.N, c.K), 0.02)
        A, Wl = to_dev(Ah), to_dev(Wlh)
        if do_cpu:
            cpu_line("linear", 4097, 2.0 * 4097 * c.K * c.N, lambda: oracle.contraction_ref(Ah, Wlh))
        del Ah, Wlh
        linear = {}
        for Mr in (4096, 4097):
            Ar = A[:Mr]
            C = torch.empty(Mr, c.N, dtype=torch.float32, device=dev)
            ms, _ = timed(lambda: tig.tig_tree_gemm(Ar, Wl, C, c.leaves), 20, 3)
            linear[f"M{Mr}"] = {"ms": ms, "roofline": mfma_line(2.0 * Mr * c.K * c.N, ms)}
            log(f"linear M={Mr}: {ms * 1e3:.1f} us, {linear[f'M{Mr}']['roofline']['achieved']:.0f} TFLOP/s")
        # The same layer in block FP8 (W8A8): per-token quantisation of the 4096 rows,
        # then the leaf-tree GEMM on the FP8 matrix cores (the weights quantised once).
        QW, SW = tig.fp8_quantize(Wl, 128)
        Ar = A[:4096]
        QA = torch.empty(4096, c.K, dtype=torch.uint8, device=dev)
        SA = torch.empty(4096, c.K // 128, dtype=torch.uint8, device=dev)
        ms_q, _, _ = device_timed(lambda: tig.tig_fp8_quantize(Ar, QA, SA, 1), 50, 3)
        tig.tig_fp8_quantize(Ar, QA, SA, 1)
        C8 = torch.empty(4096, c.N, dtype=torch.float32, device=dev)
        ws8 = torch.empty(tig.tig_fp8_gemm_workspace_bytes(4096, c.N, c.K), dtype=torch.uint8, device=dev)
        ms_g, _ = timed(lambda: tig.tig_fp8_tree_gemm(QA, SA, QW, SW, C8, c.leaves, ws8), 20, 3)
        linear["fp8"] = {"quantize_us": ms_q * 1e3, "quantize": hbm_line(3.0 * 4096 * c.K + 4096 * c.K / 128, ms_q),
                         "gemm_ms": ms_g, "gemm": dict(mfma_line(2.0 * 4096 * c.K * c.N, ms_g),
                                                       peak=PEAK_FP8_TFLOPS,
                                                       frac=2.0 * 4096 * c.K * c.N / (ms_g / 1e3) / 1e12
                                                       / PEAK_FP8_TFLOPS)}
        log(f"linear fp8: quantize {ms_q * 1e3:.1f} us, gemm {ms_g * 1e3:.1f} us")
        del A, Wl, C, QW, SW, QA, SA, C8, ws8

        c = wl.CONFIGS["moe"]
        sm = wl.streams(c.seed)
        Hmh, Weh = wl.normal_bf16(sm["H"], (c.tokens, c.K), 1.0), wl.normal_bf16(sm["W"], (c.experts, c.N, c.K), 0.02)
        Hm, We = to_dev(Hmh), to_dev(Weh)
        tid, tw = wl.routing_input(sm["route"], c.tokens, c.experts, c.topk)
        if do_cpu:
            cpu_line("moe", c.tokens, 2.0 * c.tokens * c.topk * c.K * c.N, lambda: oracle.moe_ref(Hmh, Weh, tid, tw))
        del Hmh, Weh
        tid, tw = torch.from_numpy(tid).to(dev), torch.from_numpy(tw).to(dev)
        out = torch.empty(c.tokens, c.N, dtype=torch.float32, device=dev)
        wsm = torch.empty(tig.tig_moe_workspace_bytes(c.tokens, c.N, c.K, c.experts, c.topk),
                          dtype=torch.uint8, device=dev)
        ms, _ = timed(lambda: tig.tig_moe_tree_gemm_combine(Hm, We, tid, tw, out, c.leaves, wsm), 20, 3)
        moe = {"ms": ms, "shape": f"T={c.tokens} E={c.experts} top{c.topk} K={c.K} N={c.N} leaves={c.leaves}",
               "roofline": mfma_line(2.0 * c.tokens * c.topk * c.K * c.N, ms)}
        log(f"moe: {ms * 1e3:.1f} us, {moe['roofline']['achieved']:.0f} TFLOP/s")
        del out, wsm

        # The same routed rows (32768 = 4096 tokens x top-8) as an expert GEMM on the
        # masked layout (cap = the largest count rounded up to 64) and the contiguous
        # one (segments aligned to 128), then SiLU * up on a [32768, 2 x 1408] FP32
        # gate/up output.
        order = np.argsort(tid.cpu().numpy().reshape(-1), kind="stable")
        cnt = np.bincount(tid.cpu().numpy().reshape(-1), minlength=c.experts).astype(np.int32)
        tok = torch.from_numpy(order // c.topk).to(dev)
        cap = int(-(-cnt.max() // 64) * 64)
        starts = np.concatenate([[0], np.cumsum(-(-cnt // 128) * 128)[:-1]])
        Mc = int(starts[-1] + cnt[-1])
        Xc = torch.zeros(Mc, c.K, dtype=torch.bfloat16, device=dev)
        Xm = torch.zeros(c.experts, cap, c.K, dtype=torch.bfloat16, device=dev)
        first = np.concatenate([[0], np.cumsum(cnt)[:-1]])
        for e in range(c.experts):
            rows = Hm[tok[first[e]:first[e] + cnt[e]]]
            Xc[starts[e]:starts[e] + cnt[e]] = rows
            Xm[e, :cnt[e]] = rows
        cntd = torch.from_numpy(cnt).to(dev)
        flops = 2.0 * float(cnt.sum()) * c.K * c.N
        Ym = torch.empty(c.experts, cap, c.N, dtype=torch.float32, device=dev)
        Yc = torch.empty(Mc, c.N, dtype=torch.float32, device=dev)
        wse = torch.empty(tig.tig_expert_workspace_bytes(max(Mc, c.experts * cap), c.experts), dtype=torch.uint8,
                          device=dev)
        expert = {"shape": f"rows={int(cnt.sum())} E={c.experts} K={c.K} N={c.N} leaves={c.leaves} cap={cap}"}
        ms, _ = timed(lambda: tig.tig_expert_gemm_masked(Xm, cntd, We, Ym, c.leaves, wse), 20, 3)
        expert["masked"] = {"ms": ms, "roofline": mfma_line(flops, ms)}
        ms, _ = timed(lambda: tig.tig_expert_gemm_contiguous(Xc, cntd, We, Yc, 128, c.leaves, wse), 20, 3)
        expert["contiguous"] = {"ms": ms, "roofline": mfma_line(flops, ms)}
        GU = torch.randn(int(cnt.sum()), 2 * c.N, device=dev)
        act = torch.empty(int(cnt.sum()), c.N, dtype=torch.bfloat16, device=dev)
        ms, ms_call, ahead = device_timed(lambda: tig.tig_silu_mul(GU, act), 50, 3)
        expert["silu_mul"] = {"us": ms * 1e3, "us_per_python_call": ms_call * 1e3, "device_timed": ahead,
                              "roofline": hbm_line(10.0 * act.numel(), ms)}
        # The same rows and experts in block FP8 (per-token activations, 128 x 128
        # weight blocks quantised once), and SiLU * up with its FP8 quantisation.
        QXm, SXm = tig.fp8_quantize(Xm.reshape(c.experts * cap, c.K), 1)
        QXc, SXc = tig.fp8_quantize(Xc, 1)
        qws = [tig.fp8_quantize(We[e], 128) for e in range(c.experts)]
        QWe, SWe = torch.stack([q for q, _ in qws]), torch.stack([x for _, x in qws])
        del qws
        wsf = torch.empty(tig.tig_expert_fp8_workspace_bytes(max(Mc, c.experts * cap), c.experts, c.N, c.K),
                          dtype=torch.uint8, device=dev)
        ms, _ = timed(lambda: tig.tig_expert_fp8_gemm_masked(QXm.reshape(c.experts, cap, c.K),
                                                             SXm.reshape(c.experts, cap, c.K // 128), cntd, QWe, SWe,
                                                             Ym, c.leaves, wsf), 20, 3)
        f8 = flops / (ms / 1e3) / 1e12
        expert["fp8_masked"] = {"ms": ms, "roofline": {"bound": "mfma", "achieved": f8, "peak": PEAK_FP8_TFLOPS,
                                                       "unit": "TFLOP/s", "frac": f8 / PEAK_FP8_TFLOPS}}
        ms, _ = timed(lambda: tig.tig_expert_fp8_gemm_contiguous(QXc, SXc, cntd, QWe, SWe, Yc, 128, c.leaves, wsf),
                      20, 3)
        f8 = flops / (ms / 1e3) / 1e12
        expert["fp8_contiguous"] = {"ms": ms, "roofline": {"bound": "mfma", "achieved": f8, "peak": PEAK_FP8_TFLOPS,
                                                           "unit": "TFLOP/s", "frac": f8 / PEAK_FP8_TFLOPS}}
        QA8 = torch.empty(int(cnt.sum()), c.N, dtype=torch.uint8, device=dev)
        SA8 = torch.empty(int(cnt.sum()), -(-c.N // 128), dtype=torch.uint8, device=dev)
        ms, ms_call, ahead = device_timed(lambda: tig.tig_silu_mul_fp8(GU, QA8, SA8), 50, 3)
        expert["silu_mul_fp8"] = {"us": ms * 1e3, "us_per_python_call": ms_call * 1e3, "device_timed": ahead,
                                  "roofline": hbm_line(9.0 * QA8.numel(), ms)}
        log(f"expert fp8 gemm masked {expert['fp8_masked']['ms'] * 1e3:.1f} us, contiguous "
            f"{expert['fp8_contiguous']['ms'] * 1e3:.1f} us; silu_mul_fp8 {expert['silu_mul_fp8']['us']:.1f} us")
        del QXm, SXm, QXc, SXc, QWe, SWe, wsf, QA8, SA8
        moe["expert"] = expert
        log(f"expert gemm masked {expert['masked']['ms'] * 1e3:.1f} us, contiguous "
            f"{expert['contiguous']['ms'] * 1e3:.1f} us; silu_mul {expert['silu_mul']['us']:.1f} us")
        del We, Xc, Xm, Ym, Yc, GU, act, wse

        # The router of the same layer on the GPU: FP32 logits (4096 x 64, K = 2048,
        # 8 leaves), top-8 and gates.  Bound by reading H once.
        Wr = to_dev(wl.normal_bf16(sm["router"], (c.experts, c.K), 0.02))
        lgt = torch.empty(c.tokens, c.experts, dtype=torch.float32, device=dev)
        rid = torch.empty(c.tokens, c.topk, dtype=torch.int32, device=dev)
        rw = torch.empty(c.tokens, c.topk, dtype=torch.float32, device=dev)
        ms, ms_call, ahead = device_timed(lambda: tig.tig_moe_route(Hm, Wr, lgt, rid, rw, c.leaves), 50, 3)
        rbytes = 2.0 * c.tokens * c.K + 2.0 * c.experts * c.K + 4.0 * c.tokens * c.experts + 8.0 * c.tokens * c.topk
        moe["route"] = {"us": ms * 1e3, "us_per_python_call": ms_call * 1e3, "device_timed": ahead,
                        "shape": f"T={c.tokens} E={c.experts} top{c.topk} K={c.K} leaves={c.leaves}",
                        "roofline": hbm_line(rbytes, ms)}
        log(f"route: {ms * 1e3:.1f} us on the device, {ms_call * 1e3:.1f} us per Python call")
        del Hm, Wr, lgt, rid, rw

        # Sparse-attention indexer Top-K: 128 rows of pitch 65536, k = 2048, lengths
        # mixed (uniform in [1, 65536]) and all full.  Bound by reading the scores.
        c = wl.CONFIGS["indexer"]
        si = wl.streams(c.seed)
        sc = torch.from_numpy(wl.indexer_scores(si["scores"], c.tokens, c.N)).to(dev)
        mixed = wl.request_lengths(si["lengths"], c.tokens, 1, c.N)
        tko = torch.empty(c.tokens, c.topk, dtype=torch.int32, device=dev)
        topk = {}
        for name, lens in (("mixed", mixed), ("full", np.full(c.tokens, c.N, dtype=np.int32))):
            ln = torch.from_numpy(lens).to(dev)
            ms, ms_call, ahead = device_timed(lambda: tig.tig_topk_positions(sc, ln, tko), 50, 3)
            tbytes = 4.0 * float(lens.sum()) + 4.0 * c.tokens * (c.topk + 1)
            topk[name] = {"us": ms * 1e3, "us_per_python_call": ms_call * 1e3, "device_timed": ahead,
                          "shape": f"R={c.tokens} ld={c.N} k={c.topk} lengths={name}",
                          "roofline": hbm_line(tbytes, ms)}
            log(f"topk {name}: {ms * 1e3:.1f} us on the device, {ms_call * 1e3:.1f} us per Python call")
        del sc, tko

        c = wl.CONFIGS["large"]
        sg = wl.streams(c.seed)
        Mg = c.n_seq * c.n_pos
        Hgh, Wgh = wl.normal_bf16(sg["H"], (Mg, c.K), 1.0), wl.normal_bf16(sg["W"], (c.N, c.K), 0.02)
        igh = wl.uniform_ids(sg["ids"], Mg, c.N)
        Hg, Wg = to_dev(Hgh), to_dev(Wgh)
        ig = torch.from_numpy(igh).to(dev)
        if do_cpu:
            nr = args.cpu_rows_large
            cpu_line("large", nr, 2.0 * nr * c.K * c.N, lambda: oracle.logprob_ref(Hgh[:nr], Wgh, igh[:nr]))
        del Hgh, Wgh
        large = {}
        for name, Mr, steps in (("prefill", Mg, 3), ("decode", c.n_seq, 20)):
            Hr, ir = Hg[:Mr].contiguous(), ig[:Mr].contiguous()
            wsg = torch.empty(tig.tig_logprob_workspace_bytes(Mr, c.K, c.N, c.leaves), dtype=torch.uint8,
                              device=dev)
            lpg = torch.empty(Mr, dtype=torch.float32, device=dev)
            ms, _ = timed(lambda: tig.tig_logprob_gather(Hr, Wg, ir, lpg, None, c.leaves, wsg), steps, 1)
            line = {"tokens": Mr, "ms": ms, "tokens_per_s": Mr / (ms / 1e3),
                    "roofline": mfma_line(2.0 * Mr * c.K * c.N, ms),
                    "hbm": hbm_line(2.0 * c.K * c.N + 2.0 * Mr * c.K + 12.0 * Mr, ms)}
            large[name] = line
            log(f"large {name} M={Mr}: {ms:.3f} ms, {line['roofline']['achieved']:.0f} TFLOP/s, "
                f"{line['hbm']['achieved']:.0f} GB/s")
            del wsg
        del Hg, Wg

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
        "prefill_spread": spread,
        "tree_gemm": tree,
        "clock": clock,
        "vendor_plain_gemm_context": vendor,
        "device_copy_GBs": copy_gbs,
        "decode": decode,
        "linear": linear,
        "moe": moe,
        "fp8_lmhead_gemm": fp8_lmhead,
        "topk": topk,
        "large": large,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
