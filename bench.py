"""Benchmark: tiled causal attention over a grouped-quantized KV cache on one
MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

One step = the whole hot path over one batch of the causal-prefill workload
(B=1, Hq=32, Hkv=8, head_dim 128, L=8192, int8 K/V, group 32): kv_quantize of
K and V (8192 tokens each, both caches in one launch), then attn_prefill.  `value` is the algorithmic
prefill throughput of the whole step: 4 * D * Hq * L(L+1)/2 flops divided by the
step time.  Inputs are generated once (seeded) and resident in HBM before the
timed region.

The JSON line also carries:
  roofline      the prefill kernel's own rate (HIP events around the launch, on
                the stream it runs on) against dense fp16 MFMA peak;
  decode        the long-context decode workload (B=8, Hq=32, Hkv=8, 131072
                tokens, 2 int8 + 6 int4 KV heads): KV GB/s against HBM peak;
  cpu_baseline  the fp64 oracle on the same prefill workload (host cores).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_F16_PEAK_TFLOPS = 2500.0     # MI355X dense fp16 MFMA, published
DECODE_COPIES = 3          # KV-cache copies rotated by the decode timing
HBM_PEAK_GBS = 8000.0             # MI355X HBM3E, published
METRIC = "decode KV GB/s & % HBM peak; prefill TFLOP/s & % MFMA peak"
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "tiled_attention_quantized_amd", "csrc")


def source_hash(*names) -> str:
    """sha256 (first 16 hex digits) of the kernel sources a counter run used."""
    import hashlib
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(summary: str, sources) -> "float | None":
    """HBM bytes per launch recorded in a profiles/ summary (FETCH_SIZE plus
    WRITE_SIZE, scaled by the copy-kernel factor), or None when the summary
    is missing or was taken on different kernel sources."""
    path = os.path.join(PROFILES, summary)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and line.startswith("- "):
                k, v = line[2:].split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("source_sha256_16") != source_hash(*sources):
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def make_caches(T, inp, torch):
    spec, bits = inp.spec, inp.structure.head_bits
    k = T.KVCache(spec.B, spec.Hkv, spec.D, spec.cap, bits, T.LAYOUT_TOKEN)
    v = T.KVCache(spec.B, spec.Hkv, spec.D, spec.cap, bits, T.LAYOUT_CHANNEL)
    return k, v


def bench_prefill(args, torch, T, W, A):
    spec = W.WORKLOADS["prefill_8k"]
    log(f"generating {spec.name}")
    inp = W.make_inputs(spec)
    k, v = make_caches(T, inp, torch)
    xk = torch.from_numpy(inp.k).cuda()
    xv = torch.from_numpy(inp.v).cuda()
    q = torch.from_numpy(inp.q).cuda()
    out = torch.empty_like(q)
    lens = torch.tensor(inp.structure.seq_lens, device="cuda")
    flops = A.prefill_flops(spec.Hq, spec.D, inp.structure.seq_lens)
    stream = torch.cuda.current_stream()

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]

    def step(i=None):
        T.kv_quantize_pair(k, v, xk, xv, 0)
        if i is not None:
            ev[i][0].record(stream)
        T.attn_prefill(k, v, q, lens, out=out)
        if i is not None:
            ev[i][1].record(stream)

    log("warmup")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    kern_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    tflops_step = flops / dt / 1e12
    tflops_kern = flops / (kern_ms * 1e-3) / 1e12
    log(f"prefill: step {dt * 1e3:.3f} ms ({tflops_step:.1f} TFLOP/s), kernel {kern_ms:.3f} ms "
        f"({tflops_kern:.1f} TFLOP/s)")
    return spec, inp, flops, dt, kern_ms


def bench_decode(args, torch, T, W, A):
    """Long-context decode.  Three copies of the quantised KV cache are used in
    rotation, so no copy is read again within two calls: the 256 MB Infinity
    Cache cannot serve any part of a call from the one before (with one copy,
    the scales and zero-points, 201 MB, stayed resident between calls and the
    call read 4-7% faster)."""
    spec = W.WORKLOADS["decode_128k_mixed"]
    log(f"generating {spec.name}")
    inp = W.make_inputs(spec)
    xk = torch.from_numpy(inp.k).cuda()
    xv = torch.from_numpy(inp.v).cuda()
    copies = []
    for _ in range(DECODE_COPIES):
        k, v = make_caches(T, inp, torch)
        T.kv_quantize(k, xk, 0)
        T.kv_quantize(v, xv, 0)
        copies.append((k, v))
    del xk, xv
    q = torch.from_numpy(inp.q).cuda()
    out = torch.empty_like(q)
    lens = torch.tensor(inp.structure.seq_lens, device="cuda")
    ws = torch.empty(T.decode_workspace_bytes(copies[0][0], spec.Hq, spec.max_len),
                     dtype=torch.uint8, device="cuda")
    nbytes = A.decode_bytes(spec.B, spec.Hq, spec.D, inp.structure.seq_lens,
                            inp.structure.head_bits)
    stream = torch.cuda.current_stream()

    def call(i):
        k, v = copies[i % DECODE_COPIES]
        T.attn_decode(k, v, q, lens, spec.max_len, out=out, workspace=ws)

    for i in range(max(args.warmup, 20)):        # let the clocks settle
        call(i)
    torch.cuda.synchronize()
    iters = max(args.steps, 10)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(iters)]
    for i in range(iters):
        ev[i][0].record(stream)
        call(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    med = float(np.median(ms))
    gbs = nbytes / (med * 1e-3) / 1e9
    log(f"decode: median {med * 1e3:.1f} us, p10 {np.percentile(ms, 10) * 1e3:.1f}, "
        f"p90 {np.percentile(ms, 90) * 1e3:.1f}; {gbs:.0f} GB/s")
    del copies, q, out, ws
    torch.cuda.empty_cache()
    return {"workload": spec.name, "B": spec.B, "Hq": spec.Hq, "Hkv": spec.Hkv,
            "head_dim": spec.D, "context": spec.context,
            "kv_bits": inp.structure.head_bits.tolist(),
            "bytes_per_call": int(nbytes), "median_us": round(med * 1e3, 2),
            "p10_us": round(float(np.percentile(ms, 10)) * 1e3, 2),
            "p90_us": round(float(np.percentile(ms, 90)) * 1e3, 2),
            "kv_copies_rotated": DECODE_COPIES,
            "value": round(gbs, 1), "unit": "GB/s",
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": stored_traffic("decode_split_kernel_decode_128k_mixed.md",
                                                   ["attn_decode.hip", "device_common.h"])}}


def _median_ms(torch, fn, reps, settle_s=2.0):
    """Median / p10 / p90 of `reps` calls timed with HIP events on the current
    stream, after `settle_s` seconds of untimed calls."""
    t_end = time.time() + settle_s
    while time.time() < t_end:
        fn()
        torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    return (float(np.median(ts)), float(np.percentile(ts, 10)), float(np.percentile(ts, 90)))


def bench_extras(which, torch, T, W, A):
    """Timings of the paths beside the headline step, one JSON line each:
    sparse   attn_prefill on the 128K workload with its seeded 25% tile mask;
    maskgen  tile_mask_generate (skip 250 per mille) on the same Q and K;
    chunk    a 512-row chunk against 8192 cached tokens (Hq 32, Hkv 8, int8),
             alone and with the two kv_append calls of the new tokens;
    twopass  the long-context decode with the online softmax and with the
             literal two-pass softmax (same algorithmic bytes; pass 1 re-reads K);
    headbits per-KV-head sensitivity and precision assignment over the
             long-context decode workload as the calibration set."""
    if {"sparse", "maskgen"} & set(which):
        spec = W.WORKLOADS["prefill_128k_sparse"]
        log(f"generating {spec.name}")
        inp = W.make_inputs(spec)
        st = inp.structure
        k, v = make_caches(T, inp, torch)
        T.kv_quantize(k, torch.from_numpy(inp.k).cuda(), 0)
        T.kv_quantize(v, torch.from_numpy(inp.v).cuda(), 0)
        q = torch.from_numpy(inp.q).cuda()
        lens = torch.tensor(st.seq_lens, device="cuda")
        if "sparse" in which:
            md = torch.from_numpy(np.ascontiguousarray(st.mask)).cuda()
            tm = T.TileMask(md, st.mask.shape[0], st.mask.shape[1])
            out = torch.empty_like(q)
            flops = A.prefill_flops(spec.Hq, spec.D, st.seq_lens, st.mask)
            med, p10, p90 = _median_ms(torch, lambda: T.attn_prefill(k, v, q, lens, mask=tm,
                                                                     out=out), 5)
            tf = flops / (med * 1e-3) / 1e12
            print(json.dumps({"extra": "sparse", "workload": spec.name, "ms": round(med, 3),
                              "p10_ms": round(p10, 3), "p90_ms": round(p90, 3),
                              "flops": int(flops), "TFLOP/s": round(tf, 1),
                              "frac_mfma": round(tf / MFMA_F16_PEAK_TFLOPS, 4)}), flush=True)
            del out
        if "maskgen" in which:
            spm = 250
            tm = T.tile_mask_generate(k, q, lens, spm)
            ws = torch.empty(T.tile_mask_workspace_bytes(k, spec.context), dtype=torch.uint8,
                             device="cuda")
            med, p10, p90 = _median_ms(
                torch, lambda: T.tile_mask_generate(k, q, lens, spm, out=tm.data, workspace=ws),
                20)
            nbytes = A.maskgen_bytes(spec.B, spec.Hq, spec.Hkv, spec.D, spec.context,
                                     st.head_bits)
            gbs = nbytes / (med * 1e-3) / 1e9
            print(json.dumps({"extra": "maskgen", "workload": spec.name,
                              "skip_per_mille": spm, "ms": round(med, 4),
                              "p10_ms": round(p10, 4), "p90_ms": round(p90, 4),
                              "bytes": int(nbytes), "GB/s": round(gbs, 1),
                              "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                              "kept_tiles": int(tm.data.sum())}), flush=True)
            del ws, tm
        del k, v, q
        torch.cuda.empty_cache()
    if "twopass" in which:
        spec = W.WORKLOADS["decode_128k_mixed"]
        log(f"generating {spec.name}")
        inp = W.make_inputs(spec)
        k, v = make_caches(T, inp, torch)
        T.kv_quantize(k, torch.from_numpy(inp.k).cuda(), 0)
        T.kv_quantize(v, torch.from_numpy(inp.v).cuda(), 0)
        q = torch.from_numpy(inp.q).cuda()
        out = torch.empty_like(q)
        lens = torch.tensor(inp.structure.seq_lens, device="cuda")
        ws = torch.empty(T.decode_workspace_bytes(k, spec.Hq, spec.max_len), dtype=torch.uint8,
                         device="cuda")
        nbytes = A.decode_bytes(spec.B, spec.Hq, spec.D, inp.structure.seq_lens,
                                inp.structure.head_bits)
        res = {}
        for name, tp in (("online", False), ("two_pass", True)):
            med, p10, p90 = _median_ms(torch, lambda: T.attn_decode(
                k, v, q, lens, spec.max_len, out=out, workspace=ws, two_pass=tp), 50)
            res[name] = {"us": round(med * 1e3, 1), "GB/s": round(nbytes / (med * 1e-3) / 1e9, 1)}
        print(json.dumps({"extra": "twopass", "workload": spec.name, "bytes": int(nbytes), **res,
                          "two_pass_over_online": round(res["two_pass"]["us"] /
                                                        res["online"]["us"], 3)}), flush=True)
        del k, v, q, out, ws
        torch.cuda.empty_cache()
    if "headbits" in which:
        spec = W.WORKLOADS["decode_128k_mixed"]
        log(f"generating {spec.name}")
        inp = W.make_inputs(spec)
        kx = torch.from_numpy(inp.k).cuda()
        vx = torch.from_numpy(inp.v).cuda()
        q = torch.from_numpy(inp.q).cuda()
        lens = torch.tensor(inp.structure.seq_lens, device="cuda")
        ws = torch.empty(int(T.lib().taq_head_sensitivity_workspace_bytes(
            spec.B, spec.Hkv, spec.Hq, spec.cap)), dtype=torch.uint8, device="cuda")
        n_high = 2
        scores, bits = T.head_sensitivity(kx, vx, q, lens, n_high, workspace=ws)
        med, p10, p90 = _median_ms(torch, lambda: T.head_sensitivity(kx, vx, q, lens, n_high,
                                                                     workspace=ws), 10)
        fp16_bytes = 2 * kx.numel() * 2
        print(json.dumps({"extra": "headbits", "workload": spec.name, "n_high": n_high,
                          "ms": round(med, 3), "p10_ms": round(p10, 3), "p90_ms": round(p90, 3),
                          "fp16_kv_bytes": int(fp16_bytes),
                          "GB/s_of_fp16_kv": round(fp16_bytes / (med * 1e-3) / 1e9, 1),
                          "bits": bits.cpu().tolist()}), flush=True)
        del kx, vx, q, ws
        torch.cuda.empty_cache()
    if "chunk" in which:
        B, Hq, Hkv, Lq, hist = 1, 32, 8, 512, 8192
        cap = hist + Lq
        kv = W.make_inputs(W.small("prefill", B=B, Hq=Hq, Hkv=Hkv, L=cap, bits=8, seed=901))
        qn = W.make_inputs(W.small("prefill", B=B, Hq=Hq, Hkv=Hkv, L=Lq, bits=8, seed=902)).q
        k = T.KVCache(B, Hkv, 128, cap, kv.structure.head_bits, T.LAYOUT_TOKEN)
        v = T.KVCache(B, Hkv, 128, cap, kv.structure.head_bits, T.LAYOUT_CHANNEL)
        T.kv_quantize(k, torch.from_numpy(kv.k).cuda(), 0)
        T.kv_quantize(v, torch.from_numpy(kv.v).cuda(), 0)
        q = torch.from_numpy(qn).cuda()
        out = torch.empty_like(q)
        lens = torch.tensor([cap], dtype=torch.int32, device="cuda")
        starts = torch.tensor([hist], dtype=torch.int32, device="cuda")
        xk = torch.from_numpy(np.ascontiguousarray(kv.k[:, :, hist:])).cuda()
        xv = torch.from_numpy(np.ascontiguousarray(kv.v[:, :, hist:])).cuda()
        flops = 4 * 128 * Hq * sum(hist + i + 1 for i in range(Lq))
        nb = T.prefill_chunk_workspace_bytes(k, Hq, Lq, cap)
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
        med, _, _ = _median_ms(torch, lambda: T.attn_prefill_chunk(k, v, q, lens, cap, out=out,
                                                                   workspace=ws), 20)

        def with_append():
            T.kv_append(k, xk, starts)
            T.kv_append(v, xv, starts)
            T.attn_prefill_chunk(k, v, q, lens, cap, out=out, workspace=ws)
        med2, _, _ = _median_ms(torch, with_append, 20)
        tf = flops / (med * 1e-3) / 1e12
        print(json.dumps({"extra": "chunk", "workload": f"chunk {Lq} rows after {hist} cached",
                          "key_splits_workspace_bytes": int(nb),
                          "ms": round(med, 4), "ms_with_append": round(med2, 4),
                          "flops": int(flops), "TFLOP/s": round(tf, 1),
                          "frac_mfma": round(tf / MFMA_F16_PEAK_TFLOPS, 4)}), flush=True)


def cpu_baseline(inp, A, W):
    """The oracle as it stands on the prefill workload (all 32 query heads, all
    rows), process pool over heads."""
    from oracle import attention as oa
    from oracle import quant as oq
    spec, st = inp.spec, inp.structure
    workers = oa.default_workers()
    heads = [(0, h) for h in range(spec.Hq)]
    t0 = time.perf_counter()
    kh = np.zeros((1, spec.Hkv, spec.cap, spec.D))
    vh = np.zeros((1, spec.Hkv, spec.cap, spec.D))
    for g in range(spec.Hkv):
        kh[0, g] = oq.dequantize(*oq.quantize(inp.k[0, g], int(st.head_bits[g])))
        vh[0, g] = oq.dequantize(*oq.quantize(inp.v[0, g], int(st.head_bits[g])))
    oa.prefill(inp.q, kh, vh, st.seq_lens, heads=heads, workers=workers)
    dt = time.perf_counter() - t0
    flops = A.prefill_flops(len(heads), spec.D, st.seq_lens)
    cpu = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": workers,
            "kind": "oracle", "seconds": round(dt, 2), "cpu": cpu,
            "sample": "prefill_8k in full (32 query heads x 8192 rows, quantisation included); "
                      f"fp64 NumPy, process pool of {workers} workers, 1 BLAS thread each"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=2000,
                    help="untimed steps first (the GPU clock takes about a second to settle)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode workload")
    ap.add_argument("--only", choices=["prefill", "decode", "sparse", "maskgen", "chunk",
                                       "twopass", "headbits", "extras"], default=None,
                    help="one leg alone; sparse / maskgen / chunk / twopass / headbits (or "
                         "all of them: extras) print their own JSON lines")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a plain 1 GiB device copy (for HBM counter calibration) and exit")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this library runs on one GPU; only --gpus 1 is measured "
              "(sharding is described in the design notes, not run).", file=sys.stderr)
        sys.exit(2)

    import torch
    import tiled_attention_quantized_amd as T
    import workloads as W
    from workloads import accounting as A

    torch.cuda.set_device(0)
    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": src.numel()}), flush=True)
        return
    T.device_check(0)

    if args.only in ("sparse", "maskgen", "chunk", "twopass", "headbits", "extras"):
        which = (["sparse", "maskgen", "chunk", "twopass", "headbits"] if args.only == "extras"
                 else [args.only])
        bench_extras(which, torch, T, W, A)
        return

    if args.only == "decode":
        d = bench_decode(args, torch, T, W, A)
        print(json.dumps({"decode": d}), flush=True)
        return

    spec, inp, flops, dt, kern_ms = bench_prefill(args, torch, T, W, A)
    torch.cuda.empty_cache()
    dec = None
    if not args.no_decode and args.only is None:
        dec = bench_decode(args, torch, T, W, A)
    cpu = None
    if not args.no_cpu and args.only is None:
        log("timing the oracle on a sample")
        cpu = cpu_baseline(inp, A, W)
        log(f"oracle: {cpu['seconds']} s, {cpu['value']} TFLOP/s on {cpu['cores']} workers")
    kern_tf = flops / (kern_ms * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": round(flops / dt / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dt * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": spec.name, "B": spec.B, "Hq": spec.Hq, "Hkv": spec.Hkv,
                   "head_dim": spec.D, "L": spec.context, "kv_bits": 8, "group": 32,
                   "mask": "dense causal",
                   "step": "kv_quantize_pair(K, V) + attn_prefill"},
        "roofline": {"bound": "mfma", "achieved": round(kern_tf, 2),
                     "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(kern_tf / MFMA_F16_PEAK_TFLOPS, 4),
                     "traffic": stored_traffic("prefill_kernel_prefill_8k.md",
                                               ["attn_prefill.hip", "device_common.h"]),
                     "kernel": "prefill_kernel<4, true, true>", "kernel_ms": round(kern_ms, 4),
                     "flops_per_launch": int(flops)},
        "cpu_baseline": cpu,
        "decode": dec,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
