"""Benchmark: tiled causal attention over a grouped-quantized KV cache on one
MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

Headline step = the whole hot path over one batch of the block-sparse causal
prefill workload (B=1, Hq=32, Hkv=8, head_dim 128, L=131072, int8 K/V, group
32, a 128x128 KV-tile mask keeping tile 0 and the diagonal and dropping a
seeded 25% of the other causal tiles): kv_quantize of K and V (131072 tokens
each, both caches in one launch), then attn_prefill under the mask.  `value`
is the algorithmic throughput of the whole step: 4 * D * Hq * (permitted
(row, key) pairs) flops divided by the step time.  Inputs are generated once
(seeded) and resident in HBM before the timed region.

Every timed leg first runs untimed calls for at least --warmup calls and at
least two seconds (the GPU clock needs about a second to settle; shorter
warm-ups read 10-15% low).

The JSON line also carries:
  roofline      the prefill kernel's own rate on the headline workload (HIP
                events around each launch, on the stream it runs on) against
                dense fp16 MFMA peak;
  configs       one record per workload (all five): median / p10 / p90 of the
                attention call, its rate and its fraction of the roofline
                (decode: KV GB/s against HBM peak, three KV-cache copies in
                rotation; prefill: TFLOP/s against dense fp16 MFMA peak);
  cpu_baseline  the fp64 oracle on a bounded sample of the headline workload
                (all 32 query heads at sampled rows), on the host cores.
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
HBM_PEAK_GBS = 8000.0             # MI355X HBM3E, published
DECODE_COPIES = 3                 # KV-cache copies rotated by the decode timing
SETTLE_S = 2.0                    # untimed seconds before every timed leg
METRIC = "decode KV GB/s & % HBM peak; prefill TFLOP/s & % MFMA peak"
HEADLINE = "prefill_128k_sparse"
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "tiled_attention_quantized_amd", "csrc")
PREFILL_SOURCES = ["attn_prefill.hip", "device_common.h"]
DECODE_SOURCES = ["attn_decode.hip", "device_common.h"]


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


def make_caches(T, inp):
    spec, bits = inp.spec, inp.structure.head_bits
    k = T.KVCache(spec.B, spec.Hkv, spec.D, spec.cap, bits, T.LAYOUT_TOKEN)
    v = T.KVCache(spec.B, spec.Hkv, spec.D, spec.cap, bits, T.LAYOUT_CHANNEL)
    return k, v


def settle(torch, fn, min_calls, settle_s=SETTLE_S):
    """Untimed calls: at least `min_calls` of them and at least `settle_s`
    seconds."""
    t_end = time.time() + settle_s
    n = 0
    while n < min_calls or time.time() < t_end:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def timed_calls(torch, fn, reps):
    """Per-call durations (ms) from HIP events on the current stream (the one
    the library launches on), reps calls back to back."""
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for i in range(reps):
        ev[i][0].record(stream)
        fn(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in ev])


def stats(ms):
    return (float(np.median(ms)), float(np.percentile(ms, 10)), float(np.percentile(ms, 90)),
            float(np.mean(ms)))


def mask_summary(mask) -> str:
    if mask is None:
        return "dense causal"
    low = np.tril(np.ones(mask.shape, dtype=bool), -1)
    low[:, 0] = False
    elig = int(low.sum())
    dropped = int((low & (np.asarray(mask) == 0)).sum())
    return (f"128x128 KV tiles: tile 0 and the diagonal kept, {dropped} of the {elig} other "
            f"causal tiles dropped (seeded)")


def prefill_record(spec, inp, flops, ms, traffic):
    med, p10, p90, mean = stats(ms)
    tf = flops / (med * 1e-3) / 1e12
    st = inp.structure
    return {"workload": spec.name, "kind": "prefill", "B": spec.B, "Hq": spec.Hq,
            "Hkv": spec.Hkv, "head_dim": spec.D, "L": spec.context,
            "kv_bits": st.head_bits.tolist(),
            "mask": mask_summary(st.mask),
            "flops_per_call": int(flops), "calls": int(ms.size),
            "median_ms": round(med, 4), "p10_ms": round(p10, 4), "p90_ms": round(p90, 4),
            "mean_ms": round(mean, 4),
            "value": round(tf, 1), "unit": "TFLOP/s",
            "roofline": {"bound": "mfma", "achieved": round(tf, 1),
                         "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4), "traffic": traffic}}


# ---- headline: block-sparse 128K prefill step --------------------------------------

def bench_headline(args, torch, T, W, A):
    spec = W.WORKLOADS[HEADLINE]
    log(f"generating {spec.name}")
    inp = W.make_inputs(spec)
    st = inp.structure
    k, v = make_caches(T, inp)
    xk = torch.from_numpy(inp.k).cuda()
    xv = torch.from_numpy(inp.v).cuda()
    q = torch.from_numpy(inp.q).cuda()
    out = torch.empty_like(q)
    lens = torch.tensor(st.seq_lens, device="cuda")
    md = torch.from_numpy(np.ascontiguousarray(st.mask)).cuda()
    tm = T.TileMask(md, st.mask.shape[0], st.mask.shape[1])
    flops = A.prefill_flops(spec.Hq, spec.D, st.seq_lens, st.mask)
    stream = torch.cuda.current_stream()
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]

    def step(i=None):
        T.kv_quantize_pair(k, v, xk, xv, 0)
        if i is not None:
            kev[i][0].record(stream)
        T.attn_prefill(k, v, q, lens, mask=tm, out=out)
        if i is not None:
            kev[i][1].record(stream)

    log("headline warm-up")
    n = settle(torch, step, args.warmup)
    log(f"headline: {n} untimed steps, timing {args.steps}")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    kms = np.array([a.elapsed_time(b) for a, b in kev])
    log(f"headline: step {dt * 1e3:.3f} ms ({flops / dt / 1e12:.1f} TFLOP/s), kernel mean "
        f"{kms.mean():.3f} ms ({flops / (kms.mean() * 1e-3) / 1e12:.1f} TFLOP/s)")
    del xk, xv, q, out, k, v, md
    torch.cuda.empty_cache()
    return spec, inp, flops, dt, kms


# ---- sub-records -------------------------------------------------------------------

def bench_prefill_config(name, args, torch, T, W, A):
    spec = W.WORKLOADS[name]
    log(f"generating {spec.name}")
    inp = W.make_inputs(spec)
    st = inp.structure
    k, v = make_caches(T, inp)
    T.kv_quantize(k, torch.from_numpy(inp.k).cuda(), 0)
    T.kv_quantize(v, torch.from_numpy(inp.v).cuda(), 0)
    q = torch.from_numpy(inp.q).cuda()
    out = torch.empty_like(q)
    lens = torch.tensor(st.seq_lens, device="cuda")
    tm = None
    if st.mask is not None:
        tm = T.TileMask(torch.from_numpy(np.ascontiguousarray(st.mask)).cuda(),
                        st.mask.shape[0], st.mask.shape[1])
    flops = A.prefill_flops(spec.Hq, spec.D, st.seq_lens, st.mask)

    def call(i=0):
        T.attn_prefill(k, v, q, lens, mask=tm, out=out)
    settle(torch, call, args.warmup)
    ms = timed_calls(torch, call, max(args.steps, 20))
    rec = prefill_record(spec, inp, flops, ms,
                         stored_traffic(f"prefill_kernel_{name}.md", PREFILL_SOURCES))
    log(f"{name}: median {rec['median_ms']} ms, {rec['value']} TFLOP/s "
        f"({rec['roofline']['frac']} of peak)")
    del k, v, q, out, tm
    torch.cuda.empty_cache()
    return rec


def bench_decode_config(name, args, torch, T, W, A):
    """Decode workload.  Three copies of the quantised KV cache are used in
    rotation, so no copy is read again within two calls: the 256 MB Infinity
    Cache cannot serve a call from the one before (with one copy, the 201 MB of
    scales and zero-points of the long-context workload stayed resident between
    calls and a call read 4-7% faster).  The 4K workload's 2.3 MB stay
    resident in the Infinity Cache whatever the rotation: that call is bound
    by launch and latency, not by HBM."""
    spec = W.WORKLOADS[name]
    log(f"generating {spec.name}")
    inp = W.make_inputs(spec)
    st = inp.structure
    xk = torch.from_numpy(inp.k).cuda()
    xv = torch.from_numpy(inp.v).cuda()
    copies = []
    for _ in range(DECODE_COPIES):
        k, v = make_caches(T, inp)
        T.kv_quantize(k, xk, 0)
        T.kv_quantize(v, xv, 0)
        copies.append((k, v))
    del xk, xv
    q = torch.from_numpy(inp.q).cuda()
    out = torch.empty_like(q)
    lens = torch.tensor(st.seq_lens, device="cuda")
    ws = torch.empty(T.decode_workspace_bytes(copies[0][0], spec.Hq, spec.max_len),
                     dtype=torch.uint8, device="cuda")
    nbytes = A.decode_bytes(spec.B, spec.Hq, spec.D, st.seq_lens, st.head_bits)
    it = [0]

    def call(i=None):
        kk, vv = copies[it[0] % DECODE_COPIES]
        it[0] += 1
        T.attn_decode(kk, vv, q, lens, spec.max_len, out=out, workspace=ws)
    settle(torch, call, max(args.warmup, 20))
    ms = timed_calls(torch, call, max(args.steps, 100))
    med, p10, p90, mean = stats(ms)
    gbs = nbytes / (med * 1e-3) / 1e9
    traffic = (stored_traffic("decode_split_kernel_decode_128k_mixed.md", DECODE_SOURCES)
               if name == "decode_128k_mixed" else None)
    rec = {"workload": spec.name, "kind": "decode", "B": spec.B, "Hq": spec.Hq,
           "Hkv": spec.Hkv, "head_dim": spec.D, "max_context": spec.max_len,
           "total_context": int(np.sum(st.seq_lens, dtype=np.int64)),
           "kv_bits": st.head_bits.tolist(), "bytes_per_call": int(nbytes),
           "kv_copies_rotated": DECODE_COPIES, "calls": int(ms.size),
           "median_us": round(med * 1e3, 2), "p10_us": round(p10 * 1e3, 2),
           "p90_us": round(p90 * 1e3, 2), "mean_us": round(mean * 1e3, 2),
           "value": round(gbs, 1), "unit": "GB/s",
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                        "traffic": traffic}}
    if name == "decode_4k":
        rec["note"] = ("2.3 MB of KV stay in the 256 MB Infinity Cache between calls: the call "
                       "is bound by launch and latency, not by HBM")
    log(f"{name}: median {rec['median_us']} us, {rec['value']} GB/s "
        f"({rec['roofline']['frac']} of peak)")
    del copies, q, out, ws
    torch.cuda.empty_cache()
    return rec


# ---- legs beside the path (one JSON line each) ---------------------------------------

def _median_ms(torch, fn, reps, settle_s=SETTLE_S):
    """Median / p10 / p90 of `reps` calls timed with HIP events on the current
    stream, after `settle_s` seconds of untimed calls."""
    settle(torch, fn, 1, settle_s)
    ms = timed_calls(torch, lambda i: fn(), reps)
    med, p10, p90, _ = stats(ms)
    return med, p10, p90


def bench_extras(which, torch, T, W, A):
    """Timings of the paths beside the headline step, one JSON line each:
    maskgen  tile_mask_generate (skip 250 per mille) on the 128K workload's Q
             and K;
    chunk    a 512-row chunk against 8192 cached tokens (Hq 32, Hkv 8, int8),
             alone, with the two kv_append calls of the new tokens, and the
             turn's own KV-tile mask (tile_mask_generate_chunk, skip 250 per
             mille) alone and followed by the chunk under it;
    twopass  the long-context decode with the online softmax and with the
             literal two-pass softmax (same algorithmic bytes; pass 1 re-reads K);
    headbits per-KV-head sensitivity and precision assignment over the
             long-context decode workload as the calibration set."""
    if "maskgen" in which:
        spec = W.WORKLOADS["prefill_128k_sparse"]
        log(f"generating {spec.name}")
        inp = W.make_inputs(spec)
        st = inp.structure
        k, v = make_caches(T, inp)
        T.kv_quantize(k, torch.from_numpy(inp.k).cuda(), 0)
        q = torch.from_numpy(inp.q).cuda()
        lens = torch.tensor(st.seq_lens, device="cuda")
        spm = 250
        tm = T.tile_mask_generate(k, q, lens, spm)
        ws = torch.empty(T.tile_mask_workspace_bytes(k, spec.context), dtype=torch.uint8,
                         device="cuda")
        med, p10, p90 = _median_ms(
            torch, lambda: T.tile_mask_generate(k, q, lens, spm, out=tm.data, workspace=ws), 20)
        nbytes = A.maskgen_bytes(spec.B, spec.Hq, spec.Hkv, spec.D, spec.context,
                                 st.head_bits)
        gbs = nbytes / (med * 1e-3) / 1e9
        print(json.dumps({"extra": "maskgen", "workload": spec.name,
                          "skip_per_mille": spm, "ms": round(med, 4),
                          "p10_ms": round(p10, 4), "p90_ms": round(p90, 4),
                          "bytes": int(nbytes), "GB/s": round(gbs, 1),
                          "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                          "kept_tiles": int(tm.data.sum())}), flush=True)
        del ws, tm, k, v, q
        torch.cuda.empty_cache()
    if "twopass" in which:
        spec = W.WORKLOADS["decode_128k_mixed"]
        log(f"generating {spec.name}")
        inp = W.make_inputs(spec)
        k, v = make_caches(T, inp)
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
        # the turn's own KV-tile mask (skip 250 per mille), then the chunk under it
        mws = torch.empty(T.tile_mask_workspace_bytes(k, cap), dtype=torch.uint8, device="cuda")
        tm = T.tile_mask_generate_chunk(k, q, lens, cap, 250, workspace=mws)
        med3, _, _ = _median_ms(torch, lambda: T.tile_mask_generate_chunk(
            k, q, lens, cap, 250, out=tm.data, workspace=mws), 20)

        def with_turn_mask():
            T.tile_mask_generate_chunk(k, q, lens, cap, 250, out=tm.data, workspace=mws)
            T.attn_prefill_chunk(k, v, q, lens, cap, mask=tm, out=out, workspace=ws)
        med4, _, _ = _median_ms(torch, with_turn_mask, 20)
        tf = flops / (med * 1e-3) / 1e12
        print(json.dumps({"extra": "chunk", "workload": f"chunk {Lq} rows after {hist} cached",
                          "key_splits_workspace_bytes": int(nb),
                          "ms": round(med, 4), "ms_with_append": round(med2, 4),
                          "ms_turn_mask": round(med3, 4),
                          "ms_turn_mask_then_chunk": round(med4, 4),
                          "flops": int(flops), "TFLOP/s": round(tf, 1),
                          "frac_mfma": round(tf / MFMA_F16_PEAK_TFLOPS, 4)}), flush=True)


# ---- CPU baseline --------------------------------------------------------------------

def sample_rows(L: int, n: int = 4096):
    """Rows of the oracle sample: n rows evenly spaced over the sequence, its
    first and last row included (so the sample spans short and full-length
    causal rows).  The oracle
    scores blocks of 256 rows against every key, so its time grows with the
    number of row blocks: 4096 rows of the 128K workload take ~17 s on 16 host
    cores (plus ~5 s to quantise and dequantise the cache)."""
    return np.unique(np.linspace(0, L - 1, n).round().astype(np.int64))


def cpu_workers() -> int:
    """Host threads for the oracle: the CPUs this process may run on, at most
    16 (the CPU share of one GPU on the box the bench runs on)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_model() -> str:
    """The host CPU's model name: the longer of lscpu's "Model name" and
    /proc/cpuinfo's "model name" (a virtual machine's lscpu may print only the
    family)."""
    import subprocess
    names = []
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        names += [ln.split(":", 1)[1].strip() for ln in out.splitlines()
                  if ln.strip().startswith("Model name:")]
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            names += [ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")][:1]
    except OSError:
        pass
    return max(names, key=len) if names else ""


def cpu_baseline(inp, A):
    """The oracle as it stands on a bounded sample of the headline workload:
    quantise and dequantise the whole K and V caches (all 8 KV heads), then
    the attention of every query head at `sample_rows` rows, process pool
    over heads.  Throughput = the sample's algorithmic flops / wall time."""
    from oracle import attention as oa
    from oracle import quant as oq
    spec, st = inp.spec, inp.structure
    workers = cpu_workers()
    rows = sample_rows(spec.context)
    heads = [(0, h) for h in range(spec.Hq)]
    t0 = time.perf_counter()
    kh = np.zeros((1, spec.Hkv, spec.cap, spec.D))
    vh = np.zeros((1, spec.Hkv, spec.cap, spec.D))
    for g in range(spec.Hkv):
        kh[0, g] = oq.dequantize(*oq.quantize(inp.k[0, g], int(st.head_bits[g])))
        vh[0, g] = oq.dequantize(*oq.quantize(inp.v[0, g], int(st.head_bits[g])))
    t1 = time.perf_counter()
    oa.prefill(inp.q, kh, vh, st.seq_lens, mask=st.mask, rows=rows, heads=heads,
               workers=workers)
    dt = time.perf_counter() - t0
    # permitted (row, key) pairs of the sampled rows
    pairs = 0
    for i in rows:
        qt = i // 128
        pairs += int(st.mask[qt, :qt].sum()) * 128
        if st.mask[qt, qt]:
            pairs += i - qt * 128 + 1
    flops = 4 * spec.D * spec.Hq * pairs
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": workers,
            "kind": "oracle", "seconds": round(dt, 2),
            "seconds_quantise": round(t1 - t0, 2),
            "flops": int(flops), "host_cpus": os.cpu_count(), "cpu": cpu_model(),
            "sample": (f"{spec.name}: quantise + dequantise all of K and V (8 KV heads x "
                       f"{spec.context} tokens), then attention of all {spec.Hq} query heads at "
                       f"{rows.size} rows spread over the sequence ({int(pairs)} permitted "
                       f"(row, key) pairs per head under the mask); fp64 NumPy, process pool of "
                       f"{workers} workers, 1 BLAS thread each")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="timed headline steps")
    ap.add_argument("--warmup", type=int, default=5,
                    help="untimed calls first, at least; every timed leg also runs "
                         "untimed calls for at least two seconds")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    ap.add_argument("--no-configs", action="store_true",
                    help="headline step only (no per-workload records)")
    ap.add_argument("--only", choices=["headline", "prefill_8k", "prefill_128k_sparse",
                                       "decode_4k", "decode_ragged", "decode_128k_mixed",
                                       "maskgen", "chunk", "twopass", "headbits", "extras"],
                    default=None,
                    help="one leg alone (a workload record, the headline step, or the legs "
                         "beside the path: maskgen / chunk / twopass / headbits, all of them "
                         "with extras), printed as its own JSON line")
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

    if args.only in ("maskgen", "chunk", "twopass", "headbits", "extras"):
        which = (["maskgen", "chunk", "twopass", "headbits"] if args.only == "extras"
                 else [args.only])
        bench_extras(which, torch, T, W, A)
        return
    if args.only in ("prefill_8k", "prefill_128k_sparse"):
        print(json.dumps({"config": bench_prefill_config(args.only, args, torch, T, W, A)}),
              flush=True)
        return
    if args.only in ("decode_4k", "decode_ragged", "decode_128k_mixed"):
        print(json.dumps({"config": bench_decode_config(args.only, args, torch, T, W, A)}),
              flush=True)
        return

    spec, inp, flops, dt, kms = bench_headline(args, torch, T, W, A)
    kern_ms = float(kms.mean())
    kern_tf = flops / (kern_ms * 1e-3) / 1e12
    traffic = stored_traffic(f"prefill_kernel_{HEADLINE}.md", PREFILL_SOURCES)
    configs = None
    if args.only is None and not args.no_configs:
        configs = {}
        for name in ("decode_4k", "prefill_8k", "decode_ragged", "decode_128k_mixed"):
            fn = bench_prefill_config if name.startswith("prefill") else bench_decode_config
            configs[name] = fn(name, args, torch, T, W, A)
        configs[HEADLINE] = prefill_record(spec, inp, flops, kms, traffic)
        configs[HEADLINE]["note"] = "the headline step's own prefill launches"
    cpu = None
    if args.only is None and not args.no_cpu:
        log("timing the oracle on a sample")
        cpu = cpu_baseline(inp, A)
        log(f"oracle: {cpu['seconds']} s, {cpu['value']} TFLOP/s on {cpu['cores']} workers")
    st = inp.structure
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
                   "mask": mask_summary(st.mask),
                   "step": "kv_quantize_pair(K, V) + attn_prefill"},
        "roofline": {"bound": "mfma", "achieved": round(kern_tf, 2),
                     "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(kern_tf / MFMA_F16_PEAK_TFLOPS, 4),
                     "traffic": traffic,
                     "kernel": "prefill_kernel (int8 K and V, Hq/Hkv = 4)",
                     "kernel_ms": round(kern_ms, 4), "kernel_launches": int(kms.size),
                     "flops_per_launch": int(flops)},
        "cpu_baseline": cpu,
        "configs": configs,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
