"""GPU parity at the five workloads' full sizes, in the launch configuration
the bench times, against the fp64 oracle (max-abs <= 2e-3 on every compared
element):

* decode_4k, prefill_8k, decode_ragged, decode_128k_mixed: every output
  element of the call;
* prefill_128k_sparse (under its seeded 25% tile mask): every query head at
  every row of the first two and the last 128-row query tiles, plus rows
  spread over the sequence;
* every workload's quantised K and V caches, dequantised: bit for bit.

The oracle side is computed slab by slab (one batch entry and KV head, or one
query head) in a forked process pool, so host memory stays bounded: each job
quantises and dequantises its own K/V slab with the oracle's quantiser and
evaluates the plain-definition attention on it.  The worst error of each
workload is printed."""
from __future__ import annotations

import multiprocessing as mp
import os
import time
from concurrent.futures import ProcessPoolExecutor

import numpy as np
import pytest
import torch

import tiled_attention_quantized_amd as T
import workloads as W
from oracle import attention as oa
from oracle import quant as oq
from tests.gpu_util import TOL, require_gpu, note, gpu_cache, lens_tensor

pytestmark = pytest.mark.gpu

_G = {}


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _pool_map(fn, jobs):
    """Map over a forked pool; the workers read the inputs from _G."""
    ctx = mp.get_context("fork")
    with ProcessPoolExecutor(max_workers=min(_workers(), len(jobs)), mp_context=ctx,
                             initializer=_one_thread) as ex:
        return list(ex.map(fn, jobs, chunksize=1))


def _one_thread():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _slab(x, b, g, n):
    bits = int(_G["inp"].structure.head_bits[g])
    return oq.dequantize(*oq.quantize(x[b, g, :n], bits))


def _decode_job(bg):
    """Oracle decode of the r query heads of KV head g, batch entry b."""
    b, g = bg
    inp = _G["inp"]
    r = inp.spec.r
    n = int(inp.structure.seq_lens[b])
    kh, vh = _slab(inp.k, b, g, n), _slab(inp.v, b, g, n)
    q = inp.q[b:b + 1, g * r:(g + 1) * r]
    return oa.decode(q, kh[None, None], vh[None, None], [n])[0]      # [r][D]


def _prefill_job(bh):
    """Oracle prefill of query head h, batch entry b, at the rows in _G."""
    b, h = bh
    inp = _G["inp"]
    g = h // inp.spec.r
    n = int(inp.structure.seq_lens[b])
    kh, vh = _slab(inp.k, b, g, n), _slab(inp.v, b, g, n)
    return oa.prefill(inp.q[b:b + 1, h:h + 1], kh[None, None], vh[None, None], [n],
                      mask=inp.structure.mask, rows=_G["rows"])[0, 0]  # [R][D]


def _gpu_caches(inp):
    spec, st = inp.spec, inp.structure
    kc = gpu_cache(inp.k, st.head_bits, T.LAYOUT_TOKEN, spec.cap)
    vc = gpu_cache(inp.v, st.head_bits, T.LAYOUT_CHANNEL, spec.cap)
    return kc, vc


@pytest.mark.parametrize("name", ["decode_4k", "decode_ragged", "decode_128k_mixed"])
def test_decode_full_size_every_output(name):
    require_gpu()
    spec = W.WORKLOADS[name]
    note(f"{name}: generating inputs")
    inp = W.make_inputs(spec)
    st = inp.structure
    note(f"{name}: GPU call (B={spec.B}, Hq={spec.Hq}, Hkv={spec.Hkv}, bits={st.head_bits.tolist()})")
    kc, vc = _gpu_caches(inp)
    q = torch.from_numpy(inp.q).cuda()
    out = T.attn_decode(kc, vc, q, lens_tensor(st.seq_lens), spec.max_len)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    del kc, vc, q, out
    torch.cuda.empty_cache()
    note(f"{name}: oracle over {spec.B * spec.Hkv} (batch, KV head) slabs")
    _G.clear()
    _G["inp"] = inp
    jobs = [(b, g) for b in range(spec.B) for g in range(spec.Hkv)]
    t0 = time.perf_counter()
    res = _pool_map(_decode_job, jobs)
    note(f"{name}: oracle {time.perf_counter() - t0:.1f} s on {min(_workers(), len(jobs))} "
         f"host processes")
    r = spec.r
    err = 0.0
    for (b, g), want in zip(jobs, res):
        e = float(np.abs(got[b, g * r:(g + 1) * r] - want).max())
        err = max(err, e)
        assert e <= TOL, (name, b, g, e)
    note(f"{name}: every output compared, max-abs {err:.3e}")
    _G.clear()


def _prefill_rows(name, L):
    if name == "prefill_8k":
        return np.arange(L)
    rng = np.random.default_rng(7)
    rows = set(range(0, 256)) | set(range(L - 128, L))
    rows |= set(int(x) for x in rng.integers(256, L - 128, 64))
    rows |= {127, 128, 129, L // 2, L // 2 + 1}
    return np.array(sorted(rows))


@pytest.mark.parametrize("name", ["prefill_8k", "prefill_128k_sparse"])
def test_prefill_full_size(name):
    require_gpu()
    spec = W.WORKLOADS[name]
    note(f"{name}: generating inputs")
    inp = W.make_inputs(spec)
    st = inp.structure
    note(f"{name}: GPU call (L={spec.context}, mask={'none' if st.mask is None else 'seeded'})")
    kc, vc = _gpu_caches(inp)
    q = torch.from_numpy(inp.q).cuda()
    tm = None
    if st.mask is not None:
        tm = T.TileMask(torch.from_numpy(np.ascontiguousarray(st.mask)).cuda(),
                        st.mask.shape[0], st.mask.shape[1])
    out = T.attn_prefill(kc, vc, q, lens_tensor(st.seq_lens), mask=tm)
    torch.cuda.synchronize()
    rows = _prefill_rows(name, spec.context)
    got = out[:, :, torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
    del kc, vc, q, out, tm
    torch.cuda.empty_cache()
    note(f"{name}: oracle over {spec.B * spec.Hq} query heads x {rows.size} rows")
    _G.clear()
    _G["inp"] = inp
    _G["rows"] = rows
    jobs = [(b, h) for b in range(spec.B) for h in range(spec.Hq)]
    t0 = time.perf_counter()
    res = _pool_map(_prefill_job, jobs)
    note(f"{name}: oracle {time.perf_counter() - t0:.1f} s on {min(_workers(), len(jobs))} "
         f"host processes")
    err, worst = 0.0, None
    for (b, h), want in zip(jobs, res):
        d = np.abs(got[b, h] - want)
        e = float(d.max())
        if e > err:
            i, c = np.unravel_index(int(d.argmax()), d.shape)
            err, worst = e, (b, h, int(rows[i]), int(c), float(want[i, c]))
        assert e <= TOL, (name, b, h, e)
    note(f"{name}: {len(jobs)} heads x {rows.size} rows compared, max-abs {err:.3e} "
         f"at (b, h, row, channel, value) = {worst}")
    _G.clear()


def _dequant_job(args):
    """Oracle quantise + dequantise of one (b, g) slab's token range, compared
    bit for bit (fp32) with the GPU's dequantised values in _G."""
    b, g, start, count, which = args
    inp = _G["inp"]
    x = (inp.k if which == "k" else inp.v)[b, g, start:start + count]
    bits = int(inp.structure.head_bits[g])
    want = oq.dequantize(*oq.quantize(x, bits)).astype(np.float32)
    got = _G["got"][b, g]
    same = np.array_equal(got.view(np.uint32), want.view(np.uint32))
    return same, int(np.count_nonzero(got.view(np.uint32) != want.view(np.uint32)))


@pytest.mark.parametrize("name", ["decode_4k", "prefill_8k", "decode_ragged",
                                  "decode_128k_mixed", "prefill_128k_sparse"])
def test_quantize_full_size_bit_exact(name):
    """kv_quantize of the workload's whole K and V (every token slot of the
    capacity) dequantises, through kv_dequantize, to exactly the oracle's
    fp32 values (quantise then dequantise, slab by slab)."""
    require_gpu()
    spec = W.WORKLOADS[name]
    note(f"{name}: generating inputs")
    inp = W.make_inputs(spec)
    st = inp.structure
    kc, vc = _gpu_caches(inp)
    S = inp.k.shape[2]
    chunk = 8192
    _G.clear()
    _G["inp"] = inp
    for which, cache in (("k", kc), ("v", vc)):
        for start in range(0, S, chunk):
            count = min(chunk, S - start)
            note(f"{name}: {which} tokens {start}..{start + count - 1}")
            o32, _ = T.kv_dequantize(cache, start, count)
            torch.cuda.synchronize()
            _G["got"] = o32.cpu().numpy()
            del o32
            jobs = [(b, g, start, count, which) for b in range(spec.B) for g in range(spec.Hkv)]
            res = _pool_map(_dequant_job, jobs)
            bad = [(j, n) for j, (ok, n) in zip(jobs, res) if not ok]
            assert not bad, (name, which, bad[:4])
    note(f"{name}: K and V of {spec.B} x {spec.Hkv} slabs x {S} tokens dequantise bit for bit")
    _G.clear()
