"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, sizes buffers, and rejects bad arguments with the documented
status before touching the device (fake, never dereferenced pointers)."""
import ctypes
import os
import re

import numpy as np
import pytest

import tiled_attention_quantized_amd as T

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, UNSUPPORTED, MISALIGNED, WS_SMALL, HIP = range(6)
FAKE = 0x10000  # aligned, never dereferenced


def header_functions():
    with open(os.path.join(ROOT, "include", "taq.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(taq_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L = T.lib()
    names = header_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(T.EXPORTS)
    assert L.taq_abi_version() == 1


def cache(B=2, H=2, D=128, cap=256, bits=(8, 4), layout=0, group=32, codes=FAKE,
          scales=FAKE, zeros=FAKE):
    b = np.asarray(bits, dtype=np.uint8)
    d = T._Cache(B, H, D, group, cap, layout, b.ctypes.data, codes, scales, zeros)
    d._keep = b
    return d


def status_of(rc):
    return rc, T.lib().taq_last_error().decode()


def test_sizes():
    L = T.lib()
    assert L.taq_kv_codes_bytes(ctypes.byref(cache())) == 2 * 256 * (128 + 64)
    assert L.taq_kv_meta_count(ctypes.byref(cache())) == 2 * 2 * 256 * 4
    assert L.taq_kv_codes_bytes(ctypes.byref(cache(bits=(3, 4)))) == 0
    # decode workspace: partials B * Hq * nchunk * (D + 2) floats, then the
    # chunk plan (a count, a pad word and B * Hkv * nchunk (unit, chunk) pairs);
    # here B = 1 and Hkv = 2 give 128-token chunks (nchunk = 32)
    k = cache(B=1, H=2, cap=4096, bits=(8, 8))
    ws = L.taq_attn_decode_workspace_bytes(ctypes.byref(k), 8, 4096)
    assert ws == 1 * 8 * 32 * 130 * 4 + (2 + 2 * 1 * 2 * 32) * 4


@pytest.mark.parametrize("kw,want", [
    (dict(bits=(3, 4)), UNSUPPORTED),
    (dict(group=16), UNSUPPORTED),
    (dict(D=48), UNSUPPORTED),
    (dict(D=1056), UNSUPPORTED),
    (dict(cap=200), INVALID),
    (dict(H=0, bits=()), INVALID),
    (dict(layout=7), INVALID),
    (dict(codes=0), INVALID),
    (dict(scales=FAKE + 4), MISALIGNED),
])
def test_quantize_rejects(kw, want):
    d = cache(**kw)
    rc, msg = status_of(T.lib().taq_kv_quantize(ctypes.byref(d), FAKE, 0, 4, None))
    assert rc == want, msg
    assert msg


def test_quantize_range_and_pointer_checks():
    L = T.lib()
    d = cache()
    assert L.taq_kv_quantize(ctypes.byref(d), FAKE, 250, 7, None) == INVALID
    assert L.taq_kv_quantize(ctypes.byref(d), FAKE, -1, 2, None) == INVALID
    assert L.taq_kv_quantize(ctypes.byref(d), 0, 0, 2, None) == INVALID
    assert L.taq_kv_quantize(ctypes.byref(d), FAKE + 2, 0, 2, None) == MISALIGNED
    assert L.taq_kv_dequantize(ctypes.byref(d), 0, 2, None, None, None) == INVALID
    assert L.taq_kv_dequantize(ctypes.byref(d), 0, 2, FAKE + 8, None, None) == MISALIGNED


def test_quantize_pair_rejects():
    L = T.lib()
    k = cache(layout=0)
    v = cache(layout=1)

    def call(k=k, v=v, xk=FAKE, xv=FAKE, start=0, count=4):
        return status_of(L.taq_kv_quantize_pair(ctypes.byref(k), ctypes.byref(v), xk, xv, start,
                                                count, None))
    assert call(v=cache(D=64, layout=1))[0] == INVALID           # head_dims differ
    assert call(xk=0)[0] == INVALID
    assert call(xv=0)[0] == INVALID
    assert call(xv=FAKE + 2)[0] == MISALIGNED
    assert call(start=250, count=7)[0] == INVALID                # past the capacity
    assert call(v=cache(cap=128, layout=1), start=120, count=16)[0] == INVALID
    assert call(k=cache(group=16))[0] == UNSUPPORTED             # either cache is checked
    assert call(v=cache(bits=(8, 5), layout=1))[0] != 0


def decode_call(k=None, v=None, hq=8, max_len=200, mask=None, ws_bytes=1 << 30,
                q=FAKE, o=FAKE, lens=FAKE, ws=FAKE, scale=0.0):
    k = k or cache(B=1, H=2, cap=256, bits=(8, 8), layout=0)
    v = v or cache(B=1, H=2, cap=256, bits=(8, 8), layout=1)
    m = ctypes.byref(mask) if mask is not None else None
    return status_of(T.lib().taq_attn_decode(ctypes.byref(k), ctypes.byref(v), q, hq, lens,
                                             max_len, m, scale, o, ws, ws_bytes, None))


def decode_two_pass_call(k=None, v=None, hq=8, max_len=200, mask=None, ws_bytes=1 << 30,
                         q=FAKE, o=FAKE, lens=FAKE, ws=FAKE, scale=0.0):
    k = k or cache(B=1, H=2, cap=256, bits=(8, 8), layout=0)
    v = v or cache(B=1, H=2, cap=256, bits=(8, 8), layout=1)
    m = ctypes.byref(mask) if mask is not None else None
    return status_of(T.lib().taq_attn_decode_two_pass(ctypes.byref(k), ctypes.byref(v), q, hq,
                                                      lens, max_len, m, scale, o, ws, ws_bytes,
                                                      None))


def decode_noalloc_call(k=None, v=None, hq=8, max_len=200, mask=None, q=FAKE, o=FAKE,
                        lens=FAKE, scale=0.0):
    k = k or cache(B=1, H=2, cap=256, bits=(8, 8), layout=0)
    v = v or cache(B=1, H=2, cap=256, bits=(8, 8), layout=1)
    m = ctypes.byref(mask) if mask is not None else None
    return status_of(T.lib().taq_attn_decode_noalloc(ctypes.byref(k), ctypes.byref(v), q, hq,
                                                     lens, max_len, m, scale, o, None))


def prefill_call(k=None, v=None, hq=8, max_len=200, mask=None, q=FAKE, o=FAKE, lens=FAKE,
                 scale=0.0):
    k = k or cache(B=1, H=2, cap=256, bits=(8, 8), layout=0)
    v = v or cache(B=1, H=2, cap=256, bits=(8, 8), layout=1)
    m = ctypes.byref(mask) if mask is not None else None
    return status_of(T.lib().taq_attn_prefill(ctypes.byref(k), ctypes.byref(v), q, hq, lens,
                                              max_len, m, scale, o, None))


@pytest.mark.parametrize("call", [decode_call, decode_two_pass_call, decode_noalloc_call,
                                  prefill_call])
def test_attention_rejects(call):
    assert call(hq=7)[0] == INVALID                      # Hq % Hkv != 0
    assert call(hq=6)[0] == UNSUPPORTED                  # r = 3
    assert call(hq=32)[0] == UNSUPPORTED                 # r = 16
    assert call(max_len=300)[0] == INVALID               # beyond capacity
    assert call(max_len=-1)[0] == INVALID
    assert call(q=0)[0] == INVALID
    assert call(o=FAKE + 2)[0] == MISALIGNED
    assert call(scale=float("nan"))[0] == INVALID
    assert call(scale=-0.5)[0] == UNSUPPORTED
    kd = cache(B=1, H=2, cap=256, bits=(8, 8), layout=1)
    assert call(k=kd)[0] == UNSUPPORTED                  # K must be token layout
    vd = cache(B=1, H=2, cap=256, bits=(8, 8), layout=0)
    assert call(v=vd)[0] == UNSUPPORTED                  # V must be channel layout
    k64 = cache(B=1, H=2, D=64, cap=256, bits=(8, 8), layout=0)
    assert call(k=k64)[0] == UNSUPPORTED                 # attention needs D = 128
    v2 = cache(B=1, H=2, cap=384, bits=(8, 8), layout=1)
    assert call(v=v2)[0] == INVALID                      # geometry mismatch
    kbig = cache(B=1, H=2, cap=1 << 24, bits=(8, 8), layout=0)
    assert call(k=kbig, max_len=200)[0] == UNSUPPORTED   # slab offsets beyond 32 bits
    bad_tile = T._Mask(FAKE, 64, 2, 2, 0, 0)
    assert call(mask=bad_tile)[0] == UNSUPPORTED
    small = T._Mask(FAKE, 128, 2, 1, 0, 0)
    assert call(mask=small)[0] == INVALID
    nodata = T._Mask(0, 128, 2, 2, 0, 0)
    assert call(mask=nodata)[0] == INVALID


@pytest.mark.parametrize("call", [decode_call, decode_two_pass_call, decode_noalloc_call])
def test_decode_mask_must_have_one_query_tile(call):
    """A decode mask is one row of KV tiles: any other n_q_tiles is an argument
    error, not a mask read with the wrong row stride."""
    for nq in (2, 3):
        rc, msg = call(mask=T._Mask(FAKE, 128, nq, 2, 0, 0))
        assert rc == INVALID and "n_q_tiles" in msg, (nq, msg)
    assert call(mask=T._Mask(FAKE, 128, 0, 2, 0, 0))[0] == INVALID
    if not os.path.exists("/dev/kfd"):
        rc, msg = call(mask=T._Mask(FAKE, 128, 1, 2, 0, 0))
        assert rc == HIP, msg
        # the same two-row mask is a valid prefill mask
        rc, msg = prefill_call(mask=T._Mask(FAKE, 128, 2, 2, 0, 0))
        assert rc == HIP, msg


def test_decode_workspace_too_small():
    assert decode_call(ws_bytes=16)[0] == WS_SMALL
    assert decode_call(ws=0)[0] == WS_SMALL
    assert decode_two_pass_call(ws_bytes=16)[0] == WS_SMALL


def test_decode_noalloc_rejects_shapes_beyond_its_scratch():
    """The allocation-free decode refuses, before touching the device, shapes
    whose split partials exceed its fixed scratch; shapes that fit get past
    the check."""
    k = cache(B=64, H=8, cap=131072, bits=(4,) * 8, layout=0)
    v = cache(B=64, H=8, cap=131072, bits=(4,) * 8, layout=1)
    need = T.lib().taq_attn_decode_workspace_bytes(ctypes.byref(k), 64, 131072)
    assert need > 16 * 1024 * 1024
    rc, msg = decode_noalloc_call(k=k, v=v, hq=64, max_len=131072)
    assert rc == WS_SMALL and "scratch" in msg, msg
    k = cache(B=8, H=8, cap=131072, bits=(4,) * 8, layout=0)
    v = cache(B=8, H=8, cap=131072, bits=(4,) * 8, layout=1)
    assert T.lib().taq_attn_decode_workspace_bytes(ctypes.byref(k), 32, 131072) <= 16 << 20
    if not os.path.exists("/dev/kfd"):
        # no GPU: shapes that fit get past the check and stop at the device query
        rc, msg = decode_noalloc_call(k=k, v=v, hq=32, max_len=131072)
        assert rc == HIP, msg


def test_valid_arguments_reach_the_device_check():
    # No GPU in this container: valid arguments get past validation and stop at
    # the device query with a HIP status, never at a fallback.
    if os.path.exists("/dev/kfd"):
        pytest.skip("a GPU device node is present")
    rc, msg = decode_call()
    assert rc == HIP, msg
    rc, msg = decode_two_pass_call()
    assert rc == HIP, msg
    rc, msg = decode_noalloc_call()
    assert rc == HIP, msg
    rc, msg = prefill_call()
    assert rc == HIP, msg


def test_arch_override_rejects_other_gpus():
    L = T.lib()
    try:
        L.taq_debug_set_arch_override(b"gfx942:sramecc+:xnack-")
        rc, msg = status_of(L.taq_device_check(0))
        assert rc == UNSUPPORTED and "gfx950" in msg
        L.taq_debug_set_arch_override(b"gfx950:sramecc+:xnack-")
        assert L.taq_device_check(0) == OK
    finally:
        L.taq_debug_set_arch_override(None)


def chunk_call(k=None, v=None, hq=8, q_len=64, max_len=200, mask=None, q=FAKE, o=FAKE,
               lens=FAKE, scale=0.0, ws=None, ws_bytes=0):
    k = k or cache(B=1, H=2, cap=256, bits=(8, 8), layout=0)
    v = v or cache(B=1, H=2, cap=256, bits=(8, 8), layout=1)
    m = ctypes.byref(mask) if mask is not None else None
    return status_of(T.lib().taq_attn_prefill_chunk(ctypes.byref(k), ctypes.byref(v), q, hq,
                                                    q_len, lens, max_len, m, scale, o, ws,
                                                    ws_bytes, None))


def test_chunk_prefill_rejects():
    # the checks shared with taq_attn_prefill
    assert chunk_call(hq=7)[0] == INVALID
    assert chunk_call(hq=6)[0] == UNSUPPORTED
    assert chunk_call(max_len=300)[0] == INVALID
    assert chunk_call(q=0)[0] == INVALID
    assert chunk_call(lens=FAKE + 4)[0] == MISALIGNED
    assert chunk_call(scale=-1.0)[0] == UNSUPPORTED
    assert chunk_call(mask=T._Mask(FAKE, 128, 2, 1, 0, 0))[0] == INVALID
    # its own: q_len within [0, max_seq_len]
    assert chunk_call(q_len=201)[0] == INVALID
    assert chunk_call(q_len=-1)[0] == INVALID
    # the optional key-range split workspace
    k = cache(B=1, H=2, cap=8704, bits=(8, 8), layout=0)
    v = cache(B=1, H=2, cap=8704, bits=(8, 8), layout=1)
    nb = T.lib().taq_attn_prefill_chunk_workspace_bytes(ctypes.byref(k), 8, 512, 8704)
    assert nb > 0 and nb % (132 * 4) == 0             # [splits][B][Hq][q_len][D + 4] floats
    # a whole-sequence-sized chunk over 8 KV heads has workgroups enough: no split
    k8 = cache(B=1, H=8, cap=8704, bits=(8,) * 8, layout=0)
    assert T.lib().taq_attn_prefill_chunk_workspace_bytes(ctypes.byref(k8), 32, 8704, 8704) == 0
    assert chunk_call(k=k, v=v, q_len=512, max_len=8704, ws=FAKE, ws_bytes=nb - 1)[0] == WS_SMALL
    assert chunk_call(k=k, v=v, q_len=512, max_len=8704, ws=FAKE + 8, ws_bytes=nb)[0] == MISALIGNED
    if not os.path.exists("/dev/kfd"):
        assert chunk_call(q_len=0)[0] == HIP          # valid: stops at the device query
        assert chunk_call(q_len=200)[0] == HIP
        assert chunk_call(k=k, v=v, q_len=512, max_len=8704, ws=FAKE, ws_bytes=nb)[0] == HIP


def test_kv_append_rejects():
    L = T.lib()
    d = cache()
    assert L.taq_kv_append(ctypes.byref(d), 0, FAKE, 4, None) == INVALID
    assert L.taq_kv_append(ctypes.byref(d), FAKE, 0, 4, None) == INVALID
    assert L.taq_kv_append(ctypes.byref(d), FAKE, FAKE + 4, 4, None) == MISALIGNED
    assert L.taq_kv_append(ctypes.byref(d), FAKE, FAKE, -1, None) == INVALID
    assert L.taq_kv_append(ctypes.byref(d), FAKE, FAKE, 257, None) == INVALID
    assert L.taq_kv_append(ctypes.byref(cache(bits=(3, 4))), FAKE, FAKE, 4, None) == UNSUPPORTED
    if not os.path.exists("/dev/kfd"):
        assert L.taq_kv_append(ctypes.byref(d), FAKE, FAKE, 256, None) == HIP


def maskgen_call(k=None, hq=8, max_len=1000, spm=250, q=FAKE, lens=FAKE, out=FAKE, ws=FAKE,
                 ws_bytes=1 << 30):
    k = k or cache(B=2, H=2, cap=1024, bits=(8, 4), layout=0)
    return status_of(T.lib().taq_tile_mask_generate(ctypes.byref(k), q, hq, lens, max_len, spm,
                                                    out, ws, ws_bytes, None))


def test_tile_mask_workspace_bytes():
    L = T.lib()
    k = cache(B=2, H=2, cap=1024, bits=(8, 4), layout=0)
    # query sums and key means (B * Hkv * nt * D doubles each) and scores
    # (B * Hkv * nt * nt doubles), nt = ceil(1000 / 128) = 8
    assert L.taq_tile_mask_workspace_bytes(ctypes.byref(k), 1000) == 2 * 2 * 8 * (256 + 8) * 8
    assert L.taq_tile_mask_workspace_bytes(ctypes.byref(k), 0) == 0
    assert L.taq_tile_mask_workspace_bytes(ctypes.byref(k), 2000) == 0        # beyond capacity
    kd = cache(B=2, H=2, cap=1024, bits=(8, 4), layout=1)
    assert L.taq_tile_mask_workspace_bytes(ctypes.byref(kd), 1000) == 0       # channel layout


def test_tile_mask_rejects():
    assert maskgen_call(hq=7)[0] == INVALID
    assert maskgen_call(hq=0)[0] == INVALID
    assert maskgen_call(max_len=1025)[0] == INVALID
    assert maskgen_call(max_len=-1)[0] == INVALID
    assert maskgen_call(spm=-1)[0] == INVALID
    assert maskgen_call(spm=1001)[0] == INVALID
    assert maskgen_call(q=0)[0] == INVALID
    assert maskgen_call(lens=0)[0] == INVALID
    assert maskgen_call(out=0)[0] == INVALID
    assert maskgen_call(q=FAKE + 2)[0] == MISALIGNED
    assert maskgen_call(lens=FAKE + 4)[0] == MISALIGNED
    assert maskgen_call(ws=0)[0] == WS_SMALL
    assert maskgen_call(ws_bytes=2 * 2 * 8 * (256 + 8) * 8 - 1)[0] == WS_SMALL
    assert maskgen_call(ws=FAKE + 8)[0] == MISALIGNED
    assert maskgen_call(k=cache(B=2, H=2, cap=1024, bits=(8, 4), layout=1))[0] == UNSUPPORTED
    assert maskgen_call(k=cache(B=2, H=2, D=64, cap=1024, bits=(8, 4)))[0] == UNSUPPORTED
    # at most 2048 tiles per side (262144 positions)
    big = cache(B=1, H=1, cap=262272, bits=(8,))
    assert maskgen_call(k=big, hq=1, max_len=262272)[0] == UNSUPPORTED
    if not os.path.exists("/dev/kfd"):
        assert maskgen_call(k=big, hq=1, max_len=262144)[0] == HIP   # valid: device query
        assert maskgen_call(max_len=0)[0] == HIP


def maskgen_chunk_call(k=None, hq=8, q_len=300, max_len=1000, spm=250, q=FAKE, lens=FAKE,
                       out=FAKE, ws=FAKE, ws_bytes=1 << 30):
    k = k or cache(B=2, H=2, cap=1024, bits=(8, 4), layout=0)
    return status_of(T.lib().taq_tile_mask_generate_chunk(ctypes.byref(k), q, hq, q_len, lens,
                                                          max_len, spm, out, ws, ws_bytes, None))


def test_tile_mask_chunk_rejects():
    """The per-turn generator validates like the whole-prompt one, plus the
    turn's length."""
    assert maskgen_chunk_call(q_len=-1)[0] == INVALID
    assert maskgen_chunk_call(q_len=1001)[0] == INVALID            # beyond max_seq_len
    assert maskgen_chunk_call(hq=7)[0] == INVALID
    assert maskgen_chunk_call(max_len=1025)[0] == INVALID
    assert maskgen_chunk_call(spm=1001)[0] == INVALID
    assert maskgen_chunk_call(q=0)[0] == INVALID
    assert maskgen_chunk_call(q=FAKE + 2)[0] == MISALIGNED
    assert maskgen_chunk_call(ws=0)[0] == WS_SMALL
    assert maskgen_chunk_call(k=cache(B=2, H=2, cap=1024, bits=(8, 4), layout=1))[0] == UNSUPPORTED
    assert maskgen_call(q=0)[0] == INVALID                          # a whole prompt needs q
    if not os.path.exists("/dev/kfd"):
        for ql in (0, 1, 300, 1000):
            rc, msg = maskgen_chunk_call(q_len=ql)
            assert rc == HIP, msg
        rc, msg = maskgen_chunk_call(q_len=0, q=0)                 # an empty turn reads no q
        assert rc == HIP, msg


def sens_call(B=2, hkv=4, hq=8, max_len=300, n_high=1, k=FAKE, v=FAKE, q=FAKE, lens=FAKE,
              scores=FAKE, bits=FAKE, ws=FAKE, ws_bytes=1 << 40, scale=0.0):
    return status_of(T.lib().taq_head_sensitivity(k, v, q, B, hkv, hq, lens, max_len, scale,
                                                  n_high, scores, bits, ws, ws_bytes, None))


def test_head_sensitivity_workspace_bytes():
    L = T.lib()
    # cap 384: int8 codes 2*4*384*128 per cache, int4 half; meta 2*4*384*4 (x2 scales, x1 zeros)
    nb = L.taq_head_sensitivity_workspace_bytes(2, 4, 8, 300)
    c8, meta = 2 * 4 * 384 * 128, 2 * 4 * 384 * 4
    assert nb >= 2 * c8 + 2 * (c8 // 2) + 4 * 3 * meta + 2 * 2 * 8 * 128 * 2
    assert L.taq_head_sensitivity_workspace_bytes(0, 4, 8, 300) == 0
    assert L.taq_head_sensitivity_workspace_bytes(2, 65, 65, 300) == 0


def test_head_sensitivity_rejects():
    assert sens_call(B=0)[0] == INVALID
    assert sens_call(hkv=0)[0] == INVALID
    assert sens_call(hq=6)[0] == INVALID
    assert sens_call(hq=12)[0] == UNSUPPORTED            # r = 3
    assert sens_call(max_len=-1)[0] == INVALID
    assert sens_call(n_high=-1)[0] == INVALID
    assert sens_call(n_high=5)[0] == INVALID
    assert sens_call(k=0)[0] == INVALID
    assert sens_call(bits=0)[0] == INVALID
    assert sens_call(q=FAKE + 2)[0] == MISALIGNED
    assert sens_call(scores=FAKE + 4)[0] == MISALIGNED
    assert sens_call(scale=-1.0)[0] == UNSUPPORTED
    assert sens_call(ws_bytes=16)[0] == WS_SMALL
    assert sens_call(ws=0)[0] == WS_SMALL
    if not os.path.exists("/dev/kfd"):
        assert sens_call()[0] == HIP                      # valid: stops at the device query


def test_c_consumer_of_the_header(tmp_path):
    """The header compiles as C99 and a plain C program linked against the
    library gets the documented sizes and statuses (no GPU needed)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    here = os.path.dirname(os.path.abspath(__file__))
    src = os.path.join(here, "c_abi", "abi_check.c")
    libdir = os.path.dirname(T.LIB_PATH)
    exe = str(tmp_path / "abi_check")
    hip_lib = "/opt/rocm/lib"
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
           src, "-o", exe, "-L", libdir, "-l:libtaq.so", "-Wl,--allow-shlib-undefined",
           f"-Wl,-rpath,{libdir}", f"-Wl,-rpath,{hip_lib}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
