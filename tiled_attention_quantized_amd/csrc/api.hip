// C ABI of the library: argument validation, cache geometry and launches.
// Every entry point checks what the host can see before anything is enqueued
// and never substitutes another code path ("分块稀疏注意力与KV Cache量化：长文本
// 推理显存优化实践", xdnf.cn, section 4.3, describes what a silent fallback costs).
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "taq_internal.h"

namespace {

thread_local std::string g_err;
std::mutex g_arch_mu;
std::string g_arch_override;
bool g_arch_override_set = false;

taq_status fail(taq_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

taq_status hip_fail(hipError_t e, const char* what) {
  return fail(TAQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

taq_status check_cache(const taq_kv_cache* c, const char* name, int need_layout,
                       bool attention) {
  if (!c) return fail(TAQ_ERR_INVALID_ARGUMENT, "%s: null cache descriptor", name);
  if (c->batch < 1) return fail(TAQ_ERR_INVALID_ARGUMENT, "%s: batch must be >= 1", name);
  if (c->num_kv_heads < 1 || c->num_kv_heads > TAQ_MAX_KV_HEADS)
    return fail(TAQ_ERR_INVALID_ARGUMENT, "%s: num_kv_heads must be in [1, %d]", name,
                TAQ_MAX_KV_HEADS);
  if (c->group_size != TAQ_GROUP)
    return fail(TAQ_ERR_UNSUPPORTED, "%s: group_size must be 32", name);
  if (c->head_dim <= 0 || c->head_dim % TAQ_GROUP || c->head_dim > 1024)
    return fail(TAQ_ERR_UNSUPPORTED, "%s: head_dim must be a multiple of 32 in [32, 1024]",
                name);
  if (attention && c->head_dim != 128)
    return fail(TAQ_ERR_UNSUPPORTED, "%s: attention kernels need head_dim 128", name);
  // the attention kernels address one (batch, head) slab with 32-bit offsets
  if (attention && (int64_t)c->capacity * c->head_dim >= ((int64_t)1 << 31))
    return fail(TAQ_ERR_UNSUPPORTED, "%s: capacity %d too large for the attention kernels "
                "(capacity * head_dim must stay below 2^31)", name, c->capacity);
  if (c->capacity <= 0 || c->capacity % TAQ_TILE)
    return fail(TAQ_ERR_INVALID_ARGUMENT, "%s: capacity must be a positive multiple of 128",
                name);
  if (c->layout != TAQ_LAYOUT_TOKEN && c->layout != TAQ_LAYOUT_CHANNEL)
    return fail(TAQ_ERR_INVALID_ARGUMENT, "%s: unknown layout %d", name, c->layout);
  if (need_layout >= 0 && c->layout != need_layout)
    return fail(TAQ_ERR_UNSUPPORTED, "%s: layout must be %s", name,
                need_layout == TAQ_LAYOUT_TOKEN ? "TAQ_LAYOUT_TOKEN" : "TAQ_LAYOUT_CHANNEL");
  if (!c->bits) return fail(TAQ_ERR_INVALID_ARGUMENT, "%s: null bits array", name);
  for (int h = 0; h < c->num_kv_heads; ++h)
    if (c->bits[h] != 4 && c->bits[h] != 8)
      return fail(TAQ_ERR_UNSUPPORTED, "%s: bits[%d] = %d (must be 4 or 8)", name, h,
                  (int)c->bits[h]);
  if (!c->codes || !c->scales || !c->zeros)
    return fail(TAQ_ERR_INVALID_ARGUMENT, "%s: null device buffer", name);
  if (!aligned16(c->codes) || !aligned16(c->scales) || !aligned16(c->zeros))
    return fail(TAQ_ERR_MISALIGNED, "%s: device buffers must be 16-byte aligned", name);
  return TAQ_OK;
}

taq::CacheGeom geom_of(const taq_kv_cache* c) {
  taq::CacheGeom g;
  std::memset(&g, 0, sizeof(g));
  g.codes = c->codes;
  g.scales = c->scales;
  g.zeros = c->zeros;
  int64_t acc = 0;
  for (int h = 0; h < c->num_kv_heads; ++h) {
    g.hoff[h] = acc;
    acc += (int64_t)c->capacity * c->head_dim * c->bits[h] / 8;
    if (c->bits[h] == 8) g.is8 |= 1ull << h;
  }
  g.bstride = acc;
  g.B = c->batch;
  g.H = c->num_kv_heads;
  g.D = c->head_dim;
  g.cap = c->capacity;
  g.layout = c->layout;
  return g;
}

taq_status device_ok() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  return taq_device_check(dev);
}

taq_status check_mask(const taq_tile_mask* m, int need_q, int need_k) {
  if (!m) return TAQ_OK;
  if (!m->data) return fail(TAQ_ERR_INVALID_ARGUMENT, "mask: null data");
  if (m->tile != TAQ_TILE) return fail(TAQ_ERR_UNSUPPORTED, "mask: tile must be 128");
  if (m->n_q_tiles < need_q || m->n_k_tiles < need_k)
    return fail(TAQ_ERR_INVALID_ARGUMENT,
                "mask: needs at least %d x %d tiles, got %d x %d", need_q, need_k,
                m->n_q_tiles, m->n_k_tiles);
  if (m->stride_b < 0 || m->stride_h < 0)
    return fail(TAQ_ERR_INVALID_ARGUMENT, "mask: negative stride");
  return TAQ_OK;
}

taq_status check_pair(const taq_kv_cache* k, const taq_kv_cache* v, int32_t hq,
                      int32_t max_len) {
  taq_status st = check_cache(k, "k_cache", TAQ_LAYOUT_TOKEN, true);
  if (st) return st;
  st = check_cache(v, "v_cache", TAQ_LAYOUT_CHANNEL, true);
  if (st) return st;
  if (k->batch != v->batch || k->num_kv_heads != v->num_kv_heads ||
      k->head_dim != v->head_dim || k->capacity != v->capacity)
    return fail(TAQ_ERR_INVALID_ARGUMENT, "k_cache and v_cache geometry differ");
  if (hq < 1 || hq % k->num_kv_heads)
    return fail(TAQ_ERR_INVALID_ARGUMENT, "num_q_heads (%d) must be a positive multiple of "
                "num_kv_heads (%d)", hq, k->num_kv_heads);
  const int r = hq / k->num_kv_heads;
  if (r != 1 && r != 2 && r != 4 && r != 8)
    return fail(TAQ_ERR_UNSUPPORTED, "num_q_heads / num_kv_heads = %d (supported: 1, 2, 4, 8)", r);
  if (max_len < 0 || max_len > k->capacity)
    return fail(TAQ_ERR_INVALID_ARGUMENT, "max_seq_len %d outside [0, capacity %d]", max_len,
                k->capacity);
  return TAQ_OK;
}

float scale_log2_of(float softmax_scale, int D) {
  const float s = softmax_scale == 0.f ? 1.f / std::sqrt((float)D) : softmax_scale;
  return s * 1.4426950408889634f;
}

}  // namespace

extern "C" {

const char* taq_last_error(void) { return g_err.c_str(); }

int taq_abi_version(void) { return TAQ_ABI_VERSION; }

void taq_debug_set_arch_override(const char* arch) {
  std::lock_guard<std::mutex> lk(g_arch_mu);
  g_arch_override_set = arch != nullptr;
  g_arch_override = arch ? arch : "";
}

taq_status taq_device_check(int device) {
  std::string arch;
  {
    std::lock_guard<std::mutex> lk(g_arch_mu);
    if (g_arch_override_set) arch = g_arch_override;
  }
  if (arch.empty()) {
    hipDeviceProp_t p;
    hipError_t e = hipGetDeviceProperties(&p, device);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    arch = p.gcnArchName;
  }
  if (arch.compare(0, 6, "gfx950") != 0)
    return fail(TAQ_ERR_UNSUPPORTED, "device %d is %s; this library is built for gfx950 only",
                device, arch.c_str());
  return TAQ_OK;
}

size_t taq_kv_codes_bytes(const taq_kv_cache* c) {
  if (check_cache(c, "cache", -1, false)) return 0;
  size_t per = 0;
  for (int h = 0; h < c->num_kv_heads; ++h)
    per += (size_t)c->capacity * c->head_dim * c->bits[h] / 8;
  return per * (size_t)c->batch;
}

size_t taq_kv_meta_count(const taq_kv_cache* c) {
  if (check_cache(c, "cache", -1, false)) return 0;
  return (size_t)c->batch * c->num_kv_heads * c->capacity * (c->head_dim / TAQ_GROUP);
}

taq_status taq_kv_quantize(const taq_kv_cache* c, const void* x, int32_t start,
                           int32_t count, void* stream) {
  taq_status st = check_cache(c, "cache", -1, false);
  if (st) return st;
  if (!x) return fail(TAQ_ERR_INVALID_ARGUMENT, "x: null");
  if (!aligned16(x)) return fail(TAQ_ERR_MISALIGNED, "x must be 16-byte aligned");
  if (start < 0 || count < 0 || (int64_t)start + count > c->capacity)
    return fail(TAQ_ERR_INVALID_ARGUMENT, "tokens [%d, %d + %d) outside capacity %d", start,
                start, count, c->capacity);
  st = device_ok();
  if (st) return st;
  taq::QuantArgs a;
  std::memset(&a, 0, sizeof(a));
  a.c = geom_of(c);
  a.x = static_cast<const uint16_t*>(x);
  a.start = start;
  a.count = count;
  hipError_t e = taq::launch_kv_quantize(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TAQ_OK : hip_fail(e, "kv_quantize launch");
}

taq_status taq_kv_quantize_pair(const taq_kv_cache* k, const taq_kv_cache* v, const void* xk,
                                const void* xv, int32_t start, int32_t count, void* stream) {
  taq_status st = check_cache(k, "k_cache", -1, false);
  if (st) return st;
  st = check_cache(v, "v_cache", -1, false);
  if (st) return st;
  if (k->head_dim != v->head_dim)
    return fail(TAQ_ERR_INVALID_ARGUMENT, "k and v head_dim differ (%d, %d)", k->head_dim,
                v->head_dim);
  if (!xk || !xv) return fail(TAQ_ERR_INVALID_ARGUMENT, "xk or xv: null");
  if (!aligned16(xk) || !aligned16(xv))
    return fail(TAQ_ERR_MISALIGNED, "xk and xv must be 16-byte aligned");
  const int32_t cap = k->capacity < v->capacity ? k->capacity : v->capacity;
  if (start < 0 || count < 0 || (int64_t)start + count > cap)
    return fail(TAQ_ERR_INVALID_ARGUMENT, "tokens [%d, %d + %d) outside capacity %d", start,
                start, count, cap);
  st = device_ok();
  if (st) return st;
  taq::QuantArgs a0, a1;
  std::memset(&a0, 0, sizeof(a0));
  std::memset(&a1, 0, sizeof(a1));
  a0.c = geom_of(k);
  a0.x = static_cast<const uint16_t*>(xk);
  a1.c = geom_of(v);
  a1.x = static_cast<const uint16_t*>(xv);
  a0.start = a1.start = start;
  a0.count = a1.count = count;
  hipError_t e = taq::launch_kv_quantize_pair(a0, a1, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TAQ_OK : hip_fail(e, "kv_quantize_pair launch");
}

taq_status taq_kv_dequantize(const taq_kv_cache* c, int32_t start, int32_t count,
                             float* out32, void* out16, void* stream) {
  taq_status st = check_cache(c, "cache", -1, false);
  if (st) return st;
  if (!out32 && !out16) return fail(TAQ_ERR_INVALID_ARGUMENT, "both outputs are null");
  if ((out32 && !aligned16(out32)) || (out16 && !aligned16(out16)))
    return fail(TAQ_ERR_MISALIGNED, "outputs must be 16-byte aligned");
  if (start < 0 || count < 0 || (int64_t)start + count > c->capacity)
    return fail(TAQ_ERR_INVALID_ARGUMENT, "tokens [%d, %d + %d) outside capacity %d", start,
                start, count, c->capacity);
  st = device_ok();
  if (st) return st;
  taq::QuantArgs a;
  std::memset(&a, 0, sizeof(a));
  a.c = geom_of(c);
  a.start = start;
  a.count = count;
  a.out32 = out32;
  a.out16 = static_cast<uint16_t*>(out16);
  hipError_t e = taq::launch_kv_dequantize(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TAQ_OK : hip_fail(e, "kv_dequantize launch");
}

size_t taq_attn_decode_workspace_bytes(const taq_kv_cache* k, int32_t hq, int32_t max_len) {
  if (!k || k->batch < 1 || k->num_kv_heads < 1 || hq < 1 || max_len < 0) return 0;
  return taq::decode_workspace_bytes(k->batch, k->num_kv_heads, hq, max_len);
}

}  // extern "C"

namespace {

// Host-visible arguments of a decode call other than the workspace.
taq_status decode_validate(const taq_kv_cache* k, const taq_kv_cache* v, const void* q,
                           int32_t hq, const int32_t* lens, int32_t max_len,
                           const taq_tile_mask* mask, float softmax_scale, void* o) {
  taq_status st = check_pair(k, v, hq, max_len);
  if (st) return st;
  if (!q || !o || !lens) return fail(TAQ_ERR_INVALID_ARGUMENT, "null q, o or seq_lens");
  if (!aligned16(q) || !aligned16(o) || !aligned16(lens))
    return fail(TAQ_ERR_MISALIGNED, "q, o and seq_lens must be 16-byte aligned");
  if (!std::isfinite(softmax_scale))
    return fail(TAQ_ERR_INVALID_ARGUMENT, "softmax_scale must be finite");
  if (softmax_scale < 0.f)
    return fail(TAQ_ERR_UNSUPPORTED, "softmax_scale must be >= 0 (0 selects 1/sqrt(head_dim))");
  st = check_mask(mask, 1, (max_len + TAQ_TILE - 1) / TAQ_TILE);
  if (st) return st;
  if (mask && mask->n_q_tiles != 1)
    return fail(TAQ_ERR_INVALID_ARGUMENT, "mask: decode takes n_q_tiles == 1, got %d",
                mask->n_q_tiles);
  return TAQ_OK;
}

// Shared body of taq_attn_decode (online softmax), taq_attn_decode_two_pass
// and taq_attn_decode_noalloc.
taq_status decode_common(const taq_kv_cache* k, const taq_kv_cache* v, const void* q,
                         int32_t hq, const int32_t* lens, int32_t max_len,
                         const taq_tile_mask* mask, float softmax_scale, void* o, void* ws,
                         size_t ws_bytes, void* stream, bool two_pass) {
  taq_status st = decode_validate(k, v, q, hq, lens, max_len, mask, softmax_scale, o);
  if (st) return st;
  const size_t need = taq_attn_decode_workspace_bytes(k, hq, max_len);
  if (!ws || ws_bytes < need)
    return fail(TAQ_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", need,
                ws ? ws_bytes : (size_t)0);
  if (!aligned16(ws)) return fail(TAQ_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  st = device_ok();
  if (st) return st;
  taq::DecodeArgs a;
  std::memset(&a, 0, sizeof(a));
  a.k = geom_of(k);
  a.v = geom_of(v);
  a.q = static_cast<const uint16_t*>(q);
  a.o = static_cast<uint16_t*>(o);
  a.lens = lens;
  if (mask) {
    a.mask = mask->data;
    a.mask_sb = mask->stride_b;
    a.mask_sh = mask->stride_h;
    a.mask_nk = mask->n_k_tiles;
  }
  a.ws = static_cast<float*>(ws);
  a.Hq = hq;
  a.r = hq / k->num_kv_heads;
  a.max_len = max_len;
  a.chunk = taq::decode_chunk_tokens(k->batch, k->num_kv_heads, max_len);
  a.nchunk = max_len > 0 ? (max_len + a.chunk - 1) / a.chunk : 1;
  a.scale_log2 = scale_log2_of(softmax_scale, 128);
  hipError_t e = taq::launch_attn_decode(a, static_cast<hipStream_t>(stream), two_pass);
  return e == hipSuccess ? TAQ_OK : hip_fail(e, "attn_decode launch");
}

}  // namespace

extern "C" {

taq_status taq_attn_decode(const taq_kv_cache* k, const taq_kv_cache* v, const void* q,
                           int32_t hq, const int32_t* lens, int32_t max_len,
                           const taq_tile_mask* mask, float softmax_scale, void* o,
                           void* ws, size_t ws_bytes, void* stream) {
  return decode_common(k, v, q, hq, lens, max_len, mask, softmax_scale, o, ws, ws_bytes, stream,
                       false);
}

taq_status taq_attn_decode_two_pass(const taq_kv_cache* k, const taq_kv_cache* v,
                                    const void* q, int32_t hq, const int32_t* lens,
                                    int32_t max_len, const taq_tile_mask* mask,
                                    float softmax_scale, void* o, void* ws, size_t ws_bytes,
                                    void* stream) {
  return decode_common(k, v, q, hq, lens, max_len, mask, softmax_scale, o, ws, ws_bytes, stream,
                       true);
}

}  // extern "C"

namespace {

// Scratch of taq_attn_decode_noalloc: the decode split partials, in a
// file-scope device array that every GPU the library runs on holds until the
// process ends.  In host code `scratch` names a host-side stand-in, not the
// device memory: its device address on each GPU comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// only that address is ever handed to a kernel.  Nothing in it has to start
// at zero (each call writes every partial it reads), and calls that overlap
// on one GPU share it and race.
static __device__ __align__(256) unsigned char scratch[TAQ_DECODE_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call on each device).
taq_status scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(TAQ_ERR_UNSUPPORTED, "device %d: the no-allocation scratch covers devices 0..%d",
                dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(TAQ_ERR_HIP, "hipGetSymbolAddress(scratch) gave a null address");
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return TAQ_OK;
}

}  // namespace

extern "C" {

taq_status taq_attn_decode_noalloc(const taq_kv_cache* k, const taq_kv_cache* v, const void* q,
                                   int32_t hq, const int32_t* lens, int32_t max_len,
                                   const taq_tile_mask* mask, float softmax_scale, void* o,
                                   void* stream) {
  taq_status st = decode_validate(k, v, q, hq, lens, max_len, mask, softmax_scale, o);
  if (st) return st;
  const size_t need = taq_attn_decode_workspace_bytes(k, hq, max_len);
  if (need > (size_t)TAQ_DECODE_SCRATCH_BYTES)
    return fail(TAQ_ERR_WORKSPACE_TOO_SMALL,
                "these shapes need %zu bytes of decode scratch; the no-allocation decode holds "
                "%zu (use taq_attn_decode with a workspace)", need,
                (size_t)TAQ_DECODE_SCRATCH_BYTES);
  st = device_ok();
  if (st) return st;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st) return st;
  return decode_common(k, v, q, hq, lens, max_len, mask, softmax_scale, o, ws,
                       (size_t)TAQ_DECODE_SCRATCH_BYTES, stream, false);
}

}  // extern "C"

namespace {

// Shared body of taq_attn_prefill (q_len = max_len, chunk = false) and
// taq_attn_prefill_chunk.
size_t prefill_part_bytes(int nsplit, int B, int hq, int q_len) {
  return nsplit > 1 ? (size_t)nsplit * B * hq * q_len * (128 + 4) * sizeof(float) : 0;
}

taq_status prefill_common(const taq_kv_cache* k, const taq_kv_cache* v, const void* q,
                          int32_t hq, int32_t q_len, bool chunk, const int32_t* lens,
                          int32_t max_len, const taq_tile_mask* mask, float softmax_scale,
                          void* o, void* ws, size_t ws_bytes, void* stream) {
  taq_status st = check_pair(k, v, hq, max_len);
  if (st) return st;
  if (q_len < 0 || q_len > max_len)
    return fail(TAQ_ERR_INVALID_ARGUMENT, "q_len %d outside [0, max_seq_len %d]", q_len, max_len);
  if (!q || !o || !lens) return fail(TAQ_ERR_INVALID_ARGUMENT, "null q, o or seq_lens");
  if (!aligned16(q) || !aligned16(o) || !aligned16(lens))
    return fail(TAQ_ERR_MISALIGNED, "q, o and seq_lens must be 16-byte aligned");
  if (!std::isfinite(softmax_scale))
    return fail(TAQ_ERR_INVALID_ARGUMENT, "softmax_scale must be finite");
  if (softmax_scale < 0.f)
    return fail(TAQ_ERR_UNSUPPORTED, "softmax_scale must be >= 0 (0 selects 1/sqrt(head_dim))");
  const int nt = (max_len + TAQ_TILE - 1) / TAQ_TILE;
  st = check_mask(mask, nt, nt);
  if (st) return st;
  // key-range splits when a workspace is given (chunked prefill)
  int nsplit = 1;
  if (ws) {
    if (!aligned16(ws)) return fail(TAQ_ERR_MISALIGNED, "workspace must be 16-byte aligned");
    nsplit = taq::prefill_splits(k->batch, k->num_kv_heads, hq / k->num_kv_heads, q_len, max_len);
    const size_t need = prefill_part_bytes(nsplit, k->batch, hq, q_len);
    if (ws_bytes < need)
      return fail(TAQ_ERR_WORKSPACE_TOO_SMALL, "workspace: need %zu bytes, got %zu", need,
                  ws_bytes);
  }
  st = device_ok();
  if (st) return st;
  if (max_len == 0 || q_len == 0) return TAQ_OK;
  taq::PrefillArgs a;
  std::memset(&a, 0, sizeof(a));
  a.k = geom_of(k);
  a.v = geom_of(v);
  a.q = static_cast<const uint16_t*>(q);
  a.o = static_cast<uint16_t*>(o);
  a.lens = lens;
  if (mask) {
    a.mask = mask->data;
    a.mask_sb = mask->stride_b;
    a.mask_sh = mask->stride_h;
    a.mask_nq = mask->n_q_tiles;
    a.mask_nk = mask->n_k_tiles;
  }
  a.Hq = hq;
  a.r = hq / k->num_kv_heads;
  a.L = max_len;
  a.Lq = q_len;
  a.chunk = chunk ? 1 : 0;
  const int bq = 256 / a.r;
  a.n_qblk = (q_len + bq - 1) / bq;
  a.nsplit = nsplit;
  a.part = nsplit > 1 ? static_cast<float*>(ws) : nullptr;
  a.scale_log2 = scale_log2_of(softmax_scale, 128);
  hipError_t e = taq::launch_attn_prefill(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TAQ_OK : hip_fail(e, "attn_prefill launch");
}

}  // namespace

extern "C" {

taq_status taq_attn_prefill(const taq_kv_cache* k, const taq_kv_cache* v, const void* q,
                            int32_t hq, const int32_t* lens, int32_t max_len,
                            const taq_tile_mask* mask, float softmax_scale, void* o,
                            void* stream) {
  return prefill_common(k, v, q, hq, max_len, false, lens, max_len, mask, softmax_scale, o,
                        nullptr, 0, stream);
}

size_t taq_attn_prefill_chunk_workspace_bytes(const taq_kv_cache* k, int32_t hq, int32_t q_len,
                                              int32_t max_len) {
  if (!k || k->batch < 1 || k->num_kv_heads < 1 || hq < 1 || hq % k->num_kv_heads || q_len < 0 ||
      max_len < 0)
    return 0;
  const int r = hq / k->num_kv_heads;
  if (r != 1 && r != 2 && r != 4 && r != 8) return 0;
  const int ns = taq::prefill_splits(k->batch, k->num_kv_heads, r, q_len, max_len);
  return prefill_part_bytes(ns, k->batch, hq, q_len);
}

taq_status taq_attn_prefill_chunk(const taq_kv_cache* k, const taq_kv_cache* v, const void* q,
                                  int32_t hq, int32_t q_len, const int32_t* lens,
                                  int32_t max_len, const taq_tile_mask* mask,
                                  float softmax_scale, void* o, void* ws, size_t ws_bytes,
                                  void* stream) {
  return prefill_common(k, v, q, hq, q_len, true, lens, max_len, mask, softmax_scale, o, ws,
                        ws_bytes, stream);
}

taq_status taq_kv_append(const taq_kv_cache* c, const void* x, const int32_t* starts,
                         int32_t count, void* stream) {
  taq_status st = check_cache(c, "cache", -1, false);
  if (st) return st;
  if (!x || !starts) return fail(TAQ_ERR_INVALID_ARGUMENT, "x or starts: null");
  if (!aligned16(x) || !aligned16(starts))
    return fail(TAQ_ERR_MISALIGNED, "x and starts must be 16-byte aligned");
  if (count < 0 || count > c->capacity)
    return fail(TAQ_ERR_INVALID_ARGUMENT, "count %d outside [0, capacity %d]", count,
                c->capacity);
  st = device_ok();
  if (st) return st;
  taq::QuantArgs a;
  std::memset(&a, 0, sizeof(a));
  a.c = geom_of(c);
  a.x = static_cast<const uint16_t*>(x);
  a.start = 0;
  a.count = count;
  a.starts = starts;
  hipError_t e = taq::launch_kv_quantize(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TAQ_OK : hip_fail(e, "kv_append launch");
}

size_t taq_tile_mask_workspace_bytes(const taq_kv_cache* k, int32_t max_len) {
  if (check_cache(k, "k_cache", TAQ_LAYOUT_TOKEN, true) != TAQ_OK) return 0;
  if (max_len < 0 || max_len > k->capacity) return 0;
  const size_t nt = (size_t)(max_len + TAQ_TILE - 1) / TAQ_TILE;
  // query sums and key means [B][Hkv][nt][D] each, scores [B][Hkv][nt][nt]
  return (size_t)k->batch * k->num_kv_heads * nt * (2 * k->head_dim + nt) * sizeof(double);
}

}  // extern "C"

namespace {

// Shared body of taq_tile_mask_generate (q_len = max_len, turn = false) and
// taq_tile_mask_generate_chunk (q holds the last q_len positions).
taq_status tile_mask_common(const taq_kv_cache* k, const void* q, int32_t hq, int32_t q_len,
                            bool turn, const int32_t* lens, int32_t max_len,
                            int32_t skip_per_mille, uint8_t* mask_out, void* ws,
                            size_t ws_bytes, void* stream) {
  taq_status st = check_cache(k, "k_cache", TAQ_LAYOUT_TOKEN, true);
  if (st) return st;
  if (hq < 1 || hq % k->num_kv_heads)
    return fail(TAQ_ERR_INVALID_ARGUMENT, "num_q_heads (%d) must be a positive multiple of "
                "num_kv_heads (%d)", hq, k->num_kv_heads);
  if (hq / k->num_kv_heads > 64)
    return fail(TAQ_ERR_UNSUPPORTED, "num_q_heads / num_kv_heads = %d (at most 64)",
                hq / k->num_kv_heads);
  if (max_len < 0 || max_len > k->capacity)
    return fail(TAQ_ERR_INVALID_ARGUMENT, "max_seq_len %d outside [0, capacity %d]", max_len,
                k->capacity);
  if (q_len < 0 || q_len > max_len)
    return fail(TAQ_ERR_INVALID_ARGUMENT, "q_len %d outside [0, max_seq_len %d]", q_len, max_len);
  {
    const int64_t nt = (max_len + TAQ_TILE - 1) / TAQ_TILE, nb = (nt + 63) / 64;
    const int64_t bh = (int64_t)k->batch * k->num_kv_heads;
    if (bh * nt > INT32_MAX || bh * nb * nb > INT32_MAX)
      return fail(TAQ_ERR_UNSUPPORTED, "batch * num_kv_heads * tiles beyond the grid limit");
  }
  if (max_len > taq::MASKGEN_MAX_TILES * TAQ_TILE)
    return fail(TAQ_ERR_UNSUPPORTED, "max_seq_len %d beyond %d tiles", max_len,
                taq::MASKGEN_MAX_TILES);
  if (skip_per_mille < 0 || skip_per_mille > 1000)
    return fail(TAQ_ERR_INVALID_ARGUMENT, "skip_per_mille %d outside [0, 1000]", skip_per_mille);
  // an empty turn reads no query (q may be NULL)
  if ((!q && q_len > 0) || !lens || !mask_out)
    return fail(TAQ_ERR_INVALID_ARGUMENT, "null q, seq_lens or mask");
  if ((q && !aligned16(q)) || !aligned16(lens))
    return fail(TAQ_ERR_MISALIGNED, "q and seq_lens must be 16-byte aligned");
  const size_t need = taq_tile_mask_workspace_bytes(k, max_len);
  if (!ws || ws_bytes < need)
    return fail(TAQ_ERR_WORKSPACE_TOO_SMALL, "workspace: need %zu bytes, got %zu", need,
                ws ? ws_bytes : (size_t)0);
  if (!aligned16(ws)) return fail(TAQ_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  st = device_ok();
  if (st) return st;
  if (max_len == 0) return TAQ_OK;
  taq::MaskGenArgs a;
  std::memset(&a, 0, sizeof(a));
  a.k = geom_of(k);
  a.q = static_cast<const uint16_t*>(q);
  a.lens = lens;
  a.mask = mask_out;
  a.nt = (max_len + TAQ_TILE - 1) / TAQ_TILE;
  a.qsum = static_cast<double*>(ws);
  a.kmean = a.qsum + (size_t)k->batch * k->num_kv_heads * a.nt * k->head_dim;
  a.score = a.kmean + (size_t)k->batch * k->num_kv_heads * a.nt * k->head_dim;
  a.Hq = hq;
  a.r = hq / k->num_kv_heads;
  a.L = max_len;
  a.Lq = q_len;
  a.turn = turn ? 1 : 0;
  a.skip_per_mille = skip_per_mille;
  hipError_t e = taq::launch_tile_mask(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TAQ_OK : hip_fail(e, "tile_mask launch");
}

}  // namespace

extern "C" {

taq_status taq_tile_mask_generate(const taq_kv_cache* k, const void* q, int32_t hq,
                                  const int32_t* lens, int32_t max_len,
                                  int32_t skip_per_mille, uint8_t* mask_out, void* ws,
                                  size_t ws_bytes, void* stream) {
  return tile_mask_common(k, q, hq, max_len, false, lens, max_len, skip_per_mille, mask_out, ws,
                          ws_bytes, stream);
}

taq_status taq_tile_mask_generate_chunk(const taq_kv_cache* k, const void* q, int32_t hq,
                                        int32_t q_len, const int32_t* lens, int32_t max_len,
                                        int32_t skip_per_mille, uint8_t* mask_out, void* ws,
                                        size_t ws_bytes, void* stream) {
  return tile_mask_common(k, q, hq, q_len, true, lens, max_len, skip_per_mille, mask_out, ws,
                          ws_bytes, stream);
}

}  // extern "C"

namespace {

// Workspace of taq_head_sensitivity: an int8 and an int4 copy of the K
// (token layout) and V (channel layout) caches, the two decode outputs and one
// decode workspace (the two decode calls run one after the other).
struct SensPlan {
  int cap = 0;
  size_t k8c, k8s, k8z, v8c, v8s, v8z, k4c, k4s, k4z, v4c, v4s, v4z, o8, o4, dec, total = 0;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

SensPlan sens_plan(int B, int Hkv, int hq, int max_len) {
  SensPlan p;
  p.cap = max_len > 0 ? (max_len + TAQ_TILE - 1) / TAQ_TILE * TAQ_TILE : TAQ_TILE;
  const size_t meta = (size_t)B * Hkv * p.cap * 4;
  const size_t c8 = (size_t)B * Hkv * p.cap * 128, c4 = c8 / 2;
  size_t at = 0;
  auto take = [&](size_t bytes) { const size_t o = at; at += align256(bytes); return o; };
  p.k8c = take(c8); p.k8s = take(2 * meta); p.k8z = take(meta);
  p.v8c = take(c8); p.v8s = take(2 * meta); p.v8z = take(meta);
  p.k4c = take(c4); p.k4s = take(2 * meta); p.k4z = take(meta);
  p.v4c = take(c4); p.v4s = take(2 * meta); p.v4z = take(meta);
  p.o8 = take((size_t)B * hq * 128 * 2);
  p.o4 = take((size_t)B * hq * 128 * 2);
  p.dec = take(taq::decode_workspace_bytes(B, Hkv, hq, max_len));
  p.total = at;
  return p;
}

taq::CacheGeom uniform_geom(uint8_t* base, size_t c, size_t sc, size_t z, int B, int H, int cap,
                            int bits, int layout) {
  taq::CacheGeom g;
  std::memset(&g, 0, sizeof(g));
  g.codes = base + c;
  g.scales = reinterpret_cast<uint16_t*>(base + sc);
  g.zeros = base + z;
  const int64_t per = (int64_t)cap * 128 * bits / 8;
  for (int h = 0; h < H; ++h) g.hoff[h] = h * per;
  g.bstride = H * per;
  g.is8 = bits == 8 ? (H == 64 ? ~0ull : ((1ull << H) - 1)) : 0ull;
  g.B = B;
  g.H = H;
  g.D = 128;
  g.cap = cap;
  g.layout = layout;
  return g;
}

}  // namespace

extern "C" {

size_t taq_head_sensitivity_workspace_bytes(int32_t batch, int32_t num_kv_heads,
                                            int32_t num_q_heads, int32_t max_len) {
  if (batch < 1 || num_kv_heads < 1 || num_kv_heads > TAQ_MAX_KV_HEADS || num_q_heads < 1 ||
      max_len < 0)
    return 0;
  return sens_plan(batch, num_kv_heads, num_q_heads, max_len).total;
}

taq_status taq_head_sensitivity(const void* k, const void* v, const void* q, int32_t batch,
                                int32_t hkv, int32_t hq, const int32_t* lens, int32_t max_len,
                                float softmax_scale, int32_t n_high, double* scores,
                                uint8_t* bits, void* ws, size_t ws_bytes, void* stream) {
  if (batch < 1) return fail(TAQ_ERR_INVALID_ARGUMENT, "batch must be >= 1");
  if (hkv < 1 || hkv > TAQ_MAX_KV_HEADS)
    return fail(TAQ_ERR_INVALID_ARGUMENT, "num_kv_heads must be in [1, %d]", TAQ_MAX_KV_HEADS);
  if (hq < 1 || hq % hkv)
    return fail(TAQ_ERR_INVALID_ARGUMENT, "num_q_heads (%d) must be a positive multiple of "
                "num_kv_heads (%d)", hq, hkv);
  const int r = hq / hkv;
  if (r != 1 && r != 2 && r != 4 && r != 8)
    return fail(TAQ_ERR_UNSUPPORTED, "num_q_heads / num_kv_heads = %d (supported: 1, 2, 4, 8)", r);
  if (max_len < 0) return fail(TAQ_ERR_INVALID_ARGUMENT, "max_seq_len must be >= 0");
  if (n_high < 0 || n_high > hkv)
    return fail(TAQ_ERR_INVALID_ARGUMENT, "n_high %d outside [0, num_kv_heads %d]", n_high, hkv);
  if (!k || !v || !q || !lens || !scores || !bits)
    return fail(TAQ_ERR_INVALID_ARGUMENT, "null k, v, q, seq_lens, scores or bits");
  if (!aligned16(k) || !aligned16(v) || !aligned16(q) || !aligned16(lens))
    return fail(TAQ_ERR_MISALIGNED, "k, v, q and seq_lens must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(scores) & 7u) != 0)
    return fail(TAQ_ERR_MISALIGNED, "scores must be 8-byte aligned");
  if (!std::isfinite(softmax_scale))
    return fail(TAQ_ERR_INVALID_ARGUMENT, "softmax_scale must be finite");
  if (softmax_scale < 0.f)
    return fail(TAQ_ERR_UNSUPPORTED, "softmax_scale must be >= 0 (0 selects 1/sqrt(head_dim))");
  const SensPlan p = sens_plan(batch, hkv, hq, max_len);
  if (!ws || ws_bytes < p.total)
    return fail(TAQ_ERR_WORKSPACE_TOO_SMALL, "workspace: need %zu bytes, got %zu", p.total,
                ws ? ws_bytes : (size_t)0);
  if (!aligned16(ws)) return fail(TAQ_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  taq_status st = device_ok();
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* w = static_cast<uint8_t*>(ws);
  const taq::CacheGeom k8 = uniform_geom(w, p.k8c, p.k8s, p.k8z, batch, hkv, p.cap, 8, TAQ_LAYOUT_TOKEN);
  const taq::CacheGeom v8 = uniform_geom(w, p.v8c, p.v8s, p.v8z, batch, hkv, p.cap, 8, TAQ_LAYOUT_CHANNEL);
  const taq::CacheGeom k4 = uniform_geom(w, p.k4c, p.k4s, p.k4z, batch, hkv, p.cap, 4, TAQ_LAYOUT_TOKEN);
  const taq::CacheGeom v4 = uniform_geom(w, p.v4c, p.v4s, p.v4z, batch, hkv, p.cap, 4, TAQ_LAYOUT_CHANNEL);
  hipError_t e = hipSuccess;
  if (max_len > 0) {
    const taq::CacheGeom* gs[4] = {&k8, &v8, &k4, &v4};
    const void* xs[4] = {k, v, k, v};
    for (int i = 0; i < 4 && e == hipSuccess; ++i) {
      taq::QuantArgs qa;
      std::memset(&qa, 0, sizeof(qa));
      qa.c = *gs[i];
      qa.x = static_cast<const uint16_t*>(xs[i]);
      qa.start = 0;
      qa.count = max_len;
      e = taq::launch_kv_quantize(qa, s);
    }
    if (e != hipSuccess) return hip_fail(e, "head_sensitivity quantise");
  }
  for (int pass = 0; pass < 2; ++pass) {
    taq::DecodeArgs a;
    std::memset(&a, 0, sizeof(a));
    a.k = pass == 0 ? k8 : k4;
    a.v = pass == 0 ? v8 : v4;
    a.q = static_cast<const uint16_t*>(q);
    a.o = reinterpret_cast<uint16_t*>(w + (pass == 0 ? p.o8 : p.o4));
    a.lens = lens;
    a.ws = reinterpret_cast<float*>(w + p.dec);
    a.Hq = hq;
    a.r = r;
    a.max_len = max_len;
    a.chunk = taq::decode_chunk_tokens(batch, hkv, max_len);
    a.nchunk = max_len > 0 ? (max_len + a.chunk - 1) / a.chunk : 1;
    a.scale_log2 = scale_log2_of(softmax_scale, 128);
    e = taq::launch_attn_decode(a, s, false);
    if (e != hipSuccess) return hip_fail(e, "head_sensitivity decode");
  }
  e = taq::launch_head_assign(reinterpret_cast<const uint16_t*>(w + p.o8),
                              reinterpret_cast<const uint16_t*>(w + p.o4), batch, hq, hkv,
                              n_high, scores, bits, s);
  return e == hipSuccess ? TAQ_OK : hip_fail(e, "head_sensitivity assign");
}

}  // extern "C"
