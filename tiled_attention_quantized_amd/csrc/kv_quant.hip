// Grouped asymmetric KV quantisation and dequantisation kernels.
//
// Method: "分块稀疏注意力与KV Cache量化：长文本推理显存优化实践" (xdnf.cn),
// section 2.4 -- adjacent channels form a group with its own scale and
// zero-point -- with the group size 32 of section 3.2.  The rounding rules
// (range widened to contain 0, scale rounded up to fp16, zero-point and codes
// rounded half to even on the exact quotients) are stated in include/taq.h.
//
// Exactness: an fp16 value is an integer multiple of 2^-24 below 2^41 in those
// units; the scale is rounded up in 64-bit integer counts of 2^-24, and each
// round-half-even quotient is decided by an exact fp32 comparison with the
// midpoint between its two candidates (rne_quot), so no approximate quotient
// ever decides a tie.
#include "taq_internal.h"
#include "device_common.h"

namespace taq {
namespace {

// Value of an fp16 bit pattern in units of 2^-24 (finite inputs only).
__device__ __forceinline__ int64_t f16_units(uint32_t h) {
  const uint32_t e = (h >> 10) & 31u, m = h & 1023u;
  const int64_t mag = e == 0 ? (int64_t)m : ((int64_t)(1024u + m) << (e - 1));
  return (h & 0x8000u) ? -mag : mag;
}

// Least fp16 value >= m (m >= 1, in units of 2^-24); returns it in units and
// as an fp16 bit pattern.
__device__ __forceinline__ uint64_t fp16_ceil(uint64_t m, uint32_t& bits) {
  uint64_t s = m;
  if (m >= 2048) {
    const int e = 63 - __clzll(m);
    const uint64_t step = 1ull << (e - 10);
    s = (m + step - 1) & ~(step - 1);
  }
  if (s < 1024) {
    bits = (uint32_t)s;
  } else {
    const int e = 63 - __clzll(s);
    const uint64_t mant = s >> (e - 10);
    bits = ((uint32_t)(e - 9) << 10) | (uint32_t)(mant - 1024);
  }
  return s;
}

struct GroupQ {
  uint8_t c[32];
  uint32_t scale_bits;
  uint32_t zero;
};

// round-half-even(a / s) for fp16 values 0 <= a <= 256 s, s > 0, decided
// exactly in fp32 from an approximate quotient.  With t = floor(q) for any q
// within 1/2 of a / s, the answer is t or t + 1 and the midpoint (t + 1/2) s
// separates them; that product has at most 10 + 11 significant bits, so it
// and the comparison with a are exact, ties included.  (q = a * rcp(s) is
// within a few ulp of a / s <= 256, far inside 1/2.)
__device__ __forceinline__ int rne_quot(float a, float s, float rs) {
  const float t = floorf(a * rs);
  const float mid = (t + 0.5f) * s;
  const int n = (int)t;
  return (a > mid || (a == mid && (n & 1))) ? n + 1 : n;
}

// Quantise the 32 fp16 values at p (16-byte aligned).
__device__ __forceinline__ void quantize_group(const uint16_t* p, int bits,
                                               GroupQ& out) {
  uint32_t w[16];
  const uint4* p4 = reinterpret_cast<const uint4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = p4[i];
    w[4 * i + 0] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
  }
  float x[32];
  float lo = 0.f, hi = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    x[i] = (float)bits_to_half((uint16_t)((w[i >> 1] >> (16 * (i & 1))) & 0xFFFFu));
    lo = fminf(lo, x[i]);
    hi = fmaxf(hi, x[i]);
  }
  const int qmax = (1 << bits) - 1;
  if (hi == lo) {                           // all zeros (the range contains 0)
#pragma unroll
    for (int i = 0; i < 32; ++i) out.c[i] = 0;
    out.scale_bits = 0;
    out.zero = 0;
    return;
  }
  // the scale: least fp16 >= (hi - lo) / qmax, in integer units of 2^-24
  const uint64_t span = (uint64_t)(f16_units(half_to_bits((_Float16)hi)) -
                                   f16_units(half_to_bits((_Float16)lo)));
  uint32_t sb;
  // (constant divisors: the compiler multiplies instead of dividing)
  fp16_ceil(bits == 8 ? (span + 254) / 255 : (span + 14) / 15, sb);
  const float sf = (float)bits_to_half((uint16_t)sb);
  const float rs = __builtin_amdgcn_rcpf(sf);
  const int z = rne_quot(-lo, sf, rs);
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int q = rne_quot(fabsf(x[i]), sf, rs);
    int c = (x[i] < 0.f ? -q : q) + z;
    c = c < 0 ? 0 : (c > qmax ? qmax : c);
    out.c[i] = (uint8_t)c;
  }
  out.scale_bits = sb;
  out.zero = (uint32_t)z;
}

__device__ __forceinline__ int head_bits(const CacheGeom& g, int h) {
  return ((g.is8 >> h) & 1ull) ? 8 : 4;
}

// Token layout: one thread per (b, h, token, group).
__global__ void __launch_bounds__(256)
quantize_token_kernel(QuantArgs a) {
  const CacheGeom& g = a.c;
  const int G = g.D / 32;
  const int64_t total = (int64_t)g.B * g.H * a.count * G;
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= total) return;
  const int gi = (int)(id % G);
  int64_t rest = id / G;
  const int t = (int)(rest % a.count);
  rest /= a.count;
  const int h = (int)(rest % g.H);
  const int b = (int)(rest / g.H);
  const int bits = head_bits(g, h);
  // append: per-batch start, positions outside the capacity are skipped
  const int T = (a.starts ? a.starts[b] : a.start) + t;
  if (T < 0 || T >= g.cap) return;
  GroupQ q;
  quantize_group(a.x + ((((int64_t)b * g.H + h) * a.count + t) * g.D + 32 * gi),
                 bits, q);
  uint8_t* row = g.codes + (int64_t)b * g.bstride + g.hoff[h] +
                 (int64_t)T * (g.D * bits / 8) + gi * 4 * bits;
  if (bits == 8) {
    uint32_t wv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      wv[i] = q.c[4 * i] | (q.c[4 * i + 1] << 8) | (q.c[4 * i + 2] << 16) |
              ((uint32_t)q.c[4 * i + 3] << 24);
    uint4* d = reinterpret_cast<uint4*>(row);
    d[0] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
    d[1] = make_uint4(wv[4], wv[5], wv[6], wv[7]);
  } else {
    uint32_t wv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t v = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) v |= (uint32_t)q.c[8 * i + j] << (4 * j);
      wv[i] = v;
    }
    *reinterpret_cast<uint4*>(row) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
  }
  const int64_t mi = (((int64_t)b * g.H + h) * g.cap + T) * G + gi;
  g.scales[mi] = (uint16_t)q.scale_bits;
  g.zeros[mi] = (uint8_t)q.zero;
}

// Channel layout: one thread per (b, h, group, token pair {2p, 2p+1}); both
// tokens of a pair share their int4 bytes, so one thread owns them.
__global__ void __launch_bounds__(256)
quantize_channel_kernel(QuantArgs a, int p0, int npairs) {
  const CacheGeom& g = a.c;
  const int G = g.D / 32;
  const int64_t total = (int64_t)g.B * g.H * G * npairs;
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= total) return;
  int64_t rest = id / npairs;
  const int gi = (int)(rest % G);
  rest /= G;
  const int h = (int)(rest % g.H);
  const int b = (int)(rest / g.H);
  // append: per-batch start; the pair index is relative to the start's pair
  const int start = a.starts ? a.starts[b] : a.start;
  const int p = (a.starts ? (start >> 1) : p0) + (int)(id % npairs);
  const int bits = head_bits(g, h);
  const int T0 = 2 * p;
  const bool in0 = T0 >= start && T0 < start + a.count && T0 >= 0 && T0 < g.cap;
  const bool in1 = T0 + 1 >= start && T0 + 1 < start + a.count && T0 + 1 >= 0 && T0 + 1 < g.cap;
  if (!in0 && !in1) return;
  GroupQ q0, q1;
  const int64_t xbase = ((int64_t)b * g.H + h) * a.count;
  if (in0) quantize_group(a.x + ((xbase + T0 - start) * g.D + 32 * gi), bits, q0);
  if (in1) quantize_group(a.x + ((xbase + T0 + 1 - start) * g.D + 32 * gi), bits, q1);
  const int rowb = 4 * bits;  // bytes per channel row of a 32-token block
  uint8_t* blk = g.codes + (int64_t)b * g.bstride + g.hoff[h] +
                 (int64_t)(T0 / 32) * g.D * rowb;
  const int tt = T0 % 32;
#pragma unroll 4
  for (int i = 0; i < 32; ++i) {
    uint8_t* row = blk + (int64_t)(32 * gi + i) * rowb;
    if (bits == 8) {
      if (in0 && in1) {
        *reinterpret_cast<uint16_t*>(row + tt) = (uint16_t)(q0.c[i] | (q1.c[i] << 8));
      } else if (in0) {
        row[tt] = q0.c[i];
      } else if (in1) {
        row[tt + 1] = q1.c[i];
      }
    } else {
      uint8_t* bp = row + tt / 2;
      if (in0 && in1) {
        *bp = (uint8_t)(q0.c[i] | (q1.c[i] << 4));
      } else if (in0) {
        *bp = (uint8_t)((*bp & 0xF0) | q0.c[i]);
      } else if (in1) {
        *bp = (uint8_t)((*bp & 0x0F) | (q1.c[i] << 4));
      }
    }
  }
  const int64_t mrow = (((int64_t)b * g.H + h) * G + gi) * g.cap;
  if (in0) {
    g.scales[mrow + T0] = (uint16_t)q0.scale_bits;
    g.zeros[mrow + T0] = (uint8_t)q0.zero;
  }
  if (in1) {
    g.scales[mrow + T0 + 1] = (uint16_t)q1.scale_bits;
    g.zeros[mrow + T0 + 1] = (uint8_t)q1.zero;
  }
}

// One thread per (b, h, token, group).
__global__ void __launch_bounds__(256)
dequantize_kernel(QuantArgs a) {
  const CacheGeom& g = a.c;
  const int G = g.D / 32;
  const int64_t total = (int64_t)g.B * g.H * a.count * G;
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= total) return;
  const int gi = (int)(id % G);
  int64_t rest = id / G;
  const int t = (int)(rest % a.count);
  rest /= a.count;
  const int h = (int)(rest % g.H);
  const int b = (int)(rest / g.H);
  const int bits = head_bits(g, h);
  const int T = a.start + t;
  const uint8_t* base = g.codes + (int64_t)b * g.bstride + g.hoff[h];
  int64_t mi;
  if (g.layout == TAQ_LAYOUT_TOKEN)
    mi = (((int64_t)b * g.H + h) * g.cap + T) * G + gi;
  else
    mi = (((int64_t)b * g.H + h) * G + gi) * g.cap + T;
  const float s = (float)bits_to_half((uint16_t)g.scales[mi]);
  const int z = g.zeros[mi];
  const int64_t oi = (((int64_t)b * g.H + h) * a.count + t) * g.D + 32 * gi;
  for (int i = 0; i < 32; ++i) {
    const int d = 32 * gi + i;
    int c;
    if (g.layout == TAQ_LAYOUT_TOKEN) {
      const uint8_t* row = base + (int64_t)T * (g.D * bits / 8);
      c = bits == 8 ? row[d] : ((row[d / 2] >> (4 * (d & 1))) & 15);
    } else {
      const uint8_t* row = base + ((int64_t)(T / 32) * g.D + d) * (4 * bits);
      const int tt = T % 32;
      c = bits == 8 ? row[tt] : ((row[tt / 2] >> (4 * (tt & 1))) & 15);
    }
    const float v = (float)(c - z) * s;   // exact: <= 19 significant bits
    if (a.out32) a.out32[oi + i] = v;
    if (a.out16) a.out16[oi + i] = half_to_bits((_Float16)v);
  }
}

inline unsigned blocks_for(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

}  // namespace

hipError_t launch_kv_quantize(const QuantArgs& a, hipStream_t s) {
  const int G = a.c.D / 32;
  if (a.count == 0) return hipSuccess;
  if (a.c.layout == TAQ_LAYOUT_TOKEN) {
    const int64_t n = (int64_t)a.c.B * a.c.H * a.count * G;
    hipLaunchKernelGGL(quantize_token_kernel, dim3(blocks_for(n, 256)), dim3(256), 0, s, a);
  } else {
    // per-batch starts: up to count / 2 + 1 pairs from each start's pair
    const int p0 = a.starts ? 0 : a.start / 2;
    const int np = a.starts ? a.count / 2 + 1 : (a.start + a.count - 1) / 2 - p0 + 1;
    const int64_t n = (int64_t)a.c.B * a.c.H * G * np;
    hipLaunchKernelGGL(quantize_channel_kernel, dim3(blocks_for(n, 256)), dim3(256), 0, s,
                       a, p0, np);
  }
  return hipGetLastError();
}

hipError_t launch_kv_dequantize(const QuantArgs& a, hipStream_t s) {
  const int G = a.c.D / 32;
  if (a.count == 0) return hipSuccess;
  const int64_t n = (int64_t)a.c.B * a.c.H * a.count * G;
  hipLaunchKernelGGL(dequantize_kernel, dim3(blocks_for(n, 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace taq
