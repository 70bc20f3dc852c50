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

// round-half-even(a / s) for fp16 values |a| <= 256 s, s > 0, decided exactly
// in fp32 from an approximate quotient.  With t = floor(q) for any q within
// 1/2 of a / s, the answer is t or t + 1 and the midpoint (t + 1/2) s
// separates them (ties go to the even one, for either sign of a); that
// product has at most 10 + 11 significant bits, so it and the comparison with
// a are exact.  (q = a * rcp(s) is within a few ulp of a / s, |a / s| <= 256,
// far inside 1/2.)
__device__ __forceinline__ int rne_quot(float a, float s, float rs) {
  const float t = floorf(a * rs);
  const float mid = (t + 0.5f) * s;
  const int n = (int)t;
  // branch-free: up when above the midpoint, or on it with n odd
  return n + ((int)(a > mid) | ((int)(a == mid) & n & 1));
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
    const int c = rne_quot(x[i], sf, rs) + z;
    out.c[i] = (uint8_t)min(max(c, 0), qmax);
  }
  out.scale_bits = sb;
  out.zero = (uint32_t)z;
}

__device__ __forceinline__ int head_bits(const CacheGeom& g, int h) {
  return ((g.is8 >> h) & 1ull) ? 8 : 4;
}

// Token layout: one workgroup of D threads per (b, h, 32-position block), the
// same blocks as the channel layout; thread (t = tid / G, gi = tid % G)
// quantises group gi of position 32 j + t when it lies in the written range
// (append: per-batch start; positions outside the capacity are skipped).
__device__ __forceinline__ void quantize_token_block(const QuantArgs& a, int j0, int nblk,
                                                     int blk) {
  const CacheGeom& g = a.c;
  const int G = g.D / 32;
  const int jrel = blk % nblk;
  const int bh = blk / nblk;
  const int h = bh % g.H, b = bh / g.H;
  const int start = a.starts ? a.starts[b] : a.start;
  const int j = (a.starts ? (start >> 5) : j0) + jrel;
  const int t = threadIdx.x / G, gi = threadIdx.x - t * G;
  const int T = 32 * j + t;
  if (T < start || T >= start + a.count || T < 0 || T >= g.cap) return;
  const int bits = head_bits(g, h);
  GroupQ q;
  quantize_group(a.x + ((((int64_t)b * g.H + h) * a.count + (T - start)) * g.D + 32 * gi),
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

__global__ void __launch_bounds__(1024)
quantize_token_kernel(QuantArgs a, int j0, int nblk) {
  quantize_token_block(a, j0, nblk, blockIdx.x);
}

// Channel layout: one workgroup of D threads per (b, h, 32-token block).
// Thread (token t = tid / G, group gi = tid % G) quantises its group (a wave
// reads whole token rows, contiguous), writes its scale and zero-point, and
// puts its 32 codes into an LDS copy of the block (row = channel, one byte per
// token); thread d then writes channel row d of the block (int8: 32 bytes,
// int4: 16 bytes, two tokens per byte), so the block goes out as contiguous
// 16-byte stores.  Blocks cut by the ends of the written range write only
// their tokens (an int4 byte shared with a token outside the range is
// read, merged and written back).
__device__ __forceinline__ void quantize_channel_block(const QuantArgs& a, int j0, int nblk,
                                                       int blk, uint8_t* cl_raw) {
  // cl_raw: [D][36] bytes of LDS, [channel][token] (+4: bank skew)
  uint8_t (*cl)[36] = reinterpret_cast<uint8_t (*)[36]>(cl_raw);
  const CacheGeom& g = a.c;
  const int G = g.D / 32;
  const int jrel = blk % nblk;
  const int bh = blk / nblk;
  const int h = bh % g.H, b = bh / g.H;
  const int start = a.starts ? a.starts[b] : a.start;
  const int j = (a.starts ? (start >> 5) : j0) + jrel;
  // tokens [lo, hi) of this block are written
  const int lo = max(max(start, 32 * j), 0), hi = min(min(start + a.count, 32 * j + 32), g.cap);
  if (lo >= hi) return;                         // whole workgroup
  const int bits = head_bits(g, h);
  const int tid = threadIdx.x;
  const int t = tid / G, gi = tid - t * G;
  const int T = 32 * j + t;
  if (T >= lo && T < hi) {
    GroupQ q;
    quantize_group(a.x + (((int64_t)b * g.H + h) * a.count + (T - start)) * g.D + 32 * gi, bits,
                   q);
#pragma unroll
    for (int i = 0; i < 32; ++i) cl[32 * gi + i][t] = q.c[i];
    const int64_t mi = (((int64_t)b * g.H + h) * G + gi) * g.cap + T;
    g.scales[mi] = (uint16_t)q.scale_bits;
    g.zeros[mi] = (uint8_t)q.zero;
  }
  __syncthreads();
  const int d = tid;                             // channel row
  const int rowb = 4 * bits;
  uint8_t* row = g.codes + (int64_t)b * g.bstride + g.hoff[h] + ((int64_t)j * g.D + d) * rowb;
  const int t0 = lo - 32 * j, t1 = hi - 32 * j;
  if (bits == 8) {
    if (t0 == 0 && t1 == 32) {
      u32x4 w[2];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        w[k >> 2][k & 3] = cl[d][4 * k] | (cl[d][4 * k + 1] << 8) | (cl[d][4 * k + 2] << 16) |
                           ((uint32_t)cl[d][4 * k + 3] << 24);
      reinterpret_cast<u32x4*>(row)[0] = w[0];
      reinterpret_cast<u32x4*>(row)[1] = w[1];
    } else {
      for (int k = t0; k < t1; ++k) row[k] = cl[d][k];
    }
  } else {
    if (t0 == 0 && t1 == 32) {
      u32x4 w;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint32_t v = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) v |= (uint32_t)cl[d][8 * k + e] << (4 * e);
        w[k] = v;
      }
      *reinterpret_cast<u32x4*>(row) = w;
    } else {
      for (int k = t0 >> 1; k <= (t1 - 1) >> 1; ++k) {
        const bool in0 = 2 * k >= t0, in1 = 2 * k + 1 < t1;
        uint8_t v = row[k];
        if (in0) v = (uint8_t)((v & 0xF0) | cl[d][2 * k]);
        if (in1) v = (uint8_t)((v & 0x0F) | (cl[d][2 * k + 1] << 4));
        row[k] = v;
      }
    }
  }
}

__global__ void __launch_bounds__(1024)
quantize_channel_kernel(QuantArgs a, int j0, int nblk) {
  extern __shared__ uint8_t cl_raw[];
  quantize_channel_block(a, j0, nblk, blockIdx.x, cl_raw);
}

// Two caches of equal head_dim (K and V) in one launch: workgroups below n0
// quantise a0's blocks, the others a1's, each with its cache's layout; the
// two run side by side instead of one after the other.
__global__ void __launch_bounds__(1024)
quantize_pair_kernel(QuantArgs a0, int j00, int nblk0, int n0, QuantArgs a1, int j01,
                     int nblk1) {
  extern __shared__ uint8_t cl_raw[];
  // each branch reads its own argument block directly (selecting one of the
  // two by a runtime condition would copy them to per-thread memory)
  const int blk = blockIdx.x;
  if (blk < n0) {
    if (a0.c.layout == TAQ_LAYOUT_TOKEN)
      quantize_token_block(a0, j00, nblk0, blk);
    else
      quantize_channel_block(a0, j00, nblk0, blk, cl_raw);
  } else {
    if (a1.c.layout == TAQ_LAYOUT_TOKEN)
      quantize_token_block(a1, j01, nblk1, blk - n0);
    else
      quantize_channel_block(a1, j01, nblk1, blk - n0, cl_raw);
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

// 32-position blocks: the range's own, or (per-batch starts) enough blocks
// from each start's block to cover count tokens at any alignment
static void quant_blocks(const QuantArgs& a, int& j0, int& nblk) {
  j0 = a.starts ? 0 : a.start / 32;
  nblk = a.starts ? a.count / 32 + 2 : (a.start + a.count - 1) / 32 - j0 + 1;
}

hipError_t launch_kv_quantize_pair(const QuantArgs& a0, const QuantArgs& a1, hipStream_t s) {
  if (a0.count == 0) return hipSuccess;   // both caches take the same token range
  int j00, nblk0, j01, nblk1;
  quant_blocks(a0, j00, nblk0);
  quant_blocks(a1, j01, nblk1);
  const int64_t n0 = (int64_t)a0.c.B * a0.c.H * nblk0;
  const int64_t n1 = (int64_t)a1.c.B * a1.c.H * nblk1;
  const bool chan = a0.c.layout != TAQ_LAYOUT_TOKEN || a1.c.layout != TAQ_LAYOUT_TOKEN;
  hipLaunchKernelGGL(quantize_pair_kernel, dim3((unsigned)(n0 + n1)), dim3(a0.c.D),
                     chan ? a0.c.D * 36 : 0, s, a0, j00, nblk0, (int)n0, a1, j01, nblk1);
  return hipGetLastError();
}

hipError_t launch_kv_quantize(const QuantArgs& a, hipStream_t s) {
  if (a.count == 0) return hipSuccess;
  int j0, nblk;
  quant_blocks(a, j0, nblk);
  const int64_t n = (int64_t)a.c.B * a.c.H * nblk;
  if (a.c.layout == TAQ_LAYOUT_TOKEN)
    hipLaunchKernelGGL(quantize_token_kernel, dim3((unsigned)n), dim3(a.c.D), 0, s, a, j0, nblk);
  else
    hipLaunchKernelGGL(quantize_channel_kernel, dim3((unsigned)n), dim3(a.c.D), a.c.D * 36, s, a,
                       j0, nblk);
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
