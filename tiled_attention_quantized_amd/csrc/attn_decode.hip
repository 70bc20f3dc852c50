// Single-token decode attention over the grouped-quantized KV cache.
//
// Method: scaled dot-product attention (Space Bunny inference-stack article,
// m.xxqk.cn, section 3.1) evaluated tile by tile with the running maximum and
// normaliser carried from tile to tile ("分块稀疏注意力与KV Cache量化：长文本推理
// 显存优化实践", xdnf.cn, section 2.2), reading K/V codes and dequantising them
// in the load path (same page, section 1.3; decode is bound by the KV read,
// section 5.3), skipping KV tiles the block mask drops (section 2.3).
//
// Work decomposition (gfx950, wave64):
//  * grid = (KV chunk, KV head, batch); a 256-thread workgroup owns one chunk
//    of `chunk` tokens of one (batch, KV head) and serves all r = Hq/Hkv query
//    heads of that KV head, so each K/V byte is read once.
//  * each of the 4 waves streams chunk/4 tokens in steps of 32 tokens and keeps
//    its own (max, normaliser, accumulator); the waves merge through LDS and the
//    workgroup writes one partial triple per query head to the workspace;
//  * a second kernel merges the chunk partials of each (batch, query head) in
//    chunk order and writes fp16 O.
//
// Per step, both contractions run on the matrix cores (v_mfma_f32_16x16x32_f16):
//  * scores: A = block-diagonal Q (row = (head, quant group), 16 rows per block
//    of 4 heads), B = K codes converted exactly to (c - z) in fp16.  Each lane
//    ends up with the 4 per-group partial dot products of one (head, token) and
//    applies the 4 group scales itself: score = sum_g s_g * dot_g.
//  * PV: A = V-hat^T (rows = channels) dequantised to fp16 in registers from
//    the channel-major V layout (8 consecutive tokens of one channel per lane),
//    B = P^T gathered across lanes with ds_bpermute; O^T accumulates in fp32.
#include "taq_internal.h"
#include "device_common.h"

namespace taq {
namespace {

constexpr int D = 128;
constexpr int STEP = 32;       // tokens per wave step
constexpr int WAVES = 4;
constexpr float NEG_BIG = -1.0e30f;

// Token of QK column t' (0..15) in QK block bk (0/1) of a step: chosen so that
// lane t' holds the token pair that the PV operand packs as one dword.
template <bool V8>
__device__ __forceinline__ int qk_token(int bk, int tp) {
  if (V8) return 2 * tp + bk;
  return 8 * (tp >> 2) + (tp & 3) + 4 * bk;
}

// -(1024 + z) half2 for two zero bytes, pair m of 8 consecutive tokens.
template <bool V8>
__device__ __forceinline__ uint32_t v_negz_pair(u32x2 z8, int m) {
  if (V8) {
    const uint32_t w = m < 2 ? z8[0] : z8[1];
    return perm_b32(0xE4E4E4E4u, w, (m & 1) ? 0x04030402u : 0x04010400u);
  }
  const uint32_t sel = (uint32_t)m | (0x0Cu << 8) | ((uint32_t)(4 + m) << 16) | (0x0Cu << 24);
  return perm_b32(z8[1], z8[0], sel) | 0xE400E400u;
}

template <bool V8>
__device__ __forceinline__ uint32_t v_scale_pair(u32x4 s8, int m) {
  if (V8) return s8[m];
  const uint32_t lo = s8[m >> 1], hi = s8[2 + (m >> 1)];
  return perm_b32(hi, lo, (m & 1) ? 0x07060302u : 0x05040100u);
}

template <bool V8>
__device__ __forceinline__ uint32_t v_code_pair(u32x2 c8, int m) {
  if (V8) return bytes_to_biased_h2(m < 2 ? c8[0] : c8[1], m & 1);
  return nibbles_to_biased_h2(c8[0], m);
}

// Token index (0..7 within a lane's 8) of half `hh` of pair m.
template <bool V8>
__device__ __forceinline__ int v_pair_token(int m, int hh) {
  return V8 ? 2 * m + hh : m + 4 * hh;
}

template <int R, bool K8, bool V8>
__device__ void decode_body(const DecodeArgs& a, int b, int g, int c, int n,
                            float* lds) {
  constexpr int NRB = (R + 3) / 4;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int i16 = lane & 15;
  const int lg = lane >> 4;

  const CacheGeom& K = a.k;
  const CacheGeom& V = a.v;
  const int G = D / 32;
  const uint8_t* kbase = K.codes + (int64_t)b * K.bstride + K.hoff[g];
  const uint8_t* vbase = V.codes + (int64_t)b * V.bstride + V.hoff[g];
  const uint16_t* kscale = K.scales + ((int64_t)b * K.H + g) * K.cap * G;
  const uint8_t* kzero = K.zeros + ((int64_t)b * K.H + g) * K.cap * G;
  const uint16_t* vscale = V.scales + ((int64_t)b * V.H + g) * G * (int64_t)V.cap;
  const uint8_t* vzero = V.zeros + ((int64_t)b * V.H + g) * G * (int64_t)V.cap;
  const int cap = K.cap;

  // ---- Q as the block-diagonal A operand ------------------------------------
  half8 aq[NRB][4];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int hl = 4 * rb + (i16 >> 2);
    const bool live = hl < R && (i16 & 3) == lg;
    u32x4 chunk[4] = {};
    if (live) {
      const u32x4* qp = reinterpret_cast<const u32x4*>(
          a.q + ((int64_t)b * a.Hq + g * R + hl) * D + 32 * lg);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) chunk[kk] = qp[kk];
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      u32x4 o;
      if (K8) {
        o = chunk[kk];
      } else {
        // slots (2k, 2k+1) hold channels (8kk + k, 8kk + k + 4)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t lo = chunk[kk][k >> 1], hi = chunk[kk][2 + (k >> 1)];
          o[k] = perm_b32(hi, lo, (k & 1) ? 0x07060302u : 0x05040100u);
        }
      }
      aq[rb][kk] = u4_to_h8(o);
    }
  }

  // ---- wave state ------------------------------------------------------------
  float m_run[NRB], l_run[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) { m_run[rb] = NEG_BIG; l_run[rb] = 0.f; }
  f32x4 acc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int per_wave = a.chunk / WAVES;
  const int t_begin = c * a.chunk + w * per_wave;
  const int t_end = min(t_begin + per_wave, n);
  const uint8_t* mrow = a.mask ? a.mask + (int64_t)b * a.mask_sb + (int64_t)g * a.mask_sh
                               : nullptr;

  for (int t0 = t_begin; t0 < t_end; t0 += STEP) {
    if (mrow && !mrow[t0 >> 7]) continue;
    const int nvalid = t_end - t0;  // tokens t0 .. t0+nvalid-1 are valid (if < 32)

    // ---------------- scores ----------------
    float sc[NRB][2];
#pragma unroll
    for (int bk = 0; bk < 2; ++bk) {
      const int tl = qk_token<V8>(bk, i16);
      const int T = t0 + tl;
      // B operand: (c - z) for token T, channels of group lg
      const uint32_t nz = neg_biased_zero_h2(kzero[(int64_t)T * G + lg]);
      half8 bk8[4];
      if (K8) {
        const u32x4* kp = reinterpret_cast<const u32x4*>(kbase + (int64_t)T * D + 32 * lg);
        const u32x4 c0 = kp[0], c1 = kp[1];
        const uint32_t wv[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          u32x4 o;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint32_t h2 = bytes_to_biased_h2(wv[2 * kk + (k >> 1)], k & 1);
            o[k] = h2_to_u32(u32_to_h2(h2) + u32_to_h2(nz));
          }
          bk8[kk] = u4_to_h8(o);
        }
      } else {
        const u32x4 cw = *reinterpret_cast<const u32x4*>(kbase + (int64_t)T * (D / 2) + 16 * lg);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          u32x4 o;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint32_t h2 = nibbles_to_biased_h2(cw[kk], k);
            o[k] = h2_to_u32(u32_to_h2(h2) + u32_to_h2(nz));
          }
          bk8[kk] = u4_to_h8(o);
        }
      }
      // scales of token T for the epilogue (all 4 groups)
      const u32x2 sraw = *reinterpret_cast<const u32x2*>(kscale + (int64_t)T * G);
      const float s0 = (float)u32_to_h2(sraw[0])[0], s1 = (float)u32_to_h2(sraw[0])[1];
      const float s2 = (float)u32_to_h2(sraw[1])[0], s3 = (float)u32_to_h2(sraw[1])[1];
      const bool valid = tl < nvalid;
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        f32x4 d4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) d4 = mfma16x16x32(aq[rb][kk], bk8[kk], d4);
        float s = s0 * d4[0];
        s = fmaf(s1, d4[1], s);
        s = fmaf(s2, d4[2], s);
        s = fmaf(s3, d4[3], s);
        s *= a.scale_log2;
        const bool live = 4 * rb + lg < R;
        sc[rb][bk] = valid ? (live ? s : 0.f) : -INFINITY;
      }
    }

    // ---------------- online softmax ----------------
    uint32_t p2[NRB];
    float alpha[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const float mx = row16_max(fmaxf(sc[rb][0], sc[rb][1]));
      const float mn = fmaxf(m_run[rb], mx);
      alpha[rb] = fast_exp2(m_run[rb] - mn);
      m_run[rb] = mn;
      const _Float16 p0 = (_Float16)fast_exp2(sc[rb][0] - mn);
      const _Float16 p1 = (_Float16)fast_exp2(sc[rb][1] - mn);
      l_run[rb] = fmaf(l_run[rb], alpha[rb], (float)p0 + (float)p1);
      p2[rb] = h2_to_u32(half2v{p0, p1});
    }

    // ---------------- gather P^T and alpha into the PV layout ----------------
    const int hcol = i16;                 // PV column = query head
    const int hsrc = (hcol & 3) * 16;     // QK row of that head
    u32x4 pb;
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) {
      const int src = hsrc + 4 * lg + mm;
      uint32_t v = lane_read(p2[0], src);
      if (NRB > 1) {
        const uint32_t v1 = lane_read(p2[NRB - 1], src);
        v = (hcol >> 2) ? v1 : v;
      }
      pb[mm] = hcol < R ? v : 0u;
    }
    float al = lane_read_f(alpha[0], hsrc);
    if (NRB > 1) {
      const float a1 = lane_read_f(alpha[NRB - 1], hsrc);
      al = (hcol >> 2) ? a1 : al;
    }
    const half8 bp = u4_to_h8(pb);

    // ---------------- V-hat^T operand and PV ----------------
    const int blk = t0 >> 7;
    const int tt = (t0 & 127) + 8 * lg;    // first of this lane's 8 tokens in the block
    u32x2 vz[4];
    u32x4 vs[4];
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      vz[gq] = *reinterpret_cast<const u32x2*>(vzero + (int64_t)gq * cap + t0 + 8 * lg);
      vs[gq] = *reinterpret_cast<const u32x4*>(vscale + (int64_t)gq * cap + t0 + 8 * lg);
    }
    if (nvalid < STEP) {
      // zero the scales of tokens past the end so their V-hat is exactly 0
#pragma unroll
      for (int gq = 0; gq < 4; ++gq)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t wv = vs[gq][j];
          const int ta = 8 * lg + 2 * j, tb = ta + 1;
          if (ta >= nvalid) wv &= 0xFFFF0000u;
          if (tb >= nvalid) wv &= 0x0000FFFFu;
          vs[gq][j] = wv;
        }
    }
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const int d = 16 * db + i16;
      const int gq = db >> 1;
      const uint8_t* row = vbase + ((int64_t)blk * D + d) * (V8 ? 128 : 64);
      u32x2 cw;
      if (V8) {
        cw = *reinterpret_cast<const u32x2*>(row + tt);
      } else {
        cw[0] = *reinterpret_cast<const uint32_t*>(row + tt / 2);
        cw[1] = 0;
      }
      u32x4 o;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const half2v cz = u32_to_h2(v_code_pair<V8>(cw, m)) + u32_to_h2(v_negz_pair<V8>(vz[gq], m));
        o[m] = h2_to_u32(cz * u32_to_h2(v_scale_pair<V8>(vs[gq], m)));
      }
      acc[db] = acc[db] * al;
      acc[db] = mfma16x16x32(u4_to_h8(o), bp, acc[db]);
    }
  }

  // ---- merge the 4 waves through LDS ------------------------------------------
  // layout: m[4][R], l[4][R], o[4][R][D]
  float* sm = lds;
  float* sl = lds + WAVES * R;
  float* so = lds + 2 * WAVES * R;
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const float lt = row16_sum(l_run[rb]);
    const int h = 4 * rb + lg;
    if (i16 == 0 && h < R) {
      sm[w * R + h] = m_run[rb];
      sl[w * R + h] = lt;
    }
  }
  if (i16 < R) {
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        so[(w * R + i16) * D + 16 * db + 4 * lg + v] = acc[db][v];
  }
  __syncthreads();
  const int nchunk = a.nchunk;
  for (int e = threadIdx.x; e < R * D; e += blockDim.x) {
    const int h = e / D, d = e % D;
    float M = sm[h];
#pragma unroll
    for (int ww = 1; ww < WAVES; ++ww) M = fmaxf(M, sm[ww * R + h]);
    float o = 0.f, l = 0.f;
#pragma unroll
    for (int ww = 0; ww < WAVES; ++ww) {
      const float f = fast_exp2(sm[ww * R + h] - M);
      o = fmaf(so[(ww * R + h) * D + d], f, o);
      l = fmaf(sl[ww * R + h], f, l);
    }
    float* dst = a.ws + (((int64_t)b * a.Hq + g * R + h) * nchunk + c) * (D + 2);
    dst[2 + d] = o;
    if (d == 0) {
      dst[0] = M;
      dst[1] = l;
    }
  }
}

template <int R>
__global__ void __launch_bounds__(256)
decode_split_kernel(DecodeArgs a) {
  __shared__ float lds[2 * WAVES * R + WAVES * R * D];
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  int n = a.lens[b];
  n = n < 0 ? 0 : (n > a.max_len ? a.max_len : n);
  if (c * a.chunk >= n) return;
  const bool k8 = (a.k.is8 >> g) & 1ull, v8 = (a.v.is8 >> g) & 1ull;
  if (k8) {
    if (v8) decode_body<R, true, true>(a, b, g, c, n, lds);
    else decode_body<R, true, false>(a, b, g, c, n, lds);
  } else {
    if (v8) decode_body<R, false, true>(a, b, g, c, n, lds);
    else decode_body<R, false, false>(a, b, g, c, n, lds);
  }
}

// One workgroup of D threads per (batch, query head).
__global__ void __launch_bounds__(128)
decode_merge_kernel(DecodeArgs a) {
  const int bh = blockIdx.x;
  const int b = bh / a.Hq;
  const int d = threadIdx.x;
  int n = a.lens[b];
  n = n < 0 ? 0 : (n > a.max_len ? a.max_len : n);
  const int nc = (n + a.chunk - 1) / a.chunk;
  const float* src = a.ws + (int64_t)bh * a.nchunk * (D + 2);
  float M = NEG_BIG;
  for (int c = 0; c < nc; ++c) M = fmaxf(M, src[c * (D + 2)]);
  float o = 0.f, l = 0.f;
  for (int c = 0; c < nc; ++c) {
    const float* p = src + c * (D + 2);
    const float f = fast_exp2(p[0] - M);
    l = fmaf(p[1], f, l);
    o = fmaf(p[2 + d], f, o);
  }
  const float r = l > 0.f ? o / l : 0.f;
  a.o[(int64_t)bh * D + d] = half_to_bits((_Float16)r);
}

}  // namespace

int decode_chunk_tokens(int B, int Hkv, int max_len) {
  int chunk = 128;
  const int64_t units = (int64_t)B * Hkv;
  while (chunk < 2048 && units * ((max_len + 2 * chunk - 1) / (2 * chunk)) >= 1024) chunk *= 2;
  return chunk;
}

hipError_t launch_attn_decode(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid(a.nchunk, a.k.H, a.k.B);
  switch (a.r) {
    case 1: hipLaunchKernelGGL(decode_split_kernel<1>, grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL(decode_split_kernel<2>, grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL(decode_split_kernel<4>, grid, dim3(256), 0, s, a); break;
    case 8: hipLaunchKernelGGL(decode_split_kernel<8>, grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_kernel, dim3(a.k.B * a.Hq), dim3(128), 0, s, a);
  return hipGetLastError();
}

}  // namespace taq
