// Causal prefill attention over the grouped-quantized KV cache.
//
// Method: scaled dot-product attention (Space Bunny inference-stack article,
// m.xxqk.cn, section 3.1) computed tile by tile so the L x L score matrix is
// never formed, carrying each row's running maximum and normaliser from tile to
// tile ("分块稀疏注意力与KV Cache量化：长文本推理显存优化实践", xdnf.cn, sections
// 2.1-2.2); K/V tiles are dequantised while they are staged (section 1.3) and
// tiles dropped by causality or by the block mask are never loaded (section
// 2.3; prefill is compute-bound and skips aggressively, section 5.3).
//
// Work decomposition (gfx950):
//  * a 512-thread workgroup (8 waves) owns BQ = 256 / r query rows of all
//    r = Hq/Hkv query heads that share one KV head, so every K/V tile is
//    fetched and dequantised once for r * BQ = 256 (head, row) pairs; wave w
//    takes head w % r and the 32 rows (w / r) * 32 .. +31;
//  * the key loop runs in tiles of 64 keys through two LDS stages: while
//    tile i is consumed, tile i+1 is dequantised into the other stage and
//    tile i+2 is fetched from HBM into registers (one barrier per tile);
//  * both contractions use v_mfma_f32_32x32x16_f16 in transposed form:
//    S^T = K-hat Q^T (A = K-hat tile from LDS, B = Q held in registers) and
//    O^T += V-hat^T P^T (A = V-hat^T tile from LDS, B = P straight from the
//    S^T accumulator), so every lane owns one query row for the whole loop and
//    the softmax needs only one cross-lane exchange per tile;
//  * the workgroup order runs the longest causal rows first.
#include "taq_internal.h"
#include "device_common.h"

namespace taq {
namespace {

constexpr int D = 128;
constexpr int KT = 64;                 // keys per tile
constexpr int NWAVE = 8;
constexpr int NT = 64 * NWAVE;
constexpr int KS_STRIDE = D * 2 + 16;  // bytes per K-hat row in LDS (padded)
constexpr int VS_STRIDE = KT * 2 + 16; // bytes per V-hat^T row in LDS (padded)
constexpr int LDS_K = KT * KS_STRIDE;
constexpr int LDS_V = D * VS_STRIDE;
constexpr int LDS_STAGE = LDS_K + LDS_V;   // one tile (K-hat and V-hat^T)
constexpr float NEG_BIG = -1.0e30f;

// Natural-order nibble pair: channels / keys 2j and 2j+1 of the 8 nibbles in w.
__device__ __forceinline__ uint32_t nib_pair_natural(uint32_t w, int j) {
  const uint32_t lo = __builtin_amdgcn_ubfe(w, 8 * j, 4);
  const uint32_t hi = __builtin_amdgcn_ubfe(w, 8 * j + 4, 4);
  return (lo | (hi << 16)) | 0x64006400u;
}

// Registers holding one tile's raw codes and metadata for this thread.
struct Staged {
  u32x4 kc;        // K codes: 16 channels (int8: 16 B; int4: first 8 B used)
  uint32_t kz;     // K zero byte
  uint32_t ks;     // K scale bits
  u32x4 vc;        // V codes: 16 keys of one channel
  u32x4 vz;        // V zeros of those 16 keys
  u32x4 vs0, vs1;  // V scales of those 16 keys
};

struct TileCtx {
  const uint8_t* kbase;
  const uint8_t* vbase;
  const uint16_t* kscale;
  const uint8_t* kzero;
  const uint16_t* vscale;
  const uint8_t* vzero;
  int cap;
};

template <bool K8, bool V8>
__device__ __forceinline__ void stage_load(const TileCtx& c, int kt0, int tid, Staged& s) {
  // K: thread -> (key, group, half): 16 channels
  {
    const int unit = tid >> 1, half = tid & 1;
    const int key = kt0 + (unit >> 2), grp = unit & 3;
    if (K8) {
      s.kc = *reinterpret_cast<const u32x4*>(c.kbase + (int64_t)key * D + 32 * grp + 16 * half);
    } else {
      const u32x2 t = *reinterpret_cast<const u32x2*>(c.kbase + (int64_t)key * (D / 2) + 16 * grp + 8 * half);
      s.kc = u32x4{t[0], t[1], 0u, 0u};
    }
    s.kz = c.kzero[(int64_t)key * 4 + grp];
    s.ks = c.kscale[(int64_t)key * 4 + grp];
  }
  // V: thread -> (channel d, quarter q): keys 16q .. 16q+15 of the tile
  {
    const int d = tid >> 2, q = tid & 3;
    const int grp = d >> 5;
    const int key = kt0 + 16 * q;
    const int blk = key >> 5, kin = key & 31;
    const uint8_t* row = c.vbase + ((int64_t)blk * D + d) * (V8 ? 32 : 16);
    if (V8) {
      s.vc = *reinterpret_cast<const u32x4*>(row + kin);
    } else {
      const u32x2 t = *reinterpret_cast<const u32x2*>(row + kin / 2);
      s.vc = u32x4{t[0], t[1], 0u, 0u};
    }
    s.vz = *reinterpret_cast<const u32x4*>(c.vzero + (int64_t)grp * c.cap + kt0 + 16 * q);
    const u32x4* sp = reinterpret_cast<const u32x4*>(c.vscale + (int64_t)grp * c.cap + kt0 + 16 * q);
    s.vs0 = sp[0];
    s.vs1 = sp[1];
  }
}

// Dequantise the staged registers into LDS.  Keys at or beyond n get a zero
// scale so that their (never used) V-hat entries are exactly 0 and finite.
template <bool K8, bool V8>
__device__ __forceinline__ void stage_store(const Staged& s, int kt0, int n, int tid,
                                            char* lds) {
  {
    const int unit = tid >> 1, half = tid & 1;
    const int key = unit >> 2, grp = unit & 3;
    const half2v nz = u32_to_h2(neg_biased_zero_h2(s.kz));
    const _Float16 sc = bits_to_half((uint16_t)s.ks);
    const half2v s2 = half2v{sc, sc};
    u32x4 o0, o1;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t c2;
      if (K8) c2 = bytes_to_biased_h2(s.kc[j >> 1], j & 1);
      else c2 = nib_pair_natural(s.kc[j >> 2], j & 3);
      const uint32_t v = h2_to_u32((u32_to_h2(c2) + nz) * s2);
      if (j < 4) o0[j] = v; else o1[j - 4] = v;
    }
    u32x4* dst = reinterpret_cast<u32x4*>(lds + key * KS_STRIDE + (32 * grp + 16 * half) * 2);
    dst[0] = o0;
    dst[1] = o1;
  }
  {
    const int d = tid >> 2, q = tid & 3;
    u32x4 o0, o1;
#pragma unroll
    for (int j = 0; j < 8; ++j) {  // pair j = keys 16q + 2j, +1
      uint32_t c2;
      if (V8) c2 = bytes_to_biased_h2(s.vc[j >> 1], j & 1);
      else c2 = nib_pair_natural(s.vc[j >> 2], j & 3);
      const uint32_t nz = perm_b32(0xE4E4E4E4u, s.vz[j >> 1], (j & 1) ? 0x04030402u : 0x04010400u);
      uint32_t sc = j < 4 ? s.vs0[j] : s.vs1[j - 4];
      const int k0 = kt0 + 16 * q + 2 * j;
      if (k0 >= n) sc &= 0xFFFF0000u;
      if (k0 + 1 >= n) sc &= 0x0000FFFFu;
      const uint32_t v = h2_to_u32((u32_to_h2(c2) + u32_to_h2(nz)) * u32_to_h2(sc));
      if (j < 4) o0[j] = v; else o1[j - 4] = v;
    }
    u32x4* dst = reinterpret_cast<u32x4*>(lds + LDS_K + d * VS_STRIDE + 32 * q);
    dst[0] = o0;
    dst[1] = o1;
  }
}

__device__ __forceinline__ bool mask_keep(const PrefillArgs& a, const uint8_t* mb, int qt, int kt) {
  return mb == nullptr || mb[(int64_t)qt * a.mask_nk + kt] != 0;
}

template <int R, bool K8, bool V8>
__device__ void prefill_body(const PrefillArgs& a, int b, int g, int qblk, int n, char* lds) {
  constexpr int BQ = 32 * (NWAVE / R);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int i32 = lane & 31, hb = lane >> 5;
  const int hl = w % R, rblk = w / R;
  const int hq = g * R + hl;
  const int q0 = qblk * BQ;
  const int q0w = q0 + 32 * rblk;
  const int row = q0w + i32;
  const bool row_live = row < n;

  TileCtx c;
  c.kbase = a.k.codes + (int64_t)b * a.k.bstride + a.k.hoff[g];
  c.vbase = a.v.codes + (int64_t)b * a.v.bstride + a.v.hoff[g];
  c.kscale = a.k.scales + ((int64_t)b * a.k.H + g) * a.k.cap * 4;
  c.kzero = a.k.zeros + ((int64_t)b * a.k.H + g) * a.k.cap * 4;
  c.vscale = a.v.scales + ((int64_t)b * a.v.H + g) * 4 * (int64_t)a.v.cap;
  c.vzero = a.v.zeros + ((int64_t)b * a.v.H + g) * 4 * (int64_t)a.v.cap;
  c.cap = a.k.cap;

  const uint8_t* mb = a.mask ? a.mask + (int64_t)b * a.mask_sb + (int64_t)g * a.mask_sh : nullptr;

  // Q row of this lane (B operand of S^T): channels 16ks + 8hb .. +7
  half8 qreg[8];
  {
    const uint16_t* qp = a.q + (((int64_t)b * a.Hq + hq) * a.L + row) * D + 8 * hb;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row < a.L) v = *reinterpret_cast<const u32x4*>(qp + 16 * ks);
      qreg[ks] = u4_to_h8(v);
    }
  }

  // rows of the workgroup that can see any key, and key range
  const int wg_last = min(q0 + BQ, n) - 1;            // last live row of the WG
  const int w_last = min(q0w + 31, n - 1);            // last live row of this wave
                                                      // (meaningful when q0w < n)
  const int nkt = wg_last >= 0 ? wg_last / KT + 1 : 0;
  const int qt_first = q0 >> 7, qt_last = wg_last >= 0 ? (wg_last >> 7) : -1;

  auto wg_needs = [&](int kt) -> bool {
    const int kt128 = (kt * KT) >> 7;
    for (int qt = qt_first; qt <= qt_last; ++qt)
      if (qt >= kt128 && mask_keep(a, mb, qt, kt128)) return true;
    return false;
  };
  auto next_tile = [&](int kt) -> int {
    while (kt < nkt && !wg_needs(kt)) ++kt;
    return kt;
  };

  float m_run = NEG_BIG, l_run = 0.f;
  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[db][v] = 0.f;

  const float c_log2 = a.scale_log2;   // > 0 (checked on the host)

  // ---- double-buffered LDS pipeline over the needed KV tiles -----------------
  // Iteration i: one barrier (tile i is in LDS; every wave is done with tile
  // i-1), then dequantise tile i+1 from registers into the other buffer, issue
  // the global loads of tile i+2, and consume tile i.  The dequantisation and
  // the matrix work of one iteration are independent, so they interleave.
  int cur = next_tile(0);
  Staged st;
  if (cur < nkt) {
    stage_load<K8, V8>(c, cur * KT, tid, st);
    stage_store<K8, V8>(st, cur * KT, n, tid, lds);
  }
  int nxt = cur < nkt ? next_tile(cur + 1) : nkt;
  if (nxt < nkt) stage_load<K8, V8>(c, nxt * KT, tid, st);
  int bi = 0;
  while (cur < nkt) {
    __syncthreads();
    if (nxt < nkt) stage_store<K8, V8>(st, nxt * KT, n, tid, lds + (bi ^ 1) * LDS_STAGE);
    const int nn = nxt < nkt ? next_tile(nxt + 1) : nkt;
    if (nn < nkt) stage_load<K8, V8>(c, nn * KT, tid, st);

    const int kt0 = cur * KT;
    const uint8_t* ks_lds = reinterpret_cast<const uint8_t*>(lds + bi * LDS_STAGE);
    const uint8_t* vs_lds = ks_lds + LDS_K;
    const bool wave_needs =
        q0w < n && w_last >= kt0 && mask_keep(a, mb, q0w >> 7, kt0 >> 7);
    if (wave_needs) {
      // ---- S^T = K-hat Q^T ----
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) s[kb][v] = 0.f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const u32x4 kv = *reinterpret_cast<const u32x4*>(
              ks_lds + (32 * kb + i32) * KS_STRIDE + (16 * ks + 8 * hb) * 2);
          s[kb] = mfma32x32x16(u4_to_h8(kv), qreg[ks], s[kb]);
        }
      }
      // ---- mask, online softmax ----
      // Scores stay unscaled; the scale is folded into the exponent's FMA.
      const bool need_mask = (kt0 + KT - 1 > q0w) || (kt0 + KT > n) || (q0w + 31 >= n);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = kt0 + 32 * kb + 8 * (v >> 2) + 4 * hb + (v & 3);
            if (key > row || key >= n || !row_live) s[kb][v] = -INFINITY;
          }
      }
      float mx = s[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb][v]);
      mx = fmaxf(mx, lane_read_f(mx, lane ^ 32)) * c_log2;
      // The running maximum only moves when the tile maximum exceeds it by
      // more than 8 (log2 units): weights stay below 2^8, exact enough in
      // fp16, and the accumulator is rescaled only on those tiles.
      const bool move = mx > m_run + 8.f;
      const float mn = move ? mx : m_run;
      const float alpha = move ? fast_exp2(m_run - mn) : 1.f;
      m_run = mn;
      half8 p[4];  // PV k-steps (kb, half)
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          half8 ph;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            ph[e] = (_Float16)fast_exp2(fmaf(s[kb][8 * hf + e], c_log2, -mn));
#pragma unroll
          for (int e = 0; e < 8; e += 2)
            lsum = __builtin_amdgcn_fdot2(half2v{ph[e], ph[e + 1]},
                                          half2v{(_Float16)1.f, (_Float16)1.f}, lsum, false);
          p[2 * kb + hf] = ph;
        }
      l_run = fmaf(l_run, alpha, lsum);
      if (__any(move)) {
        asm volatile("" ::: "memory");   // keep this a real (rare) branch
#pragma unroll
        for (int db = 0; db < 4; ++db) o[db] = o[db] * alpha;
      }
      // ---- O^T += V-hat^T P^T ----
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const uint8_t* vr = vs_lds + (32 * db + i32) * VS_STRIDE;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int kb = kk >> 1, hf = kk & 1;
          const int kbase = 32 * kb + 16 * hf + 4 * hb;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vr + kbase * 2);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vr + (kbase + 8) * 2);
          const u32x4 av = {lo[0], lo[1], hi[0], hi[1]};
          o[db] = mfma32x32x16(u4_to_h8(av), p[kk], o[db]);
        }
      }
    }
    cur = nxt;
    nxt = nn;
    bi ^= 1;
  }

  // ---- epilogue ----
  const float lt = l_run + lane_read_f(l_run, lane ^ 32);
  const float inv = (row_live && lt > 0.f) ? 1.f / lt : 0.f;
  if (row < a.L) {
    uint16_t* op = a.o + (((int64_t)b * a.Hq + hq) * a.L + row) * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int vq = 0; vq < 4; ++vq) {
        const int d0 = 32 * db + 8 * vq + 4 * hb;
        half4v hv;
#pragma unroll
        for (int e = 0; e < 4; ++e) hv[e] = (_Float16)(o[db][4 * vq + e] * inv);
        *reinterpret_cast<half4v*>(op + d0) = hv;
      }
  }
}

// 1-D grid.  Consecutive workgroup ids go round-robin to the 8 XCDs, so with
// the KV head as the fastest index every XCD keeps serving the same KV heads
// (its L2 holds their K/V tiles); query blocks run longest-first.
template <int R>
__global__ void __launch_bounds__(NT)
prefill_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[2 * LDS_STAGE];
  const int H = a.k.H, B = a.k.B;
  const int id = blockIdx.x;
  const int g = id % H;
  const int rest = id / H;
  const int b = rest % B;
  const int qblk = a.n_qblk - 1 - rest / B;
  int n = a.lens[b];
  n = n < 0 ? 0 : (n > a.L ? a.L : n);
  const bool k8 = (a.k.is8 >> g) & 1ull, v8 = (a.v.is8 >> g) & 1ull;
  if (k8) {
    if (v8) prefill_body<R, true, true>(a, b, g, qblk, n, lds);
    else prefill_body<R, true, false>(a, b, g, qblk, n, lds);
  } else {
    if (v8) prefill_body<R, false, true>(a, b, g, qblk, n, lds);
    else prefill_body<R, false, false>(a, b, g, qblk, n, lds);
  }
}

}  // namespace

hipError_t launch_attn_prefill(const PrefillArgs& a, hipStream_t s) {
  const dim3 grid(a.n_qblk * a.k.H * a.k.B);
  switch (a.r) {
    case 1: hipLaunchKernelGGL(prefill_kernel<1>, grid, dim3(NT), 0, s, a); break;
    case 2: hipLaunchKernelGGL(prefill_kernel<2>, grid, dim3(NT), 0, s, a); break;
    case 4: hipLaunchKernelGGL(prefill_kernel<4>, grid, dim3(NT), 0, s, a); break;
    case 8: hipLaunchKernelGGL(prefill_kernel<8>, grid, dim3(NT), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace taq
