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
//  * the key loop runs in tiles of 64 keys through three LDS stages as a
//    software pipeline: the QK^T MFMAs of tile j+1 interleave with the
//    softmax of tile j, and the PV MFMAs of tile j with the dequantisation of
//    tile j+2; tile j+3 is fetched into registers (one barrier per tile);
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
// key-range partial of one (split, b, query head, row): m, l, 2 pad, acc[D]
// (16-byte aligned records)
constexpr int PART_REC = D + 4;
#ifndef TAQ_PREFILL_READ_AHEAD
#define TAQ_PREFILL_READ_AHEAD 3
#endif
// LDS operand reads issued this many matrix instructions ahead of their use.
constexpr int PF_RA = TAQ_PREFILL_READ_AHEAD;

// V-hat^T rows hold the keys of each 16-key group in the order that the PV
// operand wants them: key 16g + 8a + 4h + c (a, h in {0,1}, c in 0..3) sits at
// column 16g + 8h + 4a + c.  A lane of row-half h then finds the 8 keys it
// feeds to one MFMA k-step contiguous, one 16-byte LDS read.  Pair j (keys
// 2j, 2j+1 of a group) lands in 32-bit column word vslot(j).
__host__ __device__ constexpr int vslot(int j) { return 4 * ((j >> 1) & 1) + 2 * (j >> 2) + (j & 1); }

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

// Tile-invariant addressing: uniform (scalar) base pointers of this (batch,
// KV head) and the per-thread offsets of its share of a tile, so a tile load
// is a scalar base plus a fixed 32-bit lane offset.
struct TileCtx {
  const uint8_t* kbase;
  const uint8_t* vbase;
  const uint16_t* kscale;
  const uint8_t* kzero;
  const uint16_t* vscale;
  const uint8_t* vzero;
  uint32_t k_off;     // K codes, bytes from the tile's first key row
  uint32_t km_off;    // K scale / zero index from the tile's first key
  uint32_t v_off;     // V codes, bytes from the tile's first 32-key block
  uint32_t vm_off;    // V scale / zero index from the tile's first key
};

// Staging threads: K -> (key = unit / 4, group = unit % 4, half) with unit =
// tid / 2, 16 channels each; V -> (channel d = tid / 4, quarter q = tid % 4),
// keys 16q .. 16q+15 of the tile.
template <bool K8, bool V8>
__device__ __forceinline__ void tile_ctx_offsets(TileCtx& c, int tid, int cap) {
  const int unit = tid >> 1, half = tid & 1;
  const int kkey = unit >> 2, kgrp = unit & 3;
  c.k_off = (uint32_t)(kkey * (K8 ? D : D / 2) + (K8 ? 32 : 16) * kgrp + (K8 ? 16 : 8) * half);
  c.km_off = (uint32_t)(kkey * 4 + kgrp);
  const int d = tid >> 2, q = tid & 3;
  const int rowb = V8 ? 32 : 16;
  // key 16q of the tile lies in 32-key block q / 2 at position 16 (q % 2)
  c.v_off = (uint32_t)(((q >> 1) * D + d) * rowb + (V8 ? 16 : 8) * (q & 1));
  c.vm_off = (uint32_t)((d >> 5) * cap + 16 * q);
}

template <bool K8, bool V8>
__device__ __forceinline__ void stage_load(const TileCtx& c, int kt0, Staged& s) {
  {
    const uint8_t* kb = c.kbase + (int64_t)kt0 * (K8 ? D : D / 2);
    if (K8) {
      s.kc = *reinterpret_cast<const u32x4*>(kb + c.k_off);
    } else {
      const u32x2 t = *reinterpret_cast<const u32x2*>(kb + c.k_off);
      s.kc = u32x4{t[0], t[1], 0u, 0u};
    }
    s.kz = (c.kzero + (int64_t)kt0 * 4)[c.km_off];
    s.ks = (c.kscale + (int64_t)kt0 * 4)[c.km_off];
  }
  {
    const uint8_t* vb = c.vbase + (int64_t)(kt0 >> 5) * D * (V8 ? 32 : 16);
    if (V8) {
      s.vc = *reinterpret_cast<const u32x4*>(vb + c.v_off);
    } else {
      const u32x2 t = *reinterpret_cast<const u32x2*>(vb + c.v_off);
      s.vc = u32x4{t[0], t[1], 0u, 0u};
    }
    s.vz = *reinterpret_cast<const u32x4*>(c.vzero + kt0 + c.vm_off);
    const u32x4* sp = reinterpret_cast<const u32x4*>(c.vscale + kt0 + c.vm_off);
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
      if (vslot(j) < 4) o0[vslot(j)] = v; else o1[vslot(j) - 4] = v;
    }
    u32x4* dst = reinterpret_cast<u32x4*>(lds + LDS_K + d * VS_STRIDE + 32 * q);
    dst[0] = o0;
    dst[1] = o1;
  }
}

// The same dequantisation as stage_store, one fp16 pair at a time and split
// in two steps (code minus zero point, then times the scale) so that the
// steps of consecutive pairs can be interleaved with matrix instructions.
// K: pair j (0..7) = channels 16*half + 2j, +1 of the thread's (key, group);
// V: pair j = keys 16q + 2j, +1 of the thread's channel.
template <bool K8>
__device__ __forceinline__ uint32_t k_centered(const Staged& s, int j, half2v nz) {
  const uint32_t c2 = K8 ? bytes_to_biased_h2(s.kc[j >> 1], j & 1) : nib_pair_natural(s.kc[j >> 2], j & 3);
  return h2_to_u32(u32_to_h2(c2) + nz);
}
template <bool V8>
__device__ __forceinline__ uint32_t v_centered(const Staged& s, int j) {
  const uint32_t c2 = V8 ? bytes_to_biased_h2(s.vc[j >> 1], j & 1) : nib_pair_natural(s.vc[j >> 2], j & 3);
  const uint32_t nz = perm_b32(vconst(0xE4E4E4E4u), s.vz[j >> 1], (j & 1) ? 0x04030402u : 0x04010400u);
  return h2_to_u32(u32_to_h2(c2) + u32_to_h2(nz));
}
__device__ __forceinline__ uint32_t v_scales(const Staged& s, int j) {
  return j < 4 ? s.vs0[j] : s.vs1[j - 4];
}
__device__ __forceinline__ uint32_t h2_mul(uint32_t a, uint32_t b) {
  return h2_to_u32(u32_to_h2(a) * u32_to_h2(b));
}

// Zero the staged V scales of keys at or beyond n (keys key0 .. key0+15 of
// this thread), so their V-hat entries are exactly 0 whatever the cache holds
// past the sequence end.
__device__ __forceinline__ void zero_tail_scales(Staged& s, int key0, int n) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int k0 = key0 + 2 * j;
    const uint32_t keep = (k0 < n ? 0x0000FFFFu : 0u) | (k0 + 1 < n ? 0xFFFF0000u : 0u);
    if (j < 4) s.vs0[j] &= keep; else s.vs1[j - 4] &= keep;
  }
}

__device__ __forceinline__ bool mask_keep(const PrefillArgs& a, const uint8_t* mb, int qt, int kt) {
  return mb == nullptr || mb[(int64_t)qt * a.mask_nk + kt] != 0;
}

template <int R, bool K8, bool V8>
__device__ void prefill_body(const PrefillArgs& a, int b, int g, int qblk, int split, int n,
                             char* lds) {
  constexpr int BQ = 32 * (NWAVE / R);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int i32 = lane & 31, hb = lane >> 5;
  const int hl = w % R, rblk = w / R;
  const int hq = g * R + hl;
  const int q0 = qblk * BQ;
  const int q0w = q0 + 32 * rblk;
  const int row = q0w + i32;             // row of q / o
  // Position of row 0 in the sequence: 0 for a whole-sequence prefill; for a
  // chunk of Lq new rows whose keys are already in the cache, n - Lq (rows
  // at negative positions are padding).  Causality and the tile mask work
  // on positions.
  const int qoff = a.chunk ? n - a.Lq : 0;
  const int pos = row + qoff;
  const int p0w = q0w + qoff;            // position of the wave's first row
  const bool row_live = row < a.Lq && pos >= 0 && pos < n;

  TileCtx c;
  c.kbase = a.k.codes + (int64_t)b * a.k.bstride + a.k.hoff[g];
  c.vbase = a.v.codes + (int64_t)b * a.v.bstride + a.v.hoff[g];
  c.kscale = a.k.scales + ((int64_t)b * a.k.H + g) * a.k.cap * 4;
  c.kzero = a.k.zeros + ((int64_t)b * a.k.H + g) * a.k.cap * 4;
  c.vscale = a.v.scales + ((int64_t)b * a.v.H + g) * 4 * (int64_t)a.v.cap;
  c.vzero = a.v.zeros + ((int64_t)b * a.v.H + g) * 4 * (int64_t)a.v.cap;
  tile_ctx_offsets<K8, V8>(c, tid, a.k.cap);

  const uint8_t* mb = a.mask ? a.mask + (int64_t)b * a.mask_sb + (int64_t)g * a.mask_sh : nullptr;

  // Q row of this lane (B operand of S^T): channels 16ks + 8hb .. +7
  half8 qreg[8];
  {
    const uint16_t* qp = a.q + (((int64_t)b * a.Hq + hq) * a.Lq + row) * D + 8 * hb;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row < a.Lq) v = *reinterpret_cast<const u32x4*>(qp + 16 * ks);
      qreg[ks] = u4_to_h8(v);
    }
  }

  // rows of the workgroup that can see any key, and key range
  // last live position of the workgroup
  const int wg_last = min(min(q0 + BQ, a.Lq) - 1 + qoff, n - 1);
  const int nkt_all = wg_last >= 0 ? wg_last / KT + 1 : 0;
  // key-range split: this workgroup takes tiles [kt_lo, nkt) of the query
  // block's range (equal shares; the partials are merged afterwards)
  const int per = (nkt_all + a.nsplit - 1) / a.nsplit;
  const int kt_lo = min(split * per, nkt_all);
  const int nkt = min(kt_lo + per, nkt_all);
  const int qt_first = max(q0 + qoff, 0) >> 7, qt_last = wg_last >= 0 ? (wg_last >> 7) : -1;

  auto wg_needs = [&](int kt) -> bool {
    const int kt128 = (kt * KT) >> 7;
    for (int qt = qt_first; qt <= qt_last; ++qt)
      if (qt >= kt128 && mask_keep(a, mb, qt, kt128)) return true;
    return false;
  };
  auto next_tile = [&](int kt) -> int {
    if (mb == nullptr) return kt;   // dense: every tile below nkt is needed
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
  // this lane's 128-row query tile (clamped, so lanes past the last row never
  // index beyond the mask's ceil(max_seq_len / 128) tile rows)
  const int qt_l = min(max(pos, 0), a.L - 1) >> 7;

  // ---- LDS stage helpers ---------------------------------------------------------
  auto stage_ptr = [&](int j) -> char* { return lds + (j % 3) * LDS_STAGE; };
  // ring stage after / before stage x (x in 0..2)
  auto ring_next = [](int x) { return x == 2 ? 0 : x + 1; };
  auto ring_prev = [](int x) { return x == 0 ? 2 : x - 1; };
  auto stage_at = [&](int x) -> char* { return lds + x * LDS_STAGE; };
  // S^T = K-hat Q^T for the tile in stage j (16 MFMAs)
  auto qk = [&](int j, f32x16* S) {
    const uint8_t* kl = reinterpret_cast<const uint8_t*>(stage_ptr(j));
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) S[kb][v] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const u32x4 kv = *reinterpret_cast<const u32x4*>(
            kl + (32 * kb + i32) * KS_STRIDE + (16 * ks + 8 * hb) * 2);
        S[kb] = mfma32x32x16(u4_to_h8(kv), qreg[ks], S[kb]);
      }
    }
  };
  // causal / length / dead-row / per-wave mask of tile kt on S (only when needed)
  auto mask_tile = [&](int kt, f32x16* S) {
    const int kt0 = kt * KT;
    const bool keep = mask_keep(a, mb, qt_l, kt0 >> 7);
    const bool need = __any(!keep) || (kt0 + KT - 1 > p0w) || (kt0 + KT > n) || (p0w + 31 >= n) ||
                      (p0w < 0) || (q0w + 31 >= a.Lq);
    if (need) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = kt0 + 32 * kb + 8 * (v >> 2) + 4 * hb + (v & 3);
          if (!keep || key > pos || key >= n || !row_live) S[kb][v] = -INFINITY;
        }
    }
  };

  // ---- software pipeline over the workgroup's KV tiles -------------------------
  // Tiles t_0, t_1, ... (causal and mask order) go through three LDS stages.
  // Iteration j (one barrier): the QK^T MFMAs of tile j+1 run interleaved with
  // the softmax of tile j, then the PV MFMAs of tile j run interleaved with the
  // dequantisation of tile j+2 into the third stage; tile j+3 is fetched from
  // HBM into registers.  Every wave walks the same tiles; rows a tile does not
  // reach are masked, so the loop has no per-wave branches.
  const int t0_ = next_tile(kt_lo);
  if (t0_ < nkt) {
    const int t1_ = next_tile(t0_ + 1);
    const int t2_ = t1_ < nkt ? next_tile(t1_ + 1) : nkt;
    Staged st;
    stage_load<K8, V8>(c, t0_ * KT, st);
    stage_store<K8, V8>(st, t0_ * KT, n, tid, stage_ptr(0));
    stage_load<K8, V8>(c, (t1_ < nkt ? t1_ : t0_) * KT, st);
    stage_store<K8, V8>(st, (t1_ < nkt ? t1_ : t0_) * KT, n, tid, stage_ptr(1));
    stage_load<K8, V8>(c, (t2_ < nkt ? t2_ : t0_) * KT, st);
    __syncthreads();
    f32x16 S0[2], S1[2];
    qk(0, S0);
    int tj = t0_, tj1 = t1_, tj2 = t2_;
    int j3 = 0;   // ring stage of tile j

    auto iteration = [&](f32x16* Sc, f32x16* Sn) {
      const int tj3 = tj2 < nkt ? next_tile(tj2 + 1) : nkt;
      __syncthreads();
      mask_tile(tj, Sc);
      // --- softmax statistics of tile j ---
      float mx = Sc[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, Sc[kb][v]);
      mx = fmaxf(mx, lane_read_f(mx, lane ^ 32)) * c_log2;
      // The running maximum only moves when the tile maximum exceeds it by
      // more than 8 (log2 units): weights stay below 2^8, exact enough in
      // fp16, and the accumulator is rescaled only on those tiles.
      const bool move = mx > m_run + 8.f;
      const float mn = move ? mx : m_run;
      const float alpha = move ? fast_exp2(m_run - mn) : 1.f;
      m_run = mn;
      // Rescale before the interleaved blocks, so that no branch separates the
      // weights of tile j from the PV block that consumes them.
      if (__any(move)) {
        asm volatile("" ::: "memory");   // keep this a real (rare) branch
#pragma unroll
        for (int db = 0; db < 4; ++db) o[db] = o[db] * alpha;
      }

      // The staged tile j+2 (past the last tile the staged registers repeat a
      // valid tile): zero its V scales past the sequence end.  Both rare
      // branches sit here so no branch splits the interleaved blocks below.
      const int skt0 = (tj2 < nkt ? tj2 : t0_) * KT;
      if (skt0 + KT > n) {
        asm volatile("" ::: "memory");
        zero_tail_scales(st, skt0 + 16 * (tid & 3), n);
      }

      // --- QK^T(j+1) interleaved with the weights of tile j ---
      // MFMA i uses accumulator kb = i % 2 and k-step ks = i / 2; its LDS
      // operand is read PF_RA MFMAs ahead; the weights of elements 2i, 2i+1 of
      // S(j) are computed behind it.  Past the last tile the MFMAs recompute
      // a resident stage (result unused).
      const uint8_t* kl = reinterpret_cast<const uint8_t*>(stage_at(ring_next(j3)));
      auto kread = [&](int i) -> u32x4 {
        const int kb = i & 1, ks = i >> 1;
        return *reinterpret_cast<const u32x4*>(kl + (32 * kb + i32) * KS_STRIDE + (16 * ks + 8 * hb) * 2);
      };
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) Sn[kb][v] = 0.f;
      half8 pk[4];  // PV k-steps (kb, half)
      float lsum = 0.f;
      const half2v ones = half2v{(_Float16)1.f, (_Float16)1.f};
      // Slice i: weights of elements 2i, 2i+1 in fp32; the fp16 rounding and
      // the row sum of pair i-1 (one slice later, behind the MFMA, so no
      // dependent instruction follows its producer directly).
      float e0 = 0.f, e1 = 0.f;
      u32x4 kv[16];
#pragma unroll
      for (int i = 0; i < PF_RA; ++i) kv[i] = kread(i);
#pragma unroll
      for (int i = 0; i <= 16; ++i) {
        if (i < 16) {
          if (i + PF_RA < 16) kv[i + PF_RA] = kread(i + PF_RA);
          Sn[i & 1] = mfma32x32x16(u4_to_h8(kv[i]), qreg[i >> 1], Sn[i & 1]);
        }
        half2v hp;
        if (i > 0) {
          const int ip = i - 1, kbp = ip >> 3, vp = 2 * (ip & 7);
          hp = half2v{(_Float16)e0, (_Float16)e1};
          pk[2 * kbp + (vp >> 3)][vp & 7] = hp[0];
          pk[2 * kbp + (vp >> 3)][(vp & 7) + 1] = hp[1];
        }
        if (i < 16) {
          const int kb = i >> 3, v = 2 * (i & 7);
          e0 = fast_exp2(fmaf(Sc[kb][v], c_log2, -mn));
          e1 = fast_exp2(fmaf(Sc[kb][v + 1], c_log2, -mn));
        }
        if (i > 0) lsum = __builtin_amdgcn_fdot2(hp, ones, lsum, false);
        __builtin_amdgcn_sched_barrier(0);
      }
      l_run = fmaf(l_run, alpha, lsum);

      // --- PV(j) interleaved with the dequantisation of tile j+2 ---
      // MFMA i uses accumulator db = i % 4 and k-step kk = i / 4; pair i of the
      // staged tile (K pairs 0..7, then V pairs 0..7) is dequantised behind it.
      {
        const uint8_t* vl = reinterpret_cast<const uint8_t*>(stage_at(j3)) + LDS_K;
        auto vread = [&](int i) -> u32x4 {
          const int db = i & 3, kk = i >> 2;
          return *reinterpret_cast<const u32x4*>(vl + (32 * db + i32) * VS_STRIDE + (16 * kk + 8 * hb) * 2);
        };
        char* sdst = stage_at(ring_prev(j3));
        const int unit = tid >> 1, khalf = tid & 1;
        const int kkey = unit >> 2, kgrp = unit & 3;
        const int vd = tid >> 2, vq = tid & 3;
        const half2v knz = u32_to_h2(neg_biased_zero_h2(st.kz));
        const _Float16 ksc = bits_to_half((uint16_t)st.ks);
        const half2v ks2 = half2v{ksc, ksc};
        const uint32_t ks2u = h2_to_u32(ks2);
        u32x4 ko0, ko1, vo0, vo1;
        u32x4 av[16];
#pragma unroll
        for (int i = 0; i < PF_RA; ++i) av[i] = vread(i);
        // Slice i: MFMA i, the scaling of pair i-1 and the centring of pair i.
        uint32_t cen = 0;
#pragma unroll
        for (int i = 0; i <= 16; ++i) {
          if (i < 16) {
            if (i + PF_RA < 16) av[i + PF_RA] = vread(i + PF_RA);
            o[i & 3] = mfma32x32x16(u4_to_h8(av[i]), pk[i >> 2], o[i & 3]);
          }
          if (i > 0) {
            const int ip = i - 1;
            if (ip < 8) {
              const uint32_t w = h2_mul(cen, ks2u);
              if (ip < 4) ko0[ip] = w; else ko1[ip - 4] = w;
            } else {
              const int jv = ip - 8;
              const uint32_t w = h2_mul(cen, v_scales(st, jv));
              if (vslot(jv) < 4) vo0[vslot(jv)] = w; else vo1[vslot(jv) - 4] = w;
            }
          }
          if (i < 8) cen = k_centered<K8>(st, i, knz);
          else if (i < 16) cen = v_centered<V8>(st, i - 8);
          if (i == 8) {
            u32x4* kd = reinterpret_cast<u32x4*>(sdst + kkey * KS_STRIDE + (32 * kgrp + 16 * khalf) * 2);
            kd[0] = ko0;
            kd[1] = ko1;
          }
          if (i == 16) {
            u32x4* vdst = reinterpret_cast<u32x4*>(sdst + LDS_K + vd * VS_STRIDE + 32 * vq);
            vdst[0] = vo0;
            vdst[1] = vo1;
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      stage_load<K8, V8>(c, (tj3 < nkt ? tj3 : t0_) * KT, st);
      tj = tj1; tj1 = tj2; tj2 = tj3;
      j3 = ring_next(j3);
    };

    while (true) {
      iteration(S0, S1);
      if (tj >= nkt) break;
      iteration(S1, S0);
      if (tj >= nkt) break;
    }
  }

  // ---- epilogue ----
  const float lt = l_run + lane_read_f(l_run, lane ^ 32);
  if (a.nsplit > 1) {
    // partial (max, normaliser, unnormalised accumulator) of this key range
    if (row < a.Lq) {
      float* dst = a.part + ((((int64_t)split * a.k.B + b) * a.Hq + hq) * a.Lq + row) * PART_REC;
      if (hb == 0) {
        dst[0] = m_run;
        dst[1] = row_live ? lt : 0.f;
      }
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int vq = 0; vq < 4; ++vq) {
          const int d0 = 32 * db + 8 * vq + 4 * hb;
          *reinterpret_cast<f32x4*>(dst + 4 + d0) =
              f32x4{o[db][4 * vq], o[db][4 * vq + 1], o[db][4 * vq + 2], o[db][4 * vq + 3]};
        }
    }
    return;
  }
  const float inv = (row_live && lt > 0.f) ? 1.f / lt : 0.f;
  if (row < a.Lq) {
    uint16_t* op = a.o + (((int64_t)b * a.Hq + hq) * a.Lq + row) * D;
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

// One kernel per (K bits, V bits) variant over the KV heads of that variant
// (a.heads).  1-D grid: consecutive workgroup ids go round-robin to the 8
// XCDs, so with the KV head as the fastest index every XCD keeps serving the
// same KV heads (its L2 holds their K/V tiles); query blocks run longest-first.
template <int R, bool K8, bool V8>
__global__ void __launch_bounds__(NT)
prefill_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[3 * LDS_STAGE];
  const int H = a.nheads, B = a.k.B;
  const int id = blockIdx.x;
  const int g = a.heads[id % H];
  const int rest = id / H;
  const int b = rest % B;
  const int rest2 = rest / B;
  const int split = rest2 % a.nsplit;
  const int qblk = a.n_qblk - 1 - rest2 / a.nsplit;
  int n = a.lens[b];
  n = n < 0 ? 0 : (n > a.L ? a.L : n);
  prefill_body<R, K8, V8>(a, b, g, qblk, split, n, lds);
}

// Merge of the key-range partials: one wave per (b, query head, row), lane =
// channel pair; splits are combined in split order.
__global__ void __launch_bounds__(256)
prefill_merge_kernel(PrefillArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t rowid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // (b, hq, row)
  const int64_t nrow = (int64_t)a.k.B * a.Hq * a.Lq;
  if (rowid >= nrow) return;
  const int64_t sstride = nrow * PART_REC;
  const float* src = a.part + rowid * PART_REC;
  float M = NEG_BIG;
  for (int sp = 0; sp < a.nsplit; ++sp) M = fmaxf(M, src[sp * sstride]);
  float l = 0.f, o0 = 0.f, o1 = 0.f;
  for (int sp = 0; sp < a.nsplit; ++sp) {
    const float* ps = src + sp * sstride;
    const float f = fast_exp2(ps[0] - M);
    l = fmaf(ps[1], f, l);
    const float2 v = *reinterpret_cast<const float2*>(ps + 4 + 2 * lane);
    o0 = fmaf(v.x, f, o0);
    o1 = fmaf(v.y, f, o1);
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  half2v h = {(_Float16)(o0 * inv), (_Float16)(o1 * inv)};
  *reinterpret_cast<half2v*>(a.o + rowid * D + 2 * lane) = h;
}

template <int R>
hipError_t launch_variants(PrefillArgs a, hipStream_t s) {
  for (int var = 0; var < 4; ++var) {
    const bool k8 = var & 2, v8 = var & 1;
    a.nheads = 0;
    for (int h = 0; h < a.k.H; ++h)
      if ((((a.k.is8 >> h) & 1ull) != 0) == k8 && (((a.v.is8 >> h) & 1ull) != 0) == v8)
        a.heads[a.nheads++] = (uint8_t)h;
    if (a.nheads == 0) continue;
    const dim3 grid(a.n_qblk * a.nsplit * a.nheads * a.k.B);
    switch (var) {
      case 0: hipLaunchKernelGGL((prefill_kernel<R, false, false>), grid, dim3(NT), 0, s, a); break;
      case 1: hipLaunchKernelGGL((prefill_kernel<R, false, true>), grid, dim3(NT), 0, s, a); break;
      case 2: hipLaunchKernelGGL((prefill_kernel<R, true, false>), grid, dim3(NT), 0, s, a); break;
      default: hipLaunchKernelGGL((prefill_kernel<R, true, true>), grid, dim3(NT), 0, s, a); break;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

int prefill_splits(int B, int Hkv, int r, int q_len, int max_len) {
  // Enough workgroups to cover the CUs once, each split keeping >= 4 key tiles:
  // the kernel's LDS admits one workgroup per CU, so one round of longer
  // splits beats two rounds of shorter ones (half the partials to write and
  // merge; 512-row chunk after 8192 cached: 118 -> 104 us).
  const int bq = 32 * (NWAVE / r);
  const int64_t wgs = (int64_t)B * Hkv * ((q_len + bq - 1) / bq);
  const int tiles = (max_len + KT - 1) / KT;
#ifndef TAQ_PREFILL_SPLIT_TARGET
#define TAQ_PREFILL_SPLIT_TARGET 256
#endif
  int ns = 1;
  while (ns < 16 && wgs * ns < TAQ_PREFILL_SPLIT_TARGET && tiles / (2 * ns) >= 4) ns *= 2;
  return ns;
}

hipError_t launch_attn_prefill(const PrefillArgs& a, hipStream_t s) {
  hipError_t e;
  switch (a.r) {
    case 1: e = launch_variants<1>(a, s); break;
    case 2: e = launch_variants<2>(a, s); break;
    case 4: e = launch_variants<4>(a, s); break;
    case 8: e = launch_variants<8>(a, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess || a.nsplit <= 1) return e;
  const int64_t nrow = (int64_t)a.k.B * a.Hq * a.Lq;
  hipLaunchKernelGGL(prefill_merge_kernel, dim3((unsigned)((nrow + 3) / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace taq
