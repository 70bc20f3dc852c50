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
//  * a 512-thread workgroup (8 waves, two per SIMD: the second wave of a SIMD
//    issues while the first waits on a matrix instruction) owns BQ = 256 / r
//    query rows of all r = Hq/Hkv query heads that share one KV head, so every
//    K/V tile is fetched and dequantised once for 256 (head, row) pairs; wave w
//    takes head w % r and the 32 rows (w / r) * 32 .. +31;
//  * the key loop runs over the workgroup's needed 64-key tiles through LDS
//    rings of four stages as a software pipeline with one barrier per tile:
//    the QK^T MFMAs of tile j+1 interleave with the weights of tile j, and
//    the PV MFMAs of tile j with the dequantisation of tile j+3; tile j+4 is
//    fetched into registers (buffer loads whose scalar offset is the tile's
//    byte offset).  The loop is unrolled four times, so every ring stage is a
//    constant LDS offset.  The two waves of a SIMD take the barrier at
//    different points of that sequence, so while one computes exponentials
//    the other dequantises.  Inside those blocks each chain of dependent
//    vector instructions (exponent argument, exponential, fp16 rounding and
//    row sum; codes to fp16, zero-point, scale) is spread over three
//    matrix-instruction slices, so no instruction waits on the one just
//    before it;
//  * both contractions use v_mfma_f32_32x32x16_f16 in transposed form:
//    S^T = K-hat Q^T (A = K-hat tile from LDS, B = Q held in registers) and
//    O^T += V-hat^T P^T (A = V-hat^T tile from LDS, B = P straight from the
//    S^T accumulator), so every lane owns one query row for the whole loop and
//    the softmax statistics stay lane-local;
//  * the running maximum m of a row is not recomputed per tile: it starts
//    at the row maximum of the first tile, the weights exp2(s - m) of each
//    tile are formed against the current m and rounded to fp16, and only when
//    a lane's sum of them exceeds 2^15 (a score more than ~15 above m, or a
//    row's first key after tiles that gave it none) is the tile's row maximum
//    taken, m moved, the accumulator and normaliser rescaled and the weights
//    recomputed (a rare branch that forms the tile's scores again).  The
//    result is the same softmax: the factor exp2(-m) cancels between
//    numerator and normaliser;
//  * the needed tiles are taken from 64-bit windows over 64 key tiles (one
//    byte load per lane and query tile and three ballots per window; a tile
//    is then a find-first-set and a clear), and the causal / length / mask
//    masking of a tile's scores only runs on tiles that need it, one compare
//    and select per score;
//  * the workgroup order runs the longest causal rows first.
#include "taq_internal.h"
#include "device_common.h"

namespace taq {
namespace {

constexpr int D = 128;
constexpr int KT = 64;                 // keys per tile
constexpr int NWAVE = 8;
constexpr int NT = 64 * NWAVE;
constexpr int NBLK = 8;                // 32-row blocks per workgroup (one per wave)
constexpr int KS_STRIDE = D * 2 + 16;  // bytes per K-hat row in LDS (padded)
constexpr int VS_STRIDE = KT * 2 + 16; // bytes per V-hat^T row in LDS (padded)
constexpr int LDS_K = KT * KS_STRIDE;
constexpr int LDS_V = D * VS_STRIDE;
// LDS rings of four stages each for K-hat and V-hat^T tiles (walk tile j in
// stage j % 4), then one int per wave for the SIMD table.
constexpr int NKST = 4;
constexpr int NVST = 4;
constexpr int LDS_TABLE = NKST * LDS_K + NVST * LDS_V;
constexpr int LDS_BYTES = LDS_TABLE + 4 * NWAVE;
constexpr float NEG_BIG = -1.0e30f;
// A lane's weights of one tile are safe in fp16 (and exact enough) while
// their sum stays at or below this; above it the tile takes the rescale path.
constexpr float P_SUM_LIMIT = 32768.f;
// key-range partial of one (split, b, query head, row): m, l, 2 pad, acc[D]
// (16-byte aligned records)
constexpr int PART_REC = D + 4;

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
// K: thread (key = tid / 8, group = (tid / 2) % 4, half = tid % 2), 16
// channels of one key.  V: thread (channel d = tid / 4, quarter q = tid % 4),
// keys 16 q .. 16 q + 15 of the tile.
struct Staged {
  u32x4 kc;        // K codes (int8: 16 B; int4: first 8 B)
  uint32_t kz;     // K zero byte
  uint32_t ks;     // K scale bits
  u32x4 vc;        // V codes (int8: 16 B; int4: first 8 B)
  u32x4 vz;        // V zeros of the 16 keys
  u32x4 vs[2];     // V scales of the 16 keys
};

// Buffer resources of one (batch, KV head) slab's six arrays.  A tile load
// is then the resource, the tile's byte offset (a scalar operand of the
// instruction) and a fixed per-lane byte offset: no address arithmetic per
// tile beyond one shift per array.  Every tile a workgroup loads lies below
// the sequence length, so all loads stay inside the slab (and a read past
// a resource's size would return 0).
struct Slab {
  __amdgpu_buffer_rsrc_t k, kz, ks, v, vz, vs;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t slab_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// Per-thread byte offsets of its share of a tile (from the tile's first key).
struct LaneOff {
  uint32_t k, kz, ks, v, vz, vs;
};

template <bool K8, bool V8>
__device__ __forceinline__ LaneOff lane_offsets(int tid, int cap) {
  LaneOff o;
  const int unit = tid >> 1, half = tid & 1;
  const int key = unit >> 2, grp = unit & 3;
  o.k = (uint32_t)(key * (K8 ? D : D / 2) + (K8 ? 32 : 16) * grp + (K8 ? 16 : 8) * half);
  o.kz = (uint32_t)(key * 4 + grp);
  o.ks = 2 * o.kz;
  const int d = tid >> 2, q = tid & 3;
  // key 16 q of the tile lies in 32-key block q / 2 at position 16 (q % 2)
  o.v = (uint32_t)(((q >> 1) * D + d) * (V8 ? 32 : 16) + (V8 ? 16 : 8) * (q & 1));
  o.vz = (uint32_t)((d >> 5) * cap + 16 * q);
  o.vs = 2 * o.vz;
  return o;
}

template <bool K8, bool V8>
__device__ __forceinline__ void stage_load(const Slab& r, const LaneOff& o, int kt0, Staged& s) {
  const int tk = kt0 * (K8 ? D : D / 2);
  if (K8) {
    s.kc = __builtin_amdgcn_raw_buffer_load_b128(r.k, o.k, tk, 0);
  } else {
    const u32x2 t = __builtin_amdgcn_raw_buffer_load_b64(r.k, o.k, tk, 0);
    s.kc = u32x4{t[0], t[1], 0u, 0u};
  }
  s.kz = __builtin_amdgcn_raw_buffer_load_b8(r.kz, o.kz, kt0 * 4, 0);
  s.ks = __builtin_amdgcn_raw_buffer_load_b16(r.ks, o.ks, kt0 * 8, 0);
  const int tv = (kt0 >> 5) * D * (V8 ? 32 : 16);
  if (V8) {
    s.vc = __builtin_amdgcn_raw_buffer_load_b128(r.v, o.v, tv, 0);
  } else {
    const u32x2 t = __builtin_amdgcn_raw_buffer_load_b64(r.v, o.v, tv, 0);
    s.vc = u32x4{t[0], t[1], 0u, 0u};
  }
  s.vz = __builtin_amdgcn_raw_buffer_load_b128(r.vz, o.vz, kt0, 0);
  s.vs[0] = __builtin_amdgcn_raw_buffer_load_b128(r.vs, o.vs, 2 * kt0, 0);
  s.vs[1] = __builtin_amdgcn_raw_buffer_load_b128(r.vs, o.vs + 16, 2 * kt0, 0);
}

// Dequantisation steps of one fp16 pair (K pair j in 0..7 = channels
// 16 half + 2j, +1 of the thread's (key, group); V pair j = keys 16 q + 2j, +1
// of the thread's channel): codes to biased fp16 (1024 + c, or the nibble
// forms), minus the biased zero-point, times the scale.
template <bool K8>
__device__ __forceinline__ uint32_t k_biased(const Staged& s, int j) {
  return K8 ? bytes_to_biased_h2(s.kc[j >> 1], j & 1) : nib_pair_natural(s.kc[j >> 2], j & 3);
}
template <bool V8>
__device__ __forceinline__ uint32_t v_biased(const Staged& s, int j) {
  return V8 ? bytes_to_biased_h2(s.vc[j >> 1], j & 1) : nib_pair_natural(s.vc[j >> 2], j & 3);
}
__device__ __forceinline__ uint32_t v_negzero(const Staged& s, int j) {
  return perm_b32(vconst(0xE4E4E4E4u), s.vz[j >> 1], (j & 1) ? 0x04030402u : 0x04010400u);
}
__device__ __forceinline__ uint32_t v_scales(const Staged& s, int j) {
  return s.vs[j >> 2][j & 3];
}
__device__ __forceinline__ uint32_t h2_add(uint32_t a, uint32_t b) {
  return h2_to_u32(u32_to_h2(a) + u32_to_h2(b));
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
    s.vs[j >> 2][j & 3] &= keep;
  }
}

// Dequantise the staged registers into LDS stage `dst` in one go (prologue).
template <bool K8, bool V8>
__device__ __forceinline__ void stage_store(const Staged& s, int tid, char* kdst, char* vdst) {
  const uint32_t knz = neg_biased_zero_h2(s.kz);
  const _Float16 ksc = bits_to_half((uint16_t)s.ks);
  const uint32_t ks2 = h2_to_u32(half2v{ksc, ksc});
  const int unit = tid >> 1, half = tid & 1;
  const int key = unit >> 2, grp = unit & 3;
  u32x4 ko[2];
#pragma unroll
  for (int j = 0; j < 8; ++j) ko[j >> 2][j & 3] = h2_mul(h2_add(k_biased<K8>(s, j), knz), ks2);
  u32x4* kd = reinterpret_cast<u32x4*>(kdst + key * KS_STRIDE + (32 * grp + 16 * half) * 2);
  kd[0] = ko[0];
  kd[1] = ko[1];
  const int d = tid >> 2, q = tid & 3;
  u32x4 vo[2];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    vo[vslot(j) >> 2][vslot(j) & 3] = h2_mul(h2_add(v_biased<V8>(s, j), v_negzero(s, j)),
                                             v_scales(s, j));
  u32x4* vd = reinterpret_cast<u32x4*>(vdst + d * VS_STRIDE + 32 * q);
  vd[0] = vo[0];
  vd[1] = vo[1];
}

template <int R, bool K8, bool V8>
__device__ void prefill_body(const PrefillArgs& a, int b, int g, int qblk, int split, int n,
                             char* lds) {
  constexpr int BQ = 32 * (NBLK / R);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int i32 = lane & 31, hb = lane >> 5;
  const int hq = g * R + w % R;
  const int q0 = qblk * BQ;
  const int q0w = q0 + 32 * (w / R);
  const int row = q0w + i32;             // row of q / o
  // Position of row 0 in the sequence: 0 for a whole-sequence prefill; for a
  // chunk of Lq new rows whose keys are already in the cache, n - Lq (rows
  // at negative positions are padding).  Causality and the tile mask work
  // on positions.
  const int qoff = a.chunk ? n - a.Lq : 0;
  const int pos = row + qoff;
  const int p0w = q0w + qoff;            // position of the wave's first row
  const bool row_live = row < a.Lq && pos >= 0 && pos < n;
  // some row of the wave is padding (masked on every tile)
  const bool blk_dead = p0w < 0 || p0w + 31 >= n || q0w + 31 >= a.Lq;

  Slab rs;
  {
    const uint32_t cap = (uint32_t)a.k.cap;
    rs.k = slab_rsrc(a.k.codes + (int64_t)b * a.k.bstride + a.k.hoff[g], cap * (K8 ? D : D / 2));
    rs.v = slab_rsrc(a.v.codes + (int64_t)b * a.v.bstride + a.v.hoff[g], cap * (V8 ? D : D / 2));
    rs.ks = slab_rsrc(a.k.scales + ((int64_t)b * a.k.H + g) * cap * 4, cap * 8);
    rs.kz = slab_rsrc(a.k.zeros + ((int64_t)b * a.k.H + g) * cap * 4, cap * 4);
    rs.vs = slab_rsrc(a.v.scales + ((int64_t)b * a.v.H + g) * 4 * (int64_t)cap, cap * 8);
    rs.vz = slab_rsrc(a.v.zeros + ((int64_t)b * a.v.H + g) * 4 * (int64_t)cap, cap * 4);
  }
  const LaneOff lo = lane_offsets<K8, V8>(tid, a.k.cap);

  const uint8_t* mb = a.mask ? a.mask + (int64_t)b * a.mask_sb + (int64_t)g * a.mask_sh : nullptr;

  // Q row of this lane (B operand of S^T): channels 16 ks + 8 hb .. +7
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

  // key range of the workgroup: up to its last live position
  const int wg_last = min(min(q0 + BQ, a.Lq) - 1 + qoff, n - 1);
  const int nkt_all = wg_last >= 0 ? wg_last / KT + 1 : 0;
  // key-range split: this workgroup takes tiles [kt_lo, nkt) of the query
  // block's range (equal shares; the partials are merged afterwards)
  const int per = (nkt_all + a.nsplit - 1) / a.nsplit;
  const int kt_lo = min(split * per, nkt_all);
  const int nkt = min(kt_lo + per, nkt_all);
  // query tiles of the workgroup's live positions (at most 3)
  const int qt_first = max(q0 + qoff, 0) >> 7;
  const int qt_last = wg_last >= 0 ? (wg_last >> 7) : -1;
  const int nqt = min(qt_last - qt_first + 1, 3);

  // query tiles of the wave's first and last live row (a wave's 32 rows span
  // at most two), and whether this lane's row lies in the first of them
  int qia, qib;
  bool lane_in_a;
  {
    const int qa = max(p0w, 0) >> 7, qb = max(min(p0w + 31, n - 1), 0) >> 7;
    qia = min(max(qa - qt_first, 0), 2);
    qib = min(max(qb - qt_first, 0), 2);
    const int ql = max(min(pos, n - 1), 0) >> 7;
    lane_in_a = min(max(ql - qt_first, 0), 2) == qia;
  }

  // ---- tile walk over 64-tile bit windows ------------------------------------
  // Window [wb, wb + 64) of 64-key tiles, one bit per tile and lane of a
  // ballot: U = tiles of [kt_lo, nkt) some query tile of the workgroup keeps
  // and not yet taken; Wa / Wb = tiles the query tile of the wave's first /
  // last row keeps (a query tile keeps a tile at or below its diagonal that
  // the mask keeps; every tile of the range without a mask).
  int wb = kt_lo & ~63;
  uint64_t U = 0, Wa = 0, Wb = 0;
  auto refill = [&]() {
    const int kt = wb + lane;
    const bool in = kt >= kt_lo && kt < nkt;
    bool any = in, keep_a = in, keep_b = in;
    if (mb != nullptr) {
      // every lane loads (lanes past the range read the range's last mask
      // tile), so the loads of all query tiles are in flight together
      any = keep_a = keep_b = false;
      const int mt = kt >> 1;
      const int mtc = min(mt, (nkt - 1) >> 1);
      uint32_t byte[3];
#pragma unroll
      for (int i = 0; i < 3; ++i)
        byte[i] = i < nqt ? mb[(int64_t)(qt_first + i) * a.mask_nk + mtc] : 0u;
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        const bool k = in && mt <= qt_first + i && byte[i] != 0u;
        any |= k;
        if (i == qia) keep_a = k;
        if (i == qib) keep_b = k;
      }
    }
    U = __builtin_amdgcn_ballot_w64(any);
    Wa = __builtin_amdgcn_ballot_w64(keep_a);
    Wb = __builtin_amdgcn_ballot_w64(keep_b);
  };
  // Next needed tile (nkt when the range is done) and its two keep bits
  // (bit 0: the wave's first query tile keeps it, bit 1: its last); the bits
  // travel with the tile, as the window may move on before it is processed.
  auto pop = [&](uint32_t& kab) -> int {
    kab = 3u;
    while (U == 0) {
      if (wb + 64 >= nkt) return nkt;
      wb += 64;
      refill();
    }
    const int i = __builtin_ctzll(U);
    U &= U - 1;
    kab = (uint32_t)((Wa >> i) & 1u) | ((uint32_t)((Wb >> i) & 1u) << 1);
    return wb + i;
  };
  // First tile that reaches past the sequence end, and the first tile whose
  // scores need the causal or length masking for some row of the wave
  // (every tile when the wave holds padding rows).
  const int t_len = ((n - KT) >> 6) + 1;
  const int t_crit = blk_dead ? -(1 << 30) : min(((p0w - (KT - 1)) >> 6) + 1, t_len);

  float m_run = NEG_BIG, l_run = 0.f;
  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[db][v] = 0.f;

  const float c_log2 = a.scale_log2;   // > 0 (checked on the host)

  auto kstage = [&](int x) -> char* { return lds + x * LDS_K; };
  auto vstage = [&](int x) -> char* { return lds + NKST * LDS_K + x * LDS_V; };

  // S^T = K-hat Q^T for the tile whose K-hat is at kl (16 MFMAs), no interleaving
  auto qk_plain = [&](const char* kl8, f32x16* S) {
    const uint8_t* kl = reinterpret_cast<const uint8_t*>(kl8);
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

  // causal / length / dead-row / mask masking of tile t's scores (keep bits
  // kab; only on tiles that need it).  The lane's keys kt0 + 4 hb + off
  // (off = 32 kb + 8 (v / 4) + v % 4) stay when off <= r, r from the row's
  // last admitted key; each element is one compare into VCC and one select
  // (kept as pairs, so the compares do not pile up in scalar registers).
  auto mask_tile = [&](int t, uint32_t kab, f32x16* S) {
    if (((~(uint32_t)(t - t_crit) >> 31) | (kab ^ 3u)) != 0u) {
      const bool keep = ((lane_in_a ? kab : kab >> 1) & 1u) != 0u;
      const int last = (keep && row_live) ? min(pos, n - 1) : -(1 << 30);
      const int r = last - t * KT - 4 * hb;
      const float ninf = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          asm("v_cmp_gt_i32_e32 vcc, %2, %1\n\tv_cndmask_b32_e32 %0, %0, %3, vcc"
              : "+v"(S[kb][v])
              : "v"(r), "n"(32 * kb + 8 * (v >> 2) + (v & 3)), "v"(ninf)
              : "vcc");
    }
  };

  // Rare path: the tile's row maximum (both lane halves of the row), m moved
  // to it if larger, the normaliser rescaled, weights recomputed into pk;
  // returns the lane's row sum of the new fp16 weights and, in alpha, the
  // factor that the accumulator still has to be multiplied by.
  auto rescale = [&](const f32x16* S, half8 (&pk)[4], float& alpha) -> float {
    float mx = S[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, S[kb][v]);
    mx = fmaxf(mx, lane_read_f(mx, lane ^ 32)) * c_log2;
    const float mn = fmaxf(m_run, mx);     // rows with no key keep NEG_BIG
    alpha = fast_exp2(m_run - mn);
    m_run = mn;
    l_run *= alpha;
    const half2v ones = half2v{(_Float16)1.f, (_Float16)1.f};
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; v += 2) {
        const float e0 = fast_exp2(fmaf(S[kb][v], c_log2, -mn));
        const float e1 = fast_exp2(fmaf(S[kb][v + 1], c_log2, -mn));
        const half2v hp = half2v{(_Float16)e0, (_Float16)e1};
        pk[2 * kb + (v >> 3)][v & 7] = hp[0];
        pk[2 * kb + (v >> 3)][(v & 7) + 1] = hp[1];
        ls = __builtin_amdgcn_fdot2(hp, ones, ls, false);
      }
    return ls;
  };

  // ---- software pipeline over the workgroup's KV tiles -------------------------
  // Tiles t_0, t_1, ... (causal and mask order) go through the LDS rings.
  // Per tile j every wave runs two interleaved blocks, in this order:
  //   QK(j): the QK^T MFMAs of tile j+1 with the weights of tile j;
  //   PV(j): the PV MFMAs of tile j with the dequantisation of a staged tile.
  // One barrier per tile separates epochs.  The first wave of each SIMD
  // ("early") takes the barrier before QK(j), the second ("late") between
  // QK(j) and PV(j), so epoch e holds the early waves' QK(e-1) and PV(e-1)
  // and the late waves' PV(e-1) and QK(e).  In each half of an epoch one wave
  // of a SIMD computes exponentials (vector-heavy) while the other
  // dequantises (vector-light), and both keep the matrix unit busy.  In
  // epoch e the waves read K-hat of tiles e and e+1 (e-1 and e on the rare
  // path) and V-hat^T of tile e-1, and write tile e+2 (dequantised in PV(e-1)
  // from the tile staged three ahead), so four stages of each ring are in
  // use.  Tiles are fetched from HBM into registers one tile ahead of their
  // dequantisation.  Every wave walks the same tiles; rows a tile does not
  // reach are masked, so the loop has no per-wave branches other than the
  // barrier's place.
  if (kt_lo < nkt) refill();
  uint32_t kab0, kab1 = 3u, kab2 = 3u, kab3 = 3u, kab4 = 3u;
  const int t0_ = pop(kab0);
  if (t0_ < nkt) {
    // tile window: walk tiles j .. j+4 (nkt past the end) and their keep bits
    const int t1_ = pop(kab1);
    const int t2_ = t1_ < nkt ? pop(kab2) : nkt;
    const int t3_ = t2_ < nkt ? pop(kab3) : nkt;
    const int t4_ = t3_ < nkt ? pop(kab4) : nkt;
    // SIMD of each wave (hardware wave id register, SIMD field); a wave is
    // late when an earlier wave of the workgroup sits on the same SIMD
    int* simd_of = reinterpret_cast<int*>(lds + LDS_TABLE);
    if (lane == 0) simd_of[w] = (int)__builtin_amdgcn_s_getreg((1 << 11) | (4 << 6) | 4);
    // a tile past the end is staged as a copy of a valid one (never read)
    auto valid = [&](int t) { return t < nkt ? t : t0_; };
    auto stage_direct = [&](int t, int kx, int vx, Staged& s) {
      stage_load<K8, V8>(rs, lo, valid(t) * KT, s);
      if (valid(t) * KT + KT > n) zero_tail_scales(s, valid(t) * KT + 16 * (tid & 3), n);
      stage_store<K8, V8>(s, tid, kstage(kx), vstage(vx));
    };
    Staged st;
    stage_direct(t0_, 0, 0, st);
    stage_direct(t1_, 1, 1, st);
    stage_direct(t2_, 2, 2, st);
    stage_load<K8, V8>(rs, lo, valid(t3_) * KT, st);
    __syncthreads();
    bool late_b = false;
    {
      const int mine = simd_of[w];
      for (int u = 0; u < w; ++u) late_b |= simd_of[u] == mine;
    }
    const int late = __builtin_amdgcn_readfirstlane((int)late_b);

    f32x16 S0[2], S1[2];
    qk_plain(kstage(0), S0);
    // m starts at the first tile's row maximum, so its weights need no rescale
    mask_tile(t0_, kab0, S0);
    {
      float mx = S0[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, S0[kb][v]);
      mx = fmaxf(mx, lane_read_f(mx, lane ^ 32)) * c_log2;
      m_run = fmaxf(m_run, mx);   // a row with no key in the tile keeps NEG_BIG
    }
    int tj = t0_, tj1 = t1_, tj2 = t2_, tj3 = t3_, tj4 = t4_;
    // keep bits of tiles j .. j+4, two per tile
    uint32_t kabs = kab0 | (kab1 << 2) | (kab2 << 4) | (kab3 << 6) | (kab4 << 8);
    // the loop is unrolled four times, so tile j's ring stage (j % 4, the
    // phase ph below) is a constant in each copy
    half8 pk[4];  // weights of tile j

    // QK block: S^T of tile j+1 into Sn, the weights of tile j (scores Sc)
    // into pk; returns the lane's sum of the weights.  MFMA i (i < 16):
    // accumulator kb = i % 2, k-step ks = i / 2; its LDS operand is read
    // two MFMAs ahead.  The weights of pair q (elements 2q, 2q+1 of S(j))
    // go through three slices so that no instruction waits on the one before
    // it: the exponent argument in slice q, the exponential in slice q + 1,
    // the fp16 rounding and the row sum in slice q + 2.  Past the last tile
    // the MFMAs recompute a resident stage (result unused).
    auto qk_block = [&](int ph, const f32x16* Sc, f32x16* Sn) -> float {
      float ls = 0.f;
      const uint8_t* kl = reinterpret_cast<const uint8_t*>(kstage((ph + 1) & 3));
      auto kread = [&](int i) -> u32x4 {
        const int kb = i & 1, ks = i >> 1;
        return *reinterpret_cast<const u32x4*>(kl + (32 * kb + i32) * KS_STRIDE +
                                               (16 * ks + 8 * hb) * 2);
      };
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) Sn[kb][v] = 0.f;
      const half2v ones = half2v{(_Float16)1.f, (_Float16)1.f};
      const float mn = m_run;
      u32x4 kv[16];
      float xa[16][2], ea[16][2];
#pragma unroll
      for (int i = 0; i < 2; ++i) kv[i] = kread(i);
#pragma unroll
      for (int i = 0; i < 18; ++i) {
        if (i < 16) {
          if (i + 2 < 16) kv[i + 2] = kread(i + 2);
          Sn[i & 1] = mfma32x32x16(u4_to_h8(kv[i]), qreg[i >> 1], Sn[i & 1]);
        }
        if (i >= 2) {
          const int q = i - 2, kb = q >> 3, v = 2 * (q & 7);
          const half2v hp = half2v{(_Float16)ea[q][0], (_Float16)ea[q][1]};
          pk[2 * kb + (v >> 3)][v & 7] = hp[0];
          pk[2 * kb + (v >> 3)][(v & 7) + 1] = hp[1];
          ls = __builtin_amdgcn_fdot2(hp, ones, ls, false);
        }
        if (i >= 1 && i <= 16) {
          const int q = i - 1;
          ea[q][0] = fast_exp2(xa[q][0]);
          ea[q][1] = fast_exp2(xa[q][1]);
        }
        if (i < 16) {
          const int kb = i >> 3, v = 2 * (i & 7);
          xa[i][0] = fmaf(Sc[kb][v], c_log2, -mn);
          xa[i][1] = fmaf(Sc[kb][v + 1], c_log2, -mn);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      return ls;
    };

    // After the QK block: every weight is computed (nothing of the block
    // sinks into the rare branch).  Rare: a lane's weight sum beyond the
    // fp16-safe limit (a score more than ~15 above m in log2 units, or a row's
    // first key after tiles that gave it none): the tile's scores are formed
    // again from its K-hat stage (so the QK block need not keep them), masked,
    // and m moved, the accumulator and normaliser rescaled and the weights
    // recomputed.
    auto settle_weights = [&](int ph, float ls) {
      asm volatile("" : "+v"(ls), "+v"(pk[0]), "+v"(pk[1]), "+v"(pk[2]), "+v"(pk[3]));
      if (__builtin_amdgcn_ballot_w64(!(ls <= P_SUM_LIMIT)) != 0) {
        asm volatile("" ::: "memory");   // the recompute stays inside this branch
        f32x16 Sr[2];
        qk_plain(kstage(ph), Sr);
        mask_tile(tj, kabs & 3u, Sr);
        float alpha;
        ls = rescale(Sr, pk, alpha);
#pragma unroll
        for (int db = 0; db < 4; ++db) o[db] = o[db] * alpha;
      }
      l_run += ls;
    };

    // PV block: O^T += V-hat^T (tile j) P^T (pk), with the dequantisation of
    // the staged tile (walk tile j+3) into its stages.  MFMA i
    // (i < 16): accumulator db = i % 4, k-step kk = i / 4; its LDS operand
    // is read four MFMAs ahead (the QK block, whose slices are longer, reads
    // two ahead: the depths that timed best).  Pair q of the
    // staged tile (K pairs 0..7, then V pairs 0..7) goes through three
    // slices: codes to biased fp16 in slice q, minus the biased zero-point in
    // slice q + 1, times the scale in slice q + 2.
    auto pv_block = [&](int ph) {
      const uint8_t* vl = reinterpret_cast<const uint8_t*>(vstage(ph));
      auto vread = [&](int i) -> u32x4 {
        const int db = i & 3, kk = i >> 2;
        return *reinterpret_cast<const u32x4*>(vl + (32 * db + i32) * VS_STRIDE +
                                               (16 * kk + 8 * hb) * 2);
      };
      char* kdst = kstage((ph + 3) & 3);
      char* vdst = vstage((ph + 3) & 3);
      const int unit = tid >> 1, khalf = tid & 1;
      const int kkey = unit >> 2, kgrp = unit & 3;
      const int vd = tid >> 2, vq = tid & 3;
      const uint32_t knz = neg_biased_zero_h2(st.kz);
      const _Float16 ksc = bits_to_half((uint16_t)st.ks);
      const uint32_t ks2 = h2_to_u32(half2v{ksc, ksc});
      u32x4 ko[2], vo[2];
      u32x4 av[16];
      uint32_t cb[16], cz[16], nzv[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = vread(i);
#pragma unroll
      for (int i = 0; i < 18; ++i) {
        if (i < 16) {
          if (i + 4 < 16) av[i + 4] = vread(i + 4);
          o[i & 3] = mfma32x32x16(u4_to_h8(av[i]), pk[i >> 2], o[i & 3]);
        }
        if (i >= 2) {
          const int q = i - 2;
          if (q < 8) {
            ko[q >> 2][q & 3] = h2_mul(cz[q], ks2);
          } else {
            const int jv2 = q - 8;
            vo[vslot(jv2) >> 2][vslot(jv2) & 3] = h2_mul(cz[q], v_scales(st, jv2));
          }
        }
        if (i >= 1 && i <= 16) {
          const int q = i - 1;
          cz[q] = h2_add(cb[q], q < 8 ? knz : nzv[q - 8]);
        }
        if (i < 16) {
          if (i < 8) {
            cb[i] = k_biased<K8>(st, i);
          } else {
            cb[i] = v_biased<V8>(st, i - 8);
            nzv[i - 8] = v_negzero(st, i - 8);
          }
        }
        if (i == 10) {
          u32x4* kd = reinterpret_cast<u32x4*>(kdst + kkey * KS_STRIDE + (32 * kgrp + 16 * khalf) * 2);
          kd[0] = ko[0];
          kd[1] = ko[1];
        }
        if (i == 17) {
          u32x4* vdp = reinterpret_cast<u32x4*>(vdst + vd * VS_STRIDE + 32 * vq);
          vdp[0] = vo[0];
          vdp[1] = vo[1];
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    auto iteration = [&](int ph, f32x16* Sc, f32x16* Sn) {
      uint32_t kab5 = 3u;
      const int tj5 = pop(kab5);
      if (late == 0) __syncthreads();
      mask_tile(tj, kabs & 3u, Sc);
      // the staged tile j+3: zero its V scales past the sequence end (rare)
      const int tstaged = valid(tj3);
      if (tstaged >= t_len) {
        asm volatile("" ::: "memory");
        zero_tail_scales(st, tstaged * KT + 16 * (tid & 3), n);
      }
      settle_weights(ph, qk_block(ph, Sc, Sn));
      if (late != 0) __syncthreads();
      pv_block(ph);
      stage_load<K8, V8>(rs, lo, valid(tj4) * KT, st);
      tj = tj1; tj1 = tj2; tj2 = tj3; tj3 = tj4; tj4 = tj5;
      kabs = (kabs >> 2) | (kab5 << 8);
    };

    while (true) {
      iteration(0, S0, S1);
      if (tj >= nkt) break;
      iteration(1, S1, S0);
      if (tj >= nkt) break;
      iteration(2, S0, S1);
      if (tj >= nkt) break;
      iteration(3, S1, S0);
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
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
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
  // merge).
  const int bq = 32 * (NBLK / r);
  const int64_t wgs = (int64_t)B * Hkv * ((q_len + bq - 1) / bq);
  const int tiles = (max_len + KT - 1) / KT;
  int ns = 1;
  while (ns < 16 && wgs * ns < 256 && tiles / (2 * ns) >= 4) ns *= 2;
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
