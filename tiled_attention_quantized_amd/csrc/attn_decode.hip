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
//  * one workgroup per (KV chunk, KV head, batch); a 256-thread workgroup owns one chunk
//    of `chunk` tokens of one (batch, KV head) and serves all r = Hq/Hkv query
//    heads of that KV head, so each K/V byte is read once.  Every precision
//    variant runs in one launch; when the launch takes more than one round
//    of workgroups, a one-workgroup plan kernel first lists the live chunks
//    heaviest first (full 8-bit chunks down to the short last chunks of the
//    sequences) and workgroup i takes entry i.
//  * the 4 waves share the chunk in steps of 32 tokens (wave w takes step w of
//    every 128-token tile) and each keeps its own (max, normaliser,
//    accumulator).  The loads of the next steps are issued before the current
//    step is computed (software pipeline over the steps).  The waves merge
//    through LDS and the workgroup writes one partial triple per query head.
//  * a second kernel merges the chunk partials of each (batch, query head) in
//    chunk order and writes fp16 O.
//  * two-pass variant (the literal reading of the "coarse max first, then fix
//    the normaliser" wording of section 2.2, kept as an ablation and cross-check
//    of the online merge): pass 1 runs the same score path and writes each
//    chunk's exact maximum; pass 2 takes the global maximum of its query head
//    from those partials, accumulates exp2(s - M) v and exp2(s - M) with no
//    rescaling, and the merge adds the chunk partials.  Pass 1 reads K only.
//
// Per step, both contractions run on the matrix cores (v_mfma_f32_16x16x32_f16):
//  * scores: A = block-diagonal Q (row = (head, quant group), 16 rows per block
//    of 4 heads), B = K codes as exact biased fp16 values (bias + c); one
//    more MFMA per 16 tokens takes sum_c q_c (bias_c + z) off (from per-row
//    sums of Q held as fp16 hi + lo pairs: exact products, fp32 sums), so no
//    per-code zero-point add is needed.  Each lane ends
//    up with the 4 per-group partial dot products of one (head, token) and
//    applies the 4 group scales itself: score = sum_g s_g * dot_g.
//  * PV: A = V-hat^T (rows = channels) dequantised to fp16 in registers from
//    the channel-major V layout (8 consecutive tokens of one channel per lane;
//    the 16 lanes of a row read 16 consecutive channel rows, so each load
//    instruction is one contiguous run; the scales and zeros of the 8 tokens
//    come per quantisation group from one lane of the row by a DPP
//    broadcast), B = P^T gathered across lanes with ds_bpermute; O^T
//    accumulates in fp32.
#include "taq_internal.h"
#include "device_common.h"

namespace taq {
namespace {

constexpr int D = 128;
constexpr int STEP = 32;       // tokens per wave step
constexpr int MAX_CHUNK = 4096;   // tokens per split chunk, at most
// a chunk's 128-token KV tiles fit one 32-bit keep mask
static_assert(MAX_CHUNK / 128 <= 32, "chunk tile mask is 32 bits");
constexpr int WAVES = 4;
constexpr float NEG_BIG = -1.0e30f;

// Softmax schedule of a decode launch.
constexpr int ONLINE = 0;      // running max with lazy rescale, one pass
constexpr int MAX_PASS = 1;    // two-pass, pass 1: exact maximum of the chunk
constexpr int FIXED_MAX = 2;   // two-pass, pass 2: weights against the global maximum

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
    return perm_b32(vconst(0xE4E4E4E4u), w, (m & 1) ? 0x04030402u : 0x04010400u);
  }
  // int4: the code pair m comes from nibbles_to_biased_h2(., ., m), whose
  // bias is 1024 for even m and 64 for odd m
  const uint32_t sel = (uint32_t)m | (0x0Cu << 8) | ((uint32_t)(4 + m) << 16) | (0x0Cu << 24);
  const uint32_t nz = perm_b32(z8[1], z8[0], sel) | 0xE400E400u;
  return (m & 1) ? odd_nibble_negz(nz) : nz;
}

template <bool V8>
__device__ __forceinline__ uint32_t v_scale_pair(u32x4 s8, int m) {
  if (V8) return s8[m];
  const uint32_t lo = s8[m >> 1], hi = s8[2 + (m >> 1)];
  return perm_b32(hi, lo, (m & 1) ? 0x07060302u : 0x05040100u);
}

template <bool V8>
__device__ __forceinline__ uint32_t v_code_pair(u32x2 c8, uint32_t c8s, int m) {
  if (V8) return bytes_to_biased_h2(m < 2 ? c8[0] : c8[1], m & 1);
  return nibbles_to_biased_h2(c8[0], c8s, m);
}

// Raw bytes of one 32-token step held by one lane: the K part (scores) and
// the V part (PV) are separate buffers because the loop consumes them one
// step apart.
struct KData {
  u32x4 kc[2][2];   // K codes of the lane's two tokens (group lg); int4 uses [bk][0]
  uint32_t kz[2];   // K zero bytes of those tokens (group lg)
  u32x2 ks[2];      // K scales of those tokens (all 4 groups)
};
struct VData {
  u32x4 vw[4];      // the step's V block, 16 bytes per lane per load: load k holds bytes
                    // 1024 k + 16 L .. +15 in lane L (int8: 4 KB, four loads; int4: 2 KB, two)
  u32x2 vz;         // V zeros of the lane's 8 tokens (group i16 % 4)
  u32x4 vs;         // V scales of the lane's 8 tokens (group i16 % 4)
};

struct Ptrs {
  const uint8_t* kbase;
  const uint8_t* vbase;
  const uint16_t* kscale;
  const uint8_t* kzero;
  const uint16_t* vscale;
  const uint8_t* vzero;
  int cap;
};

// Per-lane byte offsets of one step's loads, fixed for the whole loop: each
// load is a wave-uniform base (moved by the step) plus one of these, so the
// loop does no per-lane address arithmetic and every load destination keeps
// its own registers while the next step's loads are in flight.
struct LaneOffsets {
  uint32_t k[2], kz[2], ks[2];   // per QK block bk
  uint32_t vz, vs;               // V zeros / scales
  uint32_t vrow;                 // V codes: the lane's 16 bytes of each 1 KB of the block
};

template <bool K8, bool V8>
__device__ __forceinline__ LaneOffsets lane_offsets(int i16, int lg, int cap) {
  LaneOffsets o;
#pragma unroll
  for (int bk = 0; bk < 2; ++bk) {
    const uint32_t T = (uint32_t)qk_token<V8>(bk, i16);
    o.k[bk] = K8 ? T * D + 32 * lg : T * (D / 2) + 16 * lg;
    o.kz[bk] = T * 4 + lg;
    o.ks[bk] = T * 8;                                      // 4 fp16 scales per token
  }
  // lanes i16 = 0..3 of each row hold the row's tokens' scales and zeros of
  // groups 0..3 (the other lanes repeat them); step_pv broadcasts them
  o.vz = (uint32_t)(i16 & 3) * (uint32_t)cap + 8 * lg;
  o.vs = 2 * o.vz;
  o.vrow = 16u * (uint32_t)(16 * lg + i16);
  return o;
}

// Buffer resources of one (batch, KV head) slab: a load is then a scalar
// resource, a scalar offset that moves with the step and a fixed per-lane
// offset, with no per-lane address arithmetic in the loop (and reads past a
// slab's end return 0 instead of touching other memory).
struct Rsrc {
  __amdgpu_buffer_rsrc_t k, kz, ks, v, vz, vs;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

template <bool K8, bool V8>
__device__ __forceinline__ Rsrc make_rsrcs(const Ptrs& p) {
  Rsrc r;
  const uint32_t cap = (uint32_t)p.cap;
  r.k = make_rsrc(p.kbase, cap * (K8 ? D : D / 2));
  r.kz = make_rsrc(p.kzero, cap * 4);
  r.ks = make_rsrc(p.kscale, cap * 8);
  r.v = make_rsrc(p.vbase, cap * (V8 ? D : D / 2));
  r.vz = make_rsrc(p.vzero, cap * 4);
  r.vs = make_rsrc(p.vscale, cap * 8);
  return r;
}

// Cache policy of the K and V code loads: non-temporal (the "nt" bit of the
// buffer instruction's cache-policy operand).  Every code byte is read once
// per call and each cache line by one load instruction, so keeping the lines
// in the caches only evicts the scales and zero-points, which several lanes
// and steps share (those keep the default policy: non-temporal there was
// slower).  On the 128K mixed workload 291 -> 256 us, ragged 263 -> 240 us.
constexpr int CODE_POLICY = 2;

// Loads of one 32-token step starting at t0 (a multiple of 32): K part.
template <bool K8, bool V8>
__device__ __forceinline__ void load_k(const Rsrc& r, int t0, const LaneOffsets& o, KData& s) {
  const int tk = t0 * (K8 ? D : D / 2);
#pragma unroll
  for (int bk = 0; bk < 2; ++bk) {
    s.kc[bk][0] = __builtin_amdgcn_raw_buffer_load_b128(r.k, o.k[bk], tk, CODE_POLICY);
    if (K8) s.kc[bk][1] = __builtin_amdgcn_raw_buffer_load_b128(r.k, o.k[bk] + 16, tk, CODE_POLICY);
    s.kz[bk] = __builtin_amdgcn_raw_buffer_load_b8(r.kz, o.kz[bk], t0 * 4, 0);
    s.ks[bk] = __builtin_amdgcn_raw_buffer_load_b64(r.ks, o.ks[bk], t0 * 8, 0);
  }
}

// V part: one V block of D channel rows per step, read as 16-byte loads over
// the contiguous block (the memory pipeline's instruction rate, not its
// bandwidth, limited the step with one 4- or 8-byte operand piece per load);
// step_pv redistributes it through LDS.
template <bool V8>
__device__ __forceinline__ void load_v(const Rsrc& r, int t0, const LaneOffsets& o, VData& s) {
  const int tv = (t0 >> 5) * (D * (V8 ? 32 : 16));
#pragma unroll
  for (int k = 0; k < (V8 ? 4 : 2); ++k)
    s.vw[k] = __builtin_amdgcn_raw_buffer_load_b128(r.v, o.vrow + 1024 * k, tv, CODE_POLICY);
  s.vz = __builtin_amdgcn_raw_buffer_load_b64(r.vz, o.vz, t0, 0);
  s.vs = __builtin_amdgcn_raw_buffer_load_b128(r.vs, o.vs, 2 * t0, 0);
}

// A step with fewer than STEP live tokens (only a wave's last step can be
// one): zero the V scales of the dead tokens, so their V-hat is exactly 0
// whatever the cache holds there.
__device__ __forceinline__ void mask_v_tail(VData& s, int nvalid, int lg) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int ta = 8 * lg + 2 * j;
    s.vs[j] &= (ta < nvalid ? 0x0000FFFFu : 0u) | (ta + 1 < nvalid ? 0xFFFF0000u : 0u);
  }
}

template <int R, bool K8, bool V8>
struct WaveState {
  static constexpr int NRB = (R + 3) / 4;
  half8 aq[NRB][4];
  half8 az[NRB];       // zero-point operand (A): (Qs hi, lo, Qo hi, lo, 0, 0, 0, 0) / 2^e
  uint32_t zneg, zodd;  // zero-point operand (B): fp16 -2^e (1024 + z) byte, 960 * 2^e pair
  float m_run[NRB], l_run[NRB];
  f32x4 acc[8];
};

// Lane N of each 16-lane row copied to the whole row (DPP row_newbcast).
template <int N>
__device__ __forceinline__ uint32_t row_bcast(uint32_t x) {
  // every lane of a row reads a live lane, so no "old" value (and no
  // register initialisation) is needed
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x150 + N, 0xF, 0xF, true);
}

// PV for the two V loads of quantisation group GQ.  Every lane prepares the
// operand pairs (negated biased zero-points, masked scales) of its own group
// for the row's 8 tokens (nzl, scl); group GQ's come from lane GQ of the row.
template <bool V8, int GQ>
__device__ __forceinline__ void pv_group(f32x4 (&acc)[8], const u32x2 (&vc)[8],
                                         const uint32_t (&nzl)[4], const uint32_t (&scl)[4],
                                         half8 bp) {
  uint32_t nzp[4], scp[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    nzp[m] = row_bcast<GQ>(nzl[m]);
    scp[m] = row_bcast<GQ>(scl[m]);
  }
#pragma unroll
  for (int db = 2 * GQ; db < 2 * GQ + 2; ++db) {
    u32x4 o;
    const uint32_t c8s = V8 ? 0u : vc[db][0] >> 8;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const half2v cz = u32_to_h2(v_code_pair<V8>(vc[db], c8s, m)) + u32_to_h2(nzp[m]);
      o[m] = h2_to_u32(cz * u32_to_h2(scp[m]));
    }
    acc[db] = mfma16x16x32(u4_to_h8(o), bp, acc[db]);
  }
}

// Scores and softmax of one step: the running maximum and normaliser are
// updated, the weights come back as the PV operand (bp), and the return value
// says whether the accumulator must be rescaled by `alpha` (rare: see
// rescale_acc) before the step's PV is added.
template <int R, bool K8, bool V8, int MODE>
__device__ __forceinline__ bool step_scores(const DecodeArgs& a, WaveState<R, K8, V8>& ws,
                                            const KData& s, int nvalid, int i16, int lg,
                                            half8& bp, float (&alpha)[(R + 3) / 4]) {
  constexpr int NRB = WaveState<R, K8, V8>::NRB;
  // ---------------- scores ----------------
  float sc[NRB][2];
#pragma unroll
  for (int bk = 0; bk < 2; ++bk) {
    // B operands: the codes as exact biased fp16 values (bias + c), and
    // zb = (-2^e (1024 + z), -2^e (1024 + z), 960 * 2^e, 960 * 2^e) for the
    // zero-point MFMA (see az); -2^e (1024 + z) is the fp16 bit pattern
    // (ws.zneg byte) << 8 | z
    const uint32_t nz = perm_b32(ws.zneg, s.kz[bk], 0x04000400u);
    half8 bk8[4];
    const half8 zb = u4_to_h8(u32x4{nz, ws.zodd, 0u, 0u});
    if (K8) {
      const uint32_t wv[8] = {s.kc[bk][0][0], s.kc[bk][0][1], s.kc[bk][0][2], s.kc[bk][0][3],
                              s.kc[bk][1][0], s.kc[bk][1][1], s.kc[bk][1][2], s.kc[bk][1][3]};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        u32x4 o;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          o[k] = bytes_to_biased_h2(wv[2 * kk + (k >> 1)], k & 1);
        }
        bk8[kk] = u4_to_h8(o);
      }
    } else {
      const u32x4 cw = s.kc[bk][0];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        u32x4 o;
        const uint32_t cws = cw[kk] >> 8;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          o[k] = nibbles_to_biased_h2(cw[kk], cws, k);
        }
        bk8[kk] = u4_to_h8(o);
      }
    }
    const u32x2 sraw = s.ks[bk];
    const float s0 = (float)u32_to_h2(sraw[0])[0], s1 = (float)u32_to_h2(sraw[0])[1];
    const float s2 = (float)u32_to_h2(sraw[1])[0], s3 = (float)u32_to_h2(sraw[1])[1];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      f32x4 d4 = mfma16x16x32(ws.az[rb], zb, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) d4 = mfma16x16x32(ws.aq[rb][kk], bk8[kk], d4);
      float x = s0 * d4[0];
      x = fmaf(s1, d4[1], x);
      x = fmaf(s2, d4[2], x);
      x = fmaf(s3, d4[3], x);
      x *= a.scale_log2;
      const bool live = 4 * rb + lg < R;
      sc[rb][bk] = live ? x : 0.f;
    }
  }
  // The chunk's last step may hold fewer than STEP tokens: tokens past the
  // end get score -inf (a select, so that no branch splits the step from the
  // PV work it is scheduled with), hence weight exactly 0.
#pragma unroll
  for (int bk = 0; bk < 2; ++bk) {
    const bool dead = qk_token<V8>(bk, i16) >= nvalid;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) sc[rb][bk] = dead ? -INFINITY : sc[rb][bk];
  }

  if constexpr (MODE == MAX_PASS) {
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
      ws.m_run[rb] = fmaxf(ws.m_run[rb], row16_max(fmaxf(sc[rb][0], sc[rb][1])));
    return false;
  }

  // ---------------- online softmax ----------------
  // The running maximum m is only moved when the tile maximum exceeds it by
  // more than 2^8 (log2 units): weights exp2(s - m) then stay below 256, exact
  // enough in fp16, and the accumulator is rescaled only on those steps.  The
  // final O = acc / l is unchanged by the choice of m.  With FIXED_MAX, m is
  // the global maximum from pass 1 and never moves (weights <= 1).
  uint32_t p2[NRB];
  bool any_move = false;
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    bool move = false;
    if constexpr (MODE == ONLINE) {
      const float mx = row16_max(fmaxf(sc[rb][0], sc[rb][1]));
      move = mx > ws.m_run[rb] + 8.f;
      const float mn = move ? mx : ws.m_run[rb];
      alpha[rb] = move ? fast_exp2(ws.m_run[rb] - mn) : 1.f;
      ws.m_run[rb] = mn;
    } else {
      alpha[rb] = 1.f;
    }
    any_move |= move;
    const float mn = ws.m_run[rb];
    const _Float16 p0 = (_Float16)fast_exp2(sc[rb][0] - mn);
    const _Float16 p1 = (_Float16)fast_exp2(sc[rb][1] - mn);
    ws.l_run[rb] = fmaf(ws.l_run[rb], alpha[rb], (float)p0 + (float)p1);
    p2[rb] = h2_to_u32(half2v{p0, p1});
  }
  const bool rescale = MODE == ONLINE && __any(any_move);

  // ---------------- gather P^T and alpha into the PV layout ----------------
  const int hcol = i16;
  const int hsrc = (hcol & 3) * 16;
  u32x4 pb;
#pragma unroll
  for (int mm = 0; mm < 4; ++mm) {
    const int src = hsrc + 4 * lg + mm;
    uint32_t v = lane_read(p2[0], src);
    if (NRB > 1) {
      const uint32_t v1 = lane_read(p2[NRB - 1], src);
      v = (hcol >> 2) ? v1 : v;
    }
    // columns hcol >= R repeat a finite row of another column; their
    // accumulator columns are never written out
    pb[mm] = v;
  }
  bp = u4_to_h8(pb);
  return rescale;
}

// acc *= alpha of its query head (accumulator column = head), gathered from
// the score layout.
template <int R, bool K8, bool V8>
__device__ __forceinline__ void rescale_acc(WaveState<R, K8, V8>& ws,
                                            const float (&alpha)[(R + 3) / 4], int i16) {
  constexpr int NRB = (R + 3) / 4;
  const int hsrc = (i16 & 3) * 16;
  float al = lane_read_f(alpha[0], hsrc);
  if (NRB > 1) {
    const float a1 = lane_read_f(alpha[NRB - 1], hsrc);
    al = (i16 >> 2) ? a1 : al;
  }
#pragma unroll
  for (int db = 0; db < 8; ++db) ws.acc[db] = ws.acc[db] * al;
}

// PV of one step: the V-hat^T operand is built from the step's V block and
// multiplied with the weights bp.
template <int R, bool K8, bool V8>
__device__ __forceinline__ void step_pv(WaveState<R, K8, V8>& ws, const VData& s, half8 bp,
                                        int i16, int lg, uint32_t* vst) {
  // ---------------- V-hat^T operand and PV ----------------
  // loads 2 gq and 2 gq + 1 are channels of group gq
  // V codes in the operand layout: lane (i16, lg) takes row 16 db + i16,
  // tokens 8 lg .. +7.  The block goes through the wave's own LDS (LDS
  // operations of one wave run in order, so no barrier; every read is one
  // contiguous run over the 64 lanes, free of bank conflicts).
  const int lane = 16 * lg + i16;
#pragma unroll
  for (int k = 0; k < (V8 ? 4 : 2); ++k)
    *reinterpret_cast<u32x4*>(vst + 256 * k + 4 * lane) = s.vw[k];
  u32x2 vc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    if constexpr (V8) {
      vc[db] = *reinterpret_cast<const u32x2*>(vst + 8 * (16 * db + i16) + 2 * lg);
    } else {
      vc[db][0] = vst[4 * (16 * db + i16) + lg];
      vc[db][1] = 0u;
    }
  }
  // the lane's own group: zero-point and (tail-masked) scale pairs, once per
  // step rather than once per broadcast
  uint32_t nzl[4], scl[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    nzl[m] = v_negz_pair<V8>(s.vz, m);
    scl[m] = v_scale_pair<V8>(s.vs, m);
  }
  pv_group<V8, 0>(ws.acc, vc, nzl, scl, bp);
  pv_group<V8, 1>(ws.acc, vc, nzl, scl, bp);
  pv_group<V8, 2>(ws.acc, vc, nzl, scl, bp);
  pv_group<V8, 3>(ws.acc, vc, nzl, scl, bp);
}

template <int R, bool K8, bool V8, int MODE>
__device__ void decode_body(const DecodeArgs& a, int b, int g, int c, int n, float* lds,
                            uint32_t* vstage) {
  constexpr int NRB = (R + 3) / 4;
  const int lane = threadIdx.x & 63;
  // wave index as a scalar: all token-range and loop control below is
  // wave-uniform, so it runs on the scalar unit with real branches
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i16 = lane & 15;
  uint32_t* vst = vstage + w * (V8 ? 1024 : 512);   // the wave's V staging
  const int lg = lane >> 4;

  const CacheGeom& K = a.k;
  const CacheGeom& V = a.v;
  const int G = D / 32;
  Ptrs p;
  p.kbase = K.codes + (int64_t)b * K.bstride + K.hoff[g];
  p.vbase = V.codes + (int64_t)b * V.bstride + V.hoff[g];
  p.kscale = K.scales + ((int64_t)b * K.H + g) * K.cap * G;
  p.kzero = K.zeros + ((int64_t)b * K.H + g) * K.cap * G;
  p.vscale = V.scales + ((int64_t)b * V.H + g) * G * (int64_t)V.cap;
  p.vzero = V.zeros + ((int64_t)b * V.H + g) * G * (int64_t)V.cap;
  p.cap = K.cap;

  WaveState<R, K8, V8> ws;
  // ---- Q as the block-diagonal A operand ------------------------------------
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
      ws.aq[rb][kk] = u4_to_h8(o);
    }
  }
  // Zero-point operand of each lane's (head, group) row.  The scores' B
  // operand holds the codes with the bias of their slot (1024, or 64 for the
  // odd int4 pairs), so a row's dot needs sum_c q_c (bias_c + z) taken off:
  // -(1024 + z) Qs + 960 Qo, with Qs = sum_c q_c and Qo the sum over the odd
  // int4 pairs.  One MFMA per 16 tokens does it, with
  // A = (Qs hi, Qs lo, Qo hi, Qo lo) / 2^e and
  // B = (-2^e (1024 + z), -2^e (1024 + z), 960 * 2^e, 960 * 2^e): the
  // products are exact in fp32 and the sums fp32.  e = 0 unless a sum of the
  // wave would leave the fp16 range (then e = 5, so that |Qs| / 32 and
  // |Qo| / 32 are fp16 values for any fp16 query; e = 0 keeps the lo parts
  // out of the fp16 subnormals for small sums).
  {
    float qs[NRB], qo[NRB];
    bool big = false;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      qs[rb] = 0.f;
      qo[rb] = 0.f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float v = (float)ws.aq[rb][kk][j];
          qs[rb] += v;
          if (!K8 && ((j >> 1) & 1)) qo[rb] += v;
        }
      big |= !(fabsf(qs[rb]) <= 32768.f && fabsf(qo[rb]) <= 32768.f);
    }
    const bool wave_big = __builtin_amdgcn_ballot_w64(big) != 0;
    const float sc = wave_big ? 1.f / 32.f : 1.f;
    ws.zneg = vconst(wave_big ? 0xF8F8F8F8u : 0xE4E4E4E4u);   // -(1024 + z) * 32 or * 1
    ws.zodd = wave_big ? 0x73807380u : 0x63806380u;   // 15360 or 960
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const float s2 = qs[rb] * sc, o2 = qo[rb] * sc;
      const _Float16 qh = (_Float16)s2, oh = (_Float16)o2;
      const _Float16 ql = (_Float16)(s2 - (float)qh), ol = (_Float16)(o2 - (float)oh);
      const _Float16 z0 = (_Float16)0.f;
      ws.az[rb] = half8{qh, ql, oh, ol, z0, z0, z0, z0};
    }
  }
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) { ws.m_run[rb] = NEG_BIG; ws.l_run[rb] = 0.f; }
  if constexpr (MODE == FIXED_MAX) {
    // global maximum of each query head: the largest of the pass-1 chunk maxima
    const int nc = (n + a.chunk - 1) / a.chunk;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int h = 4 * rb + lg;
      if (h < R) {
        const float* src = a.ws + ((int64_t)b * a.Hq + g * R + h) * a.nchunk * (D + 2);
        float M = NEG_BIG;
        for (int cc = 0; cc < nc; ++cc) M = fmaxf(M, src[(int64_t)cc * (D + 2)]);
        ws.m_run[rb] = M;
      } else {
        ws.m_run[rb] = 0.f;   // rows past the r heads: score 0, weight 1, never used
      }
    }
  }
#pragma unroll
  for (int db = 0; db < 8; ++db) ws.acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // The waves share the chunk: wave w takes the 32-token step w of every
  // 128-token tile, so a partial last chunk of a sequence keeps all four waves
  // busy (with contiguous quarters, most of its waves idled while one ran its
  // full range) and the workgroup reads one contiguous stream.
  const int c0 = c * a.chunk;
  const int t_end = min(c0 + a.chunk, n);
  const int t_safe = c0;   // a valid step address (c * chunk < n)

  // KV-tile keep bits of the chunk's tiles (chunk <= MAX_CHUNK: at most 32
  // tiles of 128 tokens), read once so that the step loop does no mask loads.
  uint32_t tbits = 0xFFFFFFFFu;
  if (a.mask) {
    const uint8_t* mrow = a.mask + (int64_t)b * a.mask_sb + (int64_t)g * a.mask_sh + (c0 >> 7);
    const int ntile = (t_end - c0 + 127) >> 7;
    tbits = 0;
    for (int k = 0; k < ntile; ++k) tbits |= (mrow[k] ? 1u : 0u) << k;
  }
  // first of this wave's steps at or after t (t itself one of them) whose
  // tile is kept (t_end if none): a find-first-set on the wave-uniform keep
  // bits, no loop
  auto next_step = [&](int t) -> int {
    if (t >= t_end) return t;
    const uint32_t rest = tbits >> ((t - c0) >> 7);
    if (rest & 1u) return t;
    if (rest == 0u) return t_end;
    return t + (__builtin_ctz(rest) << 7);
  };
  constexpr int STRIDE = STEP * WAVES;   // from one of a wave's steps to the next

  // ---- software pipeline over the wave's steps -------------------------------
  // Iteration i issues the K loads of step i+2 and the V loads of step i+1,
  // then computes the PV of step i together with the scores and softmax of
  // step i+1 in one block (independent work the scheduler interleaves, so the
  // latencies of one chain hide behind the other).  The rare branches (tail
  // V scales of step i before, accumulator rescale for step i+1 after) sit
  // outside the block; the rescale after PV(i) is exact since PV(i) is
  // relative to the old maximum.  Every iteration issues exactly one step of
  // loads (past the end: a repeat of a valid step that is never used), so each
  // wait before a use is partial.  Step starts are wave-uniform: keep them
  // scalar (they are the scalar offsets of the buffer loads).
  auto addr = [&](int t) { return __builtin_amdgcn_readfirstlane(t < t_end ? t : t_safe); };
  const LaneOffsets lo = lane_offsets<K8, V8>(i16, lg, p.cap);
  const Rsrc rs = make_rsrcs<K8, V8>(p);
  int tc = next_step(c0 + w * STEP);
  if (tc < t_end) {
    int tn = next_step(tc + STRIDE);
    KData K0, K1;
    VData V0, V1;
    half8 bp;
    float alpha[NRB];
    load_k<K8, V8>(rs, addr(tc), lo, K0);
    if (MODE != MAX_PASS) load_v<V8>(rs, addr(tc), lo, V0);
    load_k<K8, V8>(rs, addr(tn), lo, K1);
    if (step_scores<R, K8, V8, MODE>(a, ws, K0, t_end - tc, i16, lg, bp, alpha)) {
      asm volatile("" ::: "memory");
      rescale_acc(ws, alpha, i16);
    }
    // V(tc) in Va, K(tn) in Kb, bp = weights of step tc; Ka and Vb are free
    auto body = [&](KData& Ka, const KData& Kb, VData& Va, VData& Vb) -> bool {
      if (tn >= t_end) {
        if (MODE != MAX_PASS) {
          if (t_end - tc < STEP) {
            asm volatile("" ::: "memory");
            mask_v_tail(Va, t_end - tc, lg);
          }
          step_pv(ws, Va, bp, i16, lg, vst);
        }
        return false;
      }
      const int t2 = next_step(tn + STRIDE);
      load_k<K8, V8>(rs, addr(t2), lo, Ka);
      if (MODE != MAX_PASS) {
        load_v<V8>(rs, addr(tn), lo, Vb);
        if (t_end - tc < STEP) {
          asm volatile("" ::: "memory");
          mask_v_tail(Va, t_end - tc, lg);
        }
        step_pv(ws, Va, bp, i16, lg, vst);
      }
      const bool rs_ = step_scores<R, K8, V8, MODE>(a, ws, Kb, t_end - tn, i16, lg, bp, alpha);
      if (rs_) {
        asm volatile("" ::: "memory");
        rescale_acc(ws, alpha, i16);
      }
      tc = tn;
      tn = t2;
      return true;
    };
    while (body(K0, K1, V0, V1) && body(K1, K0, V1, V0)) {
    }
  }

  // ---- merge the 4 waves through LDS ------------------------------------------
  // layout: m[4][R], l[4][R], o[4][R][D]
  float* sm = lds;
  float* sl = lds + WAVES * R;
  float* so = lds + 2 * WAVES * R;
  if constexpr (MODE == MAX_PASS) {
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int h = 4 * rb + lg;
      if (i16 == 0 && h < R) sm[w * R + h] = ws.m_run[rb];
    }
    __syncthreads();
    if (threadIdx.x < R) {
      const int h = threadIdx.x;
      float M = sm[h];
#pragma unroll
      for (int ww = 1; ww < WAVES; ++ww) M = fmaxf(M, sm[ww * R + h]);
      a.ws[(((int64_t)b * a.Hq + g * R + h) * a.nchunk + c) * (D + 2)] = M;
    }
    return;
  }
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const float lt = row16_sum(ws.l_run[rb]);
    const int h = 4 * rb + lg;
    if (i16 == 0 && h < R) {
      sm[w * R + h] = ws.m_run[rb];
      sl[w * R + h] = lt;
    }
  }
  if (i16 < R) {
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        so[(w * R + i16) * D + 16 * db + 4 * lg + v] = ws.acc[db][v];
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
      // FIXED_MAX: every wave used the same maximum, the weights add as they are
      const float f = MODE == FIXED_MAX ? 1.f : fast_exp2(sm[ww * R + h] - M);
      o = fmaf(so[(ww * R + h) * D + d], f, o);
      l = fmaf(sl[ww * R + h], f, l);
    }
    float* dst = a.ws + (((int64_t)b * a.Hq + g * R + h) * nchunk + c) * (D + 2);
    dst[2 + d] = o;
    if (d == 0) {
      if (MODE == ONLINE) dst[0] = M;    // FIXED_MAX: slot 0 keeps the pass-1 maximum
      dst[1] = l;
    }
  }
}

// Chunk plan: the live (unit, chunk) pairs of the call in the order the split
// kernel's workgroups take them, heaviest first.  The weight of a chunk is
// its 128-token tiles times the code bytes per token of its KV head (2, 3
// or 4 units for int4/int4, mixed, int8/int8), so full chunks of 8-bit heads
// come first and the short last chunks of the sequences fill the end of the
// launch (the longest-job-first rule), and no workgroup slot goes to a chunk
// past a sequence's end.  One workgroup: a histogram of the weights, a scan
// from the heaviest weight down, then every unit reserves its chunks' slots
// at its weights' next free positions (the order inside one weight is
// immaterial: every chunk's partial is computed and merged the same way
// wherever it runs).
constexpr int PLAN_KEYS = 4 * 32 + 1;   // weights 0 .. 128

__device__ __forceinline__ int chunk_cost(const DecodeArgs& a, int g) {
  return (((a.k.is8 >> g) & 1ull) ? 2 : 1) + (((a.v.is8 >> g) & 1ull) ? 2 : 1);
}

__global__ void __launch_bounds__(1024) decode_plan_kernel(DecodeArgs a) {
  __shared__ int count[PLAN_KEYS];
  __shared__ int next[PLAN_KEYS];
  for (int i = threadIdx.x; i < PLAN_KEYS; i += blockDim.x) count[i] = 0;
  __syncthreads();
  const int H = a.k.H, units = a.k.B * H;
  const int full_tiles = a.chunk / 128;
  for (int u = threadIdx.x; u < units; u += blockDim.x) {
    const int b = u / H, g = u - b * H;
    int n = a.lens[b];
    n = n < 0 ? 0 : (n > a.max_len ? a.max_len : n);
    const int cost = chunk_cost(a, g);
    const int nfull = n / a.chunk, rem = n - nfull * a.chunk;
    if (nfull > 0) atomicAdd(&count[full_tiles * cost], nfull);
    if (rem > 0) atomicAdd(&count[((rem + 127) >> 7) * cost], 1);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int at = 0;
    for (int key = PLAN_KEYS - 1; key >= 0; --key) {
      next[key] = at;
      at += count[key];
    }
    a.plan[0] = (uint32_t)at;
  }
  __syncthreads();
  uint2* items = reinterpret_cast<uint2*>(a.plan + 2);
  for (int u = threadIdx.x; u < units; u += blockDim.x) {
    const int b = u / H, g = u - b * H;
    int n = a.lens[b];
    n = n < 0 ? 0 : (n > a.max_len ? a.max_len : n);
    const int cost = chunk_cost(a, g);
    const int nfull = n / a.chunk, rem = n - nfull * a.chunk;
    if (nfull > 0) {
      // one reservation for the unit's full chunks (same weight), not one
      // atomic per chunk: the threads' reservations of one weight would
      // otherwise serialise on its counter chunk by chunk
      const int at = atomicAdd(&next[full_tiles * cost], nfull);
      for (int c = 0; c < nfull; ++c) items[at + c] = make_uint2((uint32_t)u, (uint32_t)c);
    }
    if (rem > 0) {
      const int at = atomicAdd(&next[((rem + 127) >> 7) * cost], 1);
      items[at] = make_uint2((uint32_t)u, (uint32_t)nfull);
    }
  }
}

// Two waves per SIMD for every variant: the register budget that leaves
// (up to 256 VGPRs) holds two steps of loads without spilling; at three waves
// the int4 variant spilled and ran 20% slower.  Workgroup i takes item i of
// the plan (the grid covers every possible chunk; the rest return at once)
// or, without a plan, chunk i % nchunk of unit i / nchunk,
// and every (K bits, V bits) variant runs in this one launch, so heads of
// different precision share the tail of the launch instead of each draining
// the GPU.
template <int R, int MODE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
decode_split_kernel(DecodeArgs a) {
  __shared__ float lds[2 * WAVES * R + WAVES * R * D];
  __shared__ __attribute__((aligned(16))) uint32_t vstage[WAVES * 1024];
  const int H = a.k.H;
  int b, g, c;
  if (a.plan != nullptr) {
    if (blockIdx.x >= a.plan[0]) return;
    const uint2 item = reinterpret_cast<const uint2*>(a.plan + 2)[blockIdx.x];
    if (item.x >= (uint32_t)(a.k.B * H) || item.y >= (uint32_t)a.nchunk) return;
    b = (int)item.x / H;
    g = (int)item.x - b * H;
    c = (int)item.y;
  } else {
    // one round of workgroups: the order is immaterial
    const int u = blockIdx.x / a.nchunk;
    c = blockIdx.x - u * a.nchunk;
    b = u / H;
    g = u - b * H;
  }
  int n = a.lens[b];
  n = n < 0 ? 0 : (n > a.max_len ? a.max_len : n);
  if (c * a.chunk >= n) return;
  const bool k8 = ((a.k.is8 >> g) & 1ull) != 0, v8 = ((a.v.is8 >> g) & 1ull) != 0;
  if (k8) {
    if (v8) decode_body<R, true, true, MODE>(a, b, g, c, n, lds, vstage);
    else decode_body<R, true, false, MODE>(a, b, g, c, n, lds, vstage);
  } else {
    if (v8) decode_body<R, false, true, MODE>(a, b, g, c, n, lds, vstage);
    else decode_body<R, false, false, MODE>(a, b, g, c, n, lds, vstage);
  }
}

// One workgroup per (batch, query head).  Every wave finds the global maximum
// over all chunks (lanes over chunks); wave w then adds chunks w, w + 4, ...
// (lane = channel pair) and the four partials are added in wave order, so the
// result is repeatable.  TWO_PASS: every chunk's partials are relative to the
// same global maximum, so they add with factor 1.
template <bool TWO_PASS>
__global__ void __launch_bounds__(256)
decode_merge_kernel(DecodeArgs a) {
  __shared__ float po[WAVES][D];
  __shared__ float pl[WAVES];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int bh = blockIdx.x;
  const int b = bh / a.Hq;
  int n = a.lens[b];
  n = n < 0 ? 0 : (n > a.max_len ? a.max_len : n);
  const int nc = (n + a.chunk - 1) / a.chunk;
  const float* src = a.ws + (int64_t)bh * a.nchunk * (D + 2);
  float M = NEG_BIG;
  if (!TWO_PASS) {
    for (int c = lane; c < nc; c += 64) M = fmaxf(M, src[(int64_t)c * (D + 2)]);
    M = fmaxf(M, __shfl_xor(M, 32));
    M = row16_max(fmaxf(M, __shfl_xor(M, 16)));
  }
  float l = 0.f, o0 = 0.f, o1 = 0.f;
#pragma unroll 4
  for (int c = w; c < nc; c += WAVES) {
    const float* cs = src + (int64_t)c * (D + 2);
    const float f = TWO_PASS ? 1.f : fast_exp2(cs[0] - M);
    l = fmaf(cs[1], f, l);
    const float2 v = *reinterpret_cast<const float2*>(cs + 2 + 2 * lane);
    o0 = fmaf(v.x, f, o0);
    o1 = fmaf(v.y, f, o1);
  }
  po[w][2 * lane] = o0;
  po[w][2 * lane + 1] = o1;
  if (lane == 0) pl[w] = l;
  __syncthreads();
  if (w == 0) {
    const float L = ((pl[0] + pl[1]) + pl[2]) + pl[3];
    const float O0 = ((po[0][2 * lane] + po[1][2 * lane]) + po[2][2 * lane]) + po[3][2 * lane];
    const float O1 = ((po[0][2 * lane + 1] + po[1][2 * lane + 1]) + po[2][2 * lane + 1]) +
                     po[3][2 * lane + 1];
    const float inv = L > 0.f ? 1.f / L : 0.f;
    half2v h = {(_Float16)(O0 * inv), (_Float16)(O1 * inv)};
    *reinterpret_cast<half2v*>(a.o + (int64_t)bh * D + 2 * lane) = h;
  }
}

}  // namespace

uint32_t* decode_plan_of(float* ws, int B, int Hq, int nchunk) {
  return reinterpret_cast<uint32_t*>(ws + (int64_t)B * Hq * nchunk * (D + 2));
}

size_t decode_workspace_bytes(int B, int Hkv, int Hq, int max_len) {
  const int chunk = decode_chunk_tokens(B, Hkv, max_len);
  const int64_t nchunk = max_len > 0 ? (max_len + chunk - 1) / chunk : 1;
  const size_t partials = (size_t)B * Hq * nchunk * (D + 2) * sizeof(float);
  const size_t plan = (2 + 2 * (size_t)B * Hkv * nchunk) * sizeof(uint32_t);
  return partials + plan;
}

int decode_chunk_tokens(int B, int Hkv, int max_len) {
  // Largest chunk (<= 4096 tokens) that still gives >= 2048 workgroups, so
  // every CU gets several; at least 128 (32 tokens per wave).
  int chunk = MAX_CHUNK;
  const int64_t units = (int64_t)B * Hkv;
  while (chunk > 128 && units * ((max_len + chunk - 1) / chunk) < 2048) chunk /= 2;
  return chunk;
}

template <int MODE>
hipError_t launch_split(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid(a.nchunk * a.k.H * a.k.B);
  switch (a.r) {
    case 1: hipLaunchKernelGGL((decode_split_kernel<1, MODE>), grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((decode_split_kernel<2, MODE>), grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((decode_split_kernel<4, MODE>), grid, dim3(256), 0, s, a); break;
    case 8: hipLaunchKernelGGL((decode_split_kernel<8, MODE>), grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_decode(const DecodeArgs& a_in, hipStream_t s, bool two_pass) {
  DecodeArgs a = a_in;
  // A launch that fits the GPU in one round of workgroups (two per CU) needs
  // no plan; a longer one takes its chunks in the plan's order.
  a.plan = nullptr;
  if ((int64_t)a.nchunk * a.k.H * a.k.B > 512) {
    a.plan = decode_plan_of(a.ws, a.k.B, a.Hq, a.nchunk);
    hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(1024), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipError_t e;
  if (two_pass) {
    e = launch_split<MAX_PASS>(a, s);
    if (e == hipSuccess) e = launch_split<FIXED_MAX>(a, s);
  } else {
    e = launch_split<ONLINE>(a, s);
  }
  if (e != hipSuccess) return e;
  const int nbh = a.k.B * a.Hq;
  if (two_pass)
    hipLaunchKernelGGL(decode_merge_kernel<true>, dim3(nbh), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(decode_merge_kernel<false>, dim3(nbh), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace taq
