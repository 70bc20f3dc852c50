// Internal declarations shared by the host API and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/taq.h"

namespace taq {

// Geometry of one cache as the kernels see it: per-head code offsets inside a
// batch entry and a bitmask of the 8-bit heads.
struct CacheGeom {
  uint8_t* codes;
  uint16_t* scales;
  uint8_t* zeros;
  int64_t bstride;                      // code bytes per batch entry
  int64_t hoff[TAQ_MAX_KV_HEADS];       // code byte offset of each head
  uint64_t is8;                         // bit h set: head h stores int8 codes
  int32_t B, H, D, cap, layout;
};

struct QuantArgs {
  CacheGeom c;
  const uint16_t* x;     // fp16 [B][H][count][D]
  int32_t start, count;
  const int32_t* starts; // device [B] per-batch start (append), or null: start
  float* out32;          // dequantise outputs (either may be null)
  uint16_t* out16;
};

struct DecodeArgs {
  CacheGeom k, v;
  const uint16_t* q;     // [B][Hq][D]
  uint16_t* o;           // [B][Hq][D]
  const int32_t* lens;   // [B]
  const uint8_t* mask;   // null = none
  int64_t mask_sb, mask_sh;
  int32_t mask_nk;
  float* ws;             // partials [B][Hq][nchunk][D + 2], then the chunk plan
  uint32_t* plan;        // [0]: live chunks; then (unit = b * Hkv + g, chunk) pairs
  int32_t Hq, r, max_len, chunk, nchunk;
  float scale_log2;      // softmax scale * log2(e)
};

struct PrefillArgs {
  CacheGeom k, v;
  const uint16_t* q;     // [B][Hq][L][D]
  uint16_t* o;
  const int32_t* lens;
  const uint8_t* mask;
  int64_t mask_sb, mask_sh;
  int32_t mask_nq, mask_nk;
  int32_t Hq, r, L;      // L: max_seq_len (bound on the sequence lengths)
  int32_t Lq;            // rows of q / o (L for a whole-sequence prefill)
  int32_t chunk;         // nonzero: row i sits at position n_b - Lq + i
  int32_t n_qblk;        // query blocks per (b, kv head) over Lq rows
  int32_t nsplit;        // key-range splits per query block (1: write O directly)
  float* part;           // nsplit > 1: partials [nsplit][B][Hq][Lq][D + 4] (m, l, -, -, acc)
  float scale_log2;
  int32_t nheads;        // KV heads handled by one launch, listed in heads[]
  uint8_t heads[TAQ_MAX_KV_HEADS];
};

// Training-free KV-tile mask generator (per (batch, KV head) 128x128 masks).
constexpr int MASKGEN_MAX_TILES = 2048;   // tiles per side (max_seq_len <= 262144)
struct MaskGenArgs {
  CacheGeom k;
  const uint16_t* q;     // [B][Hq][Lq][D]; row i of entry b at position pos0_b + i
  const int32_t* lens;
  uint8_t* mask;         // [B][Hkv][nt][nt]
  double* qsum;          // workspace [B][Hkv][nt][D]: query sums in units of 2^-24
  double* kmean;         // workspace [B][Hkv][D][nt]: mean dequantised key per tile
  double* score;         // workspace [B][Hkv][nt][nt]: importance (lower triangle)
  int32_t Hq, r, L, nt, skip_per_mille;
  int32_t Lq;            // rows of q (L for a whole prompt)
  int32_t turn;          // nonzero: q is a turn, pos0_b = n_b - Lq, and only the
                         // rows of the turn's query tiles are generated
};
hipError_t launch_tile_mask(const MaskGenArgs& a, hipStream_t s);

hipError_t launch_kv_quantize(const QuantArgs& a, hipStream_t s);
// Two caches of equal head_dim over the same token range, one launch.
hipError_t launch_kv_quantize_pair(const QuantArgs& a0, const QuantArgs& a1, hipStream_t s);
hipError_t launch_head_assign(const uint16_t* o8, const uint16_t* o4, int B, int Hq, int Hkv,
                              int n_high, double* scores, uint8_t* bits, hipStream_t s);
hipError_t launch_kv_dequantize(const QuantArgs& a, hipStream_t s);
hipError_t launch_attn_decode(const DecodeArgs& a, hipStream_t s, bool two_pass);
hipError_t launch_attn_prefill(const PrefillArgs& a, hipStream_t s);
// Key-range splits the chunked prefill uses for these shapes (1 = none).
int prefill_splits(int B, int Hkv, int r, int q_len, int max_len);

// Decode split geometry chosen on the host (used for workspace sizing too).
int decode_chunk_tokens(int B, int Hkv, int max_len);
// Decode workspace: the chunk partials, then the chunk plan.
size_t decode_workspace_bytes(int B, int Hkv, int Hq, int max_len);
// The plan's place in a decode workspace.
uint32_t* decode_plan_of(float* ws, int B, int Hq, int nchunk);

}  // namespace taq
