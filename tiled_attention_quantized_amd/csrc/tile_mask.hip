// Training-free KV-tile mask generator for block-sparse prefill.
//
// Policy: a coarse pattern of skipped 128x128 blocks with dense local blocks,
// the skipped share capped so that no block is starved ("分块稀疏注意力与KV
// Cache量化：长文本推理显存优化实践", xdnf.cn, section 2.3).  The page's
// predictor is a learned head; this generator uses a data-only importance
// instead.  Per batch entry b, KV head g and query tile i < nt_b: keep KV tile
// 0 and the diagonal; of tiles 1 .. i-1 drop the floor((i-1) * skip / 1000)
// with the lowest importance (ties: lower j first);
//   importance(i, j) = sum_d Qsum_i[d] * Kmean_j[d],
// Qsum_i = sum of the query rows of tile i over the Hq/Hkv heads of g (units
// of 2^-24), Kmean_j = mean of the dequantised keys of tile j.  The
// arithmetic is fixed so that it is reproducible bit for bit: the sums are
// exact integers (fp16 values and (c - z) * s are integer multiples of
// 2^-24), Kmean = double(Ksum) / cnt / 2^24, and the dot product runs over d
// in order as a double multiply then a double add (no fused multiply-add).
//
// For one turn of a multi-turn prefill (q holds the last Lq positions of each
// sequence, section 4.2 of the same page), the rows of the query tiles that
// hold the turn's positions are generated, each ranked from the turn's own
// rows in the tile; every other row is 0.
//
// Kernels: pool_q (one workgroup per (b, g, tile)), pool_k (same, reading the
// quantised K cache), score (the lower triangle of Qsum . Kmean^T in 64 x 64
// blocks), select (one wave per (b, g, query tile): the m lowest scores found
// by a bitwise search over order-preserving keys, then the mask row).
#include "taq_internal.h"
#include "device_common.h"

namespace taq {
namespace {

constexpr int TILE = 128;
constexpr double UNIT = 16777216.0;   // 2^24

// Pooling: 256 threads per (b, g, tile), thread = (channel octet c8, row lane
// kr); each thread reads 16-byte (Q) or 8/4-byte (K codes) pieces of rows
// lo + kr, lo + kr + 16, ..., then the 16 row lanes are summed through LDS.
constexpr int POOL_THREADS = 256;

__device__ __forceinline__ void pool_unit(const MaskGenArgs& a, int& b, int& g, int& t,
                                          int& lo, int& hi, int& n) {
  t = blockIdx.x % a.nt;
  const int rest = blockIdx.x / a.nt;
  g = rest % a.k.H;
  b = rest / a.k.H;
  n = a.lens[b];
  n = n < 0 ? 0 : (n > a.L ? a.L : n);
  lo = t * TILE;
  hi = min(lo + TILE, n);
}

// Query sums.  Every fp16 value is an integer multiple of 2^-24 below 2^16 in
// magnitude, and a tile holds at most 64 * 128 of them per channel, so every
// partial sum is a multiple of 2^-24 below 2^53 * 2^-24: double addition is
// exact here in any order.
__global__ void __launch_bounds__(POOL_THREADS)
pool_q_kernel(MaskGenArgs a) {
  __shared__ double red[16][128];
  const int tid = threadIdx.x, c8 = tid & 15, kr = tid >> 4;
  int b, g, t, lo, hi, n;
  pool_unit(a, b, g, t, lo, hi, n);
  // a turn holds positions pos0 .. n-1 (q row = position - pos0): the tile's
  // sum covers the turn's rows in it
  const int pos0 = a.turn ? n - a.Lq : 0;
  lo = max(lo, pos0);
  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;
  for (int hl = 0; hl < a.r; ++hl) {
    const uint16_t* qp = a.q + (((int64_t)b * a.Hq + g * a.r + hl) * a.Lq - pos0) * 128 + 8 * c8;
    for (int row = lo + kr; row < hi; row += 16) {
      // Q is read once here: non-temporal (keeps the caches for the K
      // pooling; 128K prompt: 451 -> 416 us for the whole generator)
      const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(qp + (int64_t)row * 128));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const half2v h = u32_to_h2(w[e]);
        acc[2 * e] += (double)(float)h[0];
        acc[2 * e + 1] += (double)(float)h[1];
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[kr][8 * c8 + e] = acc[e];
  __syncthreads();
  if (tid < 128) {
    double s = 0.0;
    for (int k = 0; k < 16; ++k) s += red[k][tid];
    a.qsum[(((int64_t)b * a.k.H + g) * a.nt + t) * 128 + tid] = s * UNIT;    // exact
  }
}

// fp16 scale -> integer multiple of 2^-24: (mantissa << shift).
__device__ __forceinline__ long long half_units(uint16_t h) {
  const int e = (h >> 10) & 31, f = h & 1023;
  const long long m = e ? (long long)(1024 | f) << (e - 1) : (long long)f;
  return (h & 0x8000) ? -m : m;
}

// Key means.  (c - z) * s is an integer multiple of 2^-24 below 2^48 in
// magnitude, so the sums over a tile are exact in int64; the mean is then
// rounded twice, as the definition states (/ count, then / 2^24).
__global__ void __launch_bounds__(POOL_THREADS)
pool_k_kernel(MaskGenArgs a) {
  __shared__ long long red[16][128];
  const int tid = threadIdx.x, c8 = tid & 15, kr = tid >> 4;
  int b, g, t, lo, hi, n;
  pool_unit(a, b, g, t, lo, hi, n);
  const bool is8 = (a.k.is8 >> g) & 1ull;
  const uint8_t* codes = a.k.codes + (int64_t)b * a.k.bstride + a.k.hoff[g];
  const int64_t mrow = ((int64_t)b * a.k.H + g) * a.k.cap * 4 + (c8 >> 2);
  long long acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0;
  for (int key = lo + kr; key < hi; key += 16) {
    const long long s = half_units(a.k.scales[mrow + (int64_t)key * 4]);
    const int z = a.k.zeros[mrow + (int64_t)key * 4];
    int c[8];
    if (is8) {
      const u32x2 w = *reinterpret_cast<const u32x2*>(codes + (int64_t)key * 128 + 8 * c8);
#pragma unroll
      for (int e = 0; e < 8; ++e) c[e] = (w[e >> 2] >> (8 * (e & 3))) & 255;
    } else {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(codes + (int64_t)key * 64 + 4 * c8);
#pragma unroll
      for (int e = 0; e < 8; ++e) c[e] = (w >> (4 * e)) & 15;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += (long long)(c[e] - z) * s;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[kr][8 * c8 + e] = acc[e];
  __syncthreads();
  if (tid < 128) {
    long long sum = 0;
    for (int k = 0; k < 16; ++k) sum += red[k][tid];
    const int cnt = hi > lo ? hi - lo : 1;
    a.kmean[(((int64_t)b * a.k.H + g) * 128 + tid) * a.nt + t] =
        ((double)sum / (double)cnt) / UNIT;
  }
}

// Scores over the lower triangle in 64 x 64 blocks of (query tile i, KV tile
// j), the blocks of the triangle only (block t of a head is the t-th
// (bi, bj) with bj <= bi, row by row).  Thread (ti, tj) of 256 owns
// i = I0 + 4 ti + x and j = J0 + 4 tj + y (x, y < 4).  Qsum and Kmean pass
// through LDS 32 channels at a time, a thread's 4 rows (columns) contiguous
// (two 16-byte reads each); every score is still accumulated over
// d = 0 .. 127 in order, multiply then add.
constexpr int SB = 64, SD = 32;

__global__ void __launch_bounds__(256)
score_kernel(MaskGenArgs a, int nb) {
#pragma clang fp contract(off)
  __shared__ __attribute__((aligned(16))) double qs[SD][SB];   // [e][row]
  __shared__ __attribute__((aligned(16))) double ks[SD][SB];   // [e][column]
  const int ntri = nb * (nb + 1) / 2;
  const int t = blockIdx.x % ntri;
  const int rest = blockIdx.x / ntri;
  const int g = rest % a.k.H, b = rest / a.k.H;
  // row bi of the triangle holds blocks bi (bi + 1) / 2 .. + bi
  int bi = (int)((sqrtf(8.f * (float)t + 1.f) - 1.f) * 0.5f);
  while (bi * (bi + 1) / 2 > t) --bi;
  while ((bi + 1) * (bi + 2) / 2 <= t) ++bi;
  const int bj = t - bi * (bi + 1) / 2;
  const int I0 = bi * SB, J0 = bj * SB;
  const int tid = threadIdx.x, ti = tid >> 4, tj = tid & 15;
  const int64_t bg = (int64_t)b * a.k.H + g;
  const double* qsum = a.qsum + bg * a.nt * 128;
  const double* kmean = a.kmean + bg * 128 * a.nt;
  double acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = 0.0;
  for (int d0 = 0; d0 < 128; d0 += SD) {
    for (int x = tid; x < SB * SD; x += 256) {
      const int r = x / SD, e = x % SD, i = I0 + r;
      qs[e][r] = i < a.nt ? qsum[(int64_t)i * 128 + d0 + e] : 0.0;
    }
    for (int x = tid; x < SD * SB; x += 256) {
      const int e = x / SB, c = x % SB, j = J0 + c;
      ks[e][c] = j < a.nt ? kmean[(int64_t)(d0 + e) * a.nt + j] : 0.0;
    }
    __syncthreads();
    for (int e = 0; e < SD; ++e) {
      double qv[4], kv[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) qv[x] = qs[e][4 * ti + x];
#pragma unroll
      for (int y = 0; y < 4; ++y) kv[y] = ks[e][4 * tj + y];
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = acc[x][y] + kv[y] * qv[x];
    }
    __syncthreads();
  }
  double* S = a.score + bg * a.nt * a.nt;
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const int i = I0 + 4 * ti + x, j = J0 + 4 * tj + y;
      if (i < a.nt && j < i) S[(int64_t)i * a.nt + j] = acc[x][y];
    }
}

// Selection: one wave per mask row (four rows per workgroup, no LDS and no
// barriers).  Lane l holds the scores of candidates c = 64r + l (KV tile
// j = c + 1) for r < RR, RR the power of two at or above ceil((i - 1) / 64).
// The m lowest (score, j) pairs are found without sorting: scores become
// unsigned keys with the same order, a bitwise search finds the m-th smallest
// key v (the largest v with fewer than m keys below it), and among the keys
// equal to v a second search drops the lowest j first.  Each count is the
// population of one compare's lane mask per register (one vector compare and
// two scalar instructions): a count that also masked off the lanes past the
// candidates took three vector instructions and ran the generator 8% slower.
__device__ __forceinline__ uint64_t order_key(double v) {
  if (v == 0.0) v = 0.0;                         // -0 and +0 compare equal
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  return (u >> 63) ? ~u : (u | (1ull << 63));
}

template <int RR>
__device__ __forceinline__ void select_row(const double* srow, int ncand, int m, int lane,
                                           uint8_t* row) {
  // lanes past the candidates hold the largest key, which no search value
  // exceeds and no selected value equals (scores are finite, so every real
  // key is smaller), so the counts need no mask of live lanes
  uint64_t key[RR];
#pragma unroll
  for (int r = 0; r < RR; ++r) {
    const uint64_t k = order_key(srow[1 + min(64 * r + lane, ncand - 1)]);
    key[r] = 64 * r + lane < ncand ? k : ~0ull;
  }
  auto count_below = [&](uint64_t t) {
    int cnt = 0;
#pragma unroll
    for (int r = 0; r < RR; ++r) cnt += __popcll(__ballot(key[r] < t));
    return cnt;
  };
  uint64_t v = 0;
  for (int bit = 63; bit >= 0; --bit) {
    const uint64_t t = v | (1ull << bit);
    if (count_below(t) < m) v = t;
  }
  const int need = m - count_below(v);          // >= 1 keys equal to v to drop
  int u = 0;
  for (int bit = 10; bit >= 0; --bit) {
    const int t = u | (1 << bit);
    int cnt = 0;
#pragma unroll
    for (int r = 0; r < RR; ++r) cnt += __popcll(__ballot(key[r] == v && 64 * r + lane < t));
    if (cnt < need) u = t;
  }
#pragma unroll
  for (int r = 0; r < RR; ++r) {
    const int c = 64 * r + lane;
    if (c < ncand) row[c + 1] = (key[r] < v || (key[r] == v && c <= u)) ? 0 : 1;
  }
}

__global__ void __launch_bounds__(256)
select_kernel(MaskGenArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nrow4 = (a.nt + 3) / 4;
  const int rest = blockIdx.x / nrow4;
  const int i = (blockIdx.x % nrow4) * 4 + wave;
  const int g = rest % a.k.H, b = rest / a.k.H;
  if (i >= a.nt) return;                         // whole wave
  int n = a.lens[b];
  n = n < 0 ? 0 : (n > a.L ? a.L : n);
  const int nt_b = (n + TILE - 1) / TILE;
  // a turn generates the rows of the query tiles that hold its positions
  const int first = a.turn ? (a.Lq > 0 ? max(n - a.Lq, 0) / TILE : nt_b) : 0;
  const bool live = i < nt_b && i >= first;
  const int ncand = i - 1;                       // tiles 1 .. i-1
  const int64_t bg = (int64_t)b * a.k.H + g;
  uint8_t* row = a.mask + (bg * a.nt + i) * a.nt;
  // every entry but the candidates: tile 0 and the diagonal kept, the rest 0
  for (int j = lane; j < a.nt; j += 64)
    if (!(live && j >= 1 && j < i)) row[j] = (live && (j == 0 || j == i)) ? 1 : 0;
  if (!live || ncand < 1) return;
  const int m = (int)(((int64_t)ncand * a.skip_per_mille) / 1000);
  if (m == 0) {
    for (int j = 1 + lane; j < i; j += 64) row[j] = 1;
    return;
  }
  const double* srow = a.score + (bg * a.nt + i) * a.nt;
  const int R = (ncand + 63) >> 6;
  if (R <= 1)       select_row<1>(srow, ncand, m, lane, row);
  else if (R <= 2)  select_row<2>(srow, ncand, m, lane, row);
  else if (R <= 4)  select_row<4>(srow, ncand, m, lane, row);
  else if (R <= 8)  select_row<8>(srow, ncand, m, lane, row);
  else if (R <= 16) select_row<16>(srow, ncand, m, lane, row);
  else              select_row<32>(srow, ncand, m, lane, row);
}

}  // namespace

hipError_t launch_tile_mask(const MaskGenArgs& a, hipStream_t s) {
  const unsigned units = (unsigned)(a.k.B * a.k.H * a.nt);
  hipLaunchKernelGGL(pool_q_kernel, dim3(units), dim3(POOL_THREADS), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(pool_k_kernel, dim3(units), dim3(POOL_THREADS), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nb = (a.nt + SB - 1) / SB;
  hipLaunchKernelGGL(score_kernel, dim3((unsigned)(a.k.B * a.k.H * (nb * (nb + 1) / 2))),
                     dim3(256), 0, s, a, nb);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned rows4 = (unsigned)(a.k.B * a.k.H * ((a.nt + 3) / 4));
  hipLaunchKernelGGL(select_kernel, dim3(rows4), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace taq
