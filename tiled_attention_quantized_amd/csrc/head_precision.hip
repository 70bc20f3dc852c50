// Per-KV-head precision assignment from measured sensitivity.
//
// "分块稀疏注意力与KV Cache量化：长文本推理显存优化实践" (xdnf.cn), section 2.4:
// each attention head carries a sensitivity score, sensitive heads keep the
// higher precision and the rest are stored with fewer bits (section 3.4: more
// high-precision heads, less memory saved).  The score of KV head g is how far
// its decode outputs move when its cache drops from int8 to int4,
//   S_g = sum over batch entries b, the query heads h of g and channels d of
//         (O4[b][h][d] - O8[b][h][d])^2,
// for calibration queries; the n_high largest scores get 8 bits (ties: lower
// g), the rest 4.  The two decode outputs come from the library's own
// quantise and decode kernels; this file holds the reduction and the choice.
#include "taq_internal.h"
#include "device_common.h"

namespace taq {
namespace {

constexpr int SENS_THREADS = 256;

// One workgroup per KV head: each thread sums its elements in fp64, then a
// fixed-order tree in LDS (the result is repeatable bit for bit).
__global__ void __launch_bounds__(SENS_THREADS)
sensitivity_kernel(const uint16_t* o8, const uint16_t* o4, int B, int Hq, int r,
                   double* scores) {
  __shared__ double part[SENS_THREADS];
  const int g = blockIdx.x;
  const int per_b = r * 128;
  double acc = 0.0;
  for (int e = threadIdx.x; e < B * per_b; e += SENS_THREADS) {
    const int b = e / per_b, rem = e - b * per_b;
    const int64_t idx = ((int64_t)b * Hq + g * r) * 128 + rem;   // heads g*r .. g*r+r-1
    const double diff = (double)(float)bits_to_half(o4[idx]) - (double)(float)bits_to_half(o8[idx]);
    acc += diff * diff;
  }
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int w = SENS_THREADS / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) scores[g] = part[0];
}

// One wave: lane g ranks its head by counting the heads ahead of it.
__global__ void __launch_bounds__(64)
assign_kernel(const double* scores, int H, int n_high, uint8_t* bits) {
  const int g = threadIdx.x;
  if (g >= H) return;
  const double s = scores[g];
  int rank = 0;
  for (int h = 0; h < H; ++h) {
    const double t = scores[h];
    rank += (t > s || (t == s && h < g)) ? 1 : 0;
  }
  bits[g] = rank < n_high ? 8 : 4;
}

}  // namespace

hipError_t launch_head_assign(const uint16_t* o8, const uint16_t* o4, int B, int Hq, int Hkv,
                              int n_high, double* scores, uint8_t* bits, hipStream_t s) {
  hipLaunchKernelGGL(sensitivity_kernel, dim3(Hkv), dim3(SENS_THREADS), 0, s, o8, o4, B, Hq,
                     Hq / Hkv, scores);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(assign_kernel, dim3(1), dim3(64), 0, s, scores, Hkv, n_high, bits);
  return hipGetLastError();
}

}  // namespace taq
