// attn_combine.hip -- merge of split-KV partial results (flash-decoding).
//
// Each split s of the key axis leaves, per query row, a normalised partial
// output O_s and its log-sum-exp LSE_s.  The result over all keys is the
// block-combine of the streaming softmax (Hopper tag page, contents 3.2.1, and
// the split-KV combine, contents 10.2.1):
//
//     m = max_s LSE_s,  w_s = exp(LSE_s - m),  LSE = m + log sum_s w_s,
//     O = sum_s w_s O_s / sum_s w_s
//
// A split that saw no key of a row has LSE_s = -inf and contributes nothing
// (its O_s is never used, whatever it holds); a row with no key at all gets
// O = 0 and LSE = -inf.
//
// HBM-bound and short: the partials of a decode step are a few MiB, so the
// kernel is built for memory-level parallelism rather than for many rows.
// D/4 consecutive threads own one row (4 channels each).  They read the row's
// LSE values with a stride of D/4 splits, reduce max and sum across the row's
// lanes with shuffles, and leave the weights in LDS; then every thread sums
// its 4 channels over all splits with unconditional, unrolled loads (a weight
// of 0 selects nothing, so the loads need no branch and stay in flight
// together).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kernels.h"

namespace attn {

template <int W>
__device__ __forceinline__ float row_max(float x) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, W));
  return x;
}
template <int W>
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) x += __shfl_xor(x, o, W);
  return x;
}

template <typename T, int D>
__global__ void __launch_bounds__(256) combine_kernel(CombineParams p) {
  constexpr int TPR = D / 4;        // threads per row
  constexpr int RPB = 256 / TPR;    // rows per workgroup
  constexpr float NEG_INF = -__builtin_inff();
  __shared__ float wsh[RPB][kCombineMaxSplits];

  const int t = threadIdx.x % TPR;
  const int rl = threadIdx.x / TPR;
  const long long rows = (long long)p.B * p.Sq * p.Hq;
  const long long row = (long long)blockIdx.x * RPB + rl;   // token-major: (b * Sq + i) * Hq + h
  const bool valid = row < rows;
  const long long r = valid ? row : rows - 1;               // keeps every address in bounds
  const int hq = (int)(r % p.Hq);
  const long long bi = r / p.Hq;
  const int i = (int)(bi % p.Sq);
  const int b = (int)(bi / p.Sq);
  const long long lse_idx = ((long long)b * p.Hq + hq) * p.Sq + i;
  const long long lplane = rows;        // LSE values per split
  const long long oplane = rows * D;    // O values per split

  float m = NEG_INF;
  for (int s = t; s < p.splits; s += TPR) m = fmaxf(m, p.lse_part[s * lplane + lse_idx]);
  m = row_max<TPR>(m);
  const float m_safe = (m == NEG_INF) ? 0.f : m;
  float wsum = 0.f;
  for (int s = t; s < p.splits; s += TPR) {
    const float ls = p.lse_part[s * lplane + lse_idx];
    const float w = (ls == NEG_INF) ? 0.f : expf(ls - m_safe);
    wsh[rl][s] = w;
    wsum += w;
  }
  wsum = row_sum<TPR>(wsum);
  __syncthreads();

  const float* op = p.o_part + r * D + 4 * t;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
  for (int s = 0; s < p.splits; ++s) {
    const float4 v = *(const float4*)(op + s * oplane);
    const float w = wsh[rl][s];
    const bool use = w != 0.f;
    acc.x += use ? w * v.x : 0.f;
    acc.y += use ? w * v.y : 0.f;
    acc.z += use ? w * v.z : 0.f;
    acc.w += use ? w * v.w : 0.f;
  }
  if (!valid) return;
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  typedef T T4 __attribute__((ext_vector_type(4)));
  T4 out;
  out[0] = (T)(acc.x * inv);
  out[1] = (T)(acc.y * inv);
  out[2] = (T)(acc.z * inv);
  out[3] = (T)(acc.w * inv);
  *(T4*)((T*)p.o + r * D + 4 * t) = out;
  if (p.lse != nullptr && t == 0) p.lse[lse_idx] = wsum > 0.f ? m + logf(wsum) : NEG_INF;
}

template <typename T, int D>
static hipError_t launch_combine_t(const CombineParams& p, hipStream_t s) {
  constexpr int RPB = 256 / (D / 4);
  const long long rows = (long long)p.B * p.Sq * p.Hq;
  const unsigned grid = (unsigned)((rows + RPB - 1) / RPB);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((combine_kernel<T, D>), dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineParams& p, int dtype, hipStream_t s) {
  if (dtype == 0) return p.d == 128 ? launch_combine_t<__bf16, 128>(p, s) : launch_combine_t<__bf16, 64>(p, s);
  return p.d == 128 ? launch_combine_t<_Float16, 128>(p, s) : launch_combine_t<_Float16, 64>(p, s);
}

}  // namespace attn
