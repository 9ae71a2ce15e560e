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
// A split that saw no key of a row has LSE_s = -inf and contributes nothing;
// a row with no key at all gets O = 0 and LSE = -inf.
//
// HBM-bound: one thread per (row, 4 channels) reads the splits' LSE values
// (the same few floats for all threads of a row, served from cache) and its
// 16 bytes of every partial, and writes 4 output elements.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kernels.h"

namespace attn {

template <typename T>
__global__ void __launch_bounds__(256) combine_kernel(CombineParams p) {
  const int c4n = p.d / 4;
  const long long rows = (long long)p.B * p.Sq * p.Hq;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= rows * c4n) return;
  const long long row = idx / c4n;          // token-major row: (b * Sq + i) * Hq + h
  const int c4 = (int)(idx % c4n);
  const int hq = (int)(row % p.Hq);
  const long long bi = row / p.Hq;
  const int i = (int)(bi % p.Sq);
  const int b = (int)(bi / p.Sq);
  const long long lse_idx = ((long long)b * p.Hq + hq) * p.Sq + i;
  const long long lplane = rows;            // LSE values per split
  const long long oplane = rows * p.d;      // O values per split

  float m = -__builtin_inff();
  for (int s = 0; s < p.splits; ++s) m = fmaxf(m, p.lse_part[s * lplane + lse_idx]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float wsum = 0.f;
  if (m != -__builtin_inff()) {
    for (int s = 0; s < p.splits; ++s) {
      const float ls = p.lse_part[s * lplane + lse_idx];
      if (ls == -__builtin_inff()) continue;
      const float w = expf(ls - m);
      const float4 v = *(const float4*)(p.o_part + s * oplane + row * p.d + 4 * c4);
      acc.x += w * v.x;
      acc.y += w * v.y;
      acc.z += w * v.z;
      acc.w += w * v.w;
      wsum += w;
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  typedef T T4 __attribute__((ext_vector_type(4)));
  T4 out;
  out[0] = (T)(acc.x * inv);
  out[1] = (T)(acc.y * inv);
  out[2] = (T)(acc.z * inv);
  out[3] = (T)(acc.w * inv);
  *(T4*)((T*)p.o + row * p.d + 4 * c4) = out;
  if (p.lse != nullptr && c4 == 0) p.lse[lse_idx] = wsum > 0.f ? m + logf(wsum) : -__builtin_inff();
}

hipError_t launch_combine(const CombineParams& p, int dtype, hipStream_t s) {
  const long long threads = (long long)p.B * p.Sq * p.Hq * (p.d / 4);
  const unsigned grid = (unsigned)((threads + 255) / 256);
  if (grid == 0) return hipSuccess;
  if (dtype == 0) hipLaunchKernelGGL(combine_kernel<__bf16>, dim3(grid), dim3(256), 0, s, p);
  else hipLaunchKernelGGL(combine_kernel<_Float16>, dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace attn
