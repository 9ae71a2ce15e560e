// attn_bwd.hip -- attention backward for bf16 / fp16, d in {64, 128}, dense,
// causal or not, GQA.
//
// Gradient math (the backward listed in the Hopper tag page, contents 7.1 --
// 7.1.5; the chain rule through O = softmax(scale Q K^T + mask) V):
//   P = exp(scale S - LSE) recomputed from the forward's LSE (no max pass),
//   dV = P^T dO,  dP = dO V^T,  dS = P (dP - delta),  delta_i = dO_i . O_i
//   (minus dLSE_i when the LSE output has a gradient),
//   dQ = scale dS K,  dK = scale dS^T Q.
//
// Three kernels:
//   bwd_pre_kernel   per query row: (LSE log2 e, delta) into a small fp32
//                    array [B, Hq, Sq_pad] (the preprocess of contents
//                    7.3.1), padded to 32 rows per head.  This file.
//   dK / dV          one workgroup per (batch, KV head, 128 keys); each wave
//                    owns 32 keys and keeps their K, V fragments and dK, dV
//                    accumulators in registers, and walks the query blocks of
//                    every query head of the KV group (so GQA sums in
//                    registers and no atomics are needed).  Per 32-query step:
//                    S = Q K^T and dP = dO V^T (query rows x keys, so the
//                    accumulator of each is directly the B operand of the
//                    next MFMAs), P, dS, then dV^T += dO^T P and
//                    dK^T += Q^T dS with the transposed operands read from
//                    LDS by ds_read_b64_tr_b16.  attn_bwd_dkdv.hip.
//   dQ               one workgroup per (batch, query head, 128 query rows),
//                    like the forward: S^T = K Q^T, dP^T = V dO^T (a lane
//                    owns a query, so LSE and delta are lane scalars),
//                    dS^T, then dQ^T += K^T dS^T.  attn_bwd_dq.hip.
// The pages resolve the dQ race across key blocks with atomics or
// semaphores (contents 7.2.3, 7.6); here dQ has a kernel of its own, which
// recomputes S and dP (7 GEMMs instead of 5) and is deterministic.
//
// Operand layouts follow the forward kernels: v_mfma_f32_32x32x16, lane l
// supplies row l % 32 and 8 consecutive k values 8 (l / 32) .. + 7; the first
// GEMM's rows are permuted (key_perm) so that its accumulator registers,
// taken 8 at a time, are the next GEMM's B operand in natural order.
// Tiles move global -> LDS with buffer_load ... lds; a tile read both ways is
// stored twice, once with the row-read swizzle and once with the
// transposed-read swizzle, so neither access has bank conflicts.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "kernel_common.h"
#include "kernels.h"

namespace attn {

// ---------------------------------------------------------------- preprocess
// D/8 consecutive threads own one row (16 bytes of o and dO each, one
// coalesced row per thread group) and sum their partial dot products with
// shuffles.  Rows i in [Sq, Sq_pad) of the statistics get (+inf, 0): P = 0
// there; so do the 32 spare pairs past the array (the varlen dK/dV kernel
// reads a step's 32 rows from one address, past the last token on the last
// head).
template <typename T, int D>
__global__ void __launch_bounds__(256) bwd_pre_kernel(BwdParams p) {
  typedef typename Mma<T>::vec8 vec8;
  constexpr int TPR = D / 8;                 // threads per row
  const long long rows = (long long)p.B * p.Sq_pad * p.Hq;
  const long long rp = ((long long)blockIdx.x * 256 + threadIdx.x) / TPR;   // (b * Sq_pad + i) * Hq + h
  const int t = threadIdx.x % TPR;
  if (rp >= rows) {                          // whole thread groups leave together
    if (t == 0 && rp < rows + 32) p.stats[rp] = make_float2(__builtin_inff(), 0.f);
    return;
  }
  const int hq = (int)(rp % p.Hq);
  const long long bi = rp / p.Hq;
  const int i = (int)(bi % p.Sq_pad);
  const int b = (int)(bi / p.Sq_pad);
  const long long li = ((long long)b * p.Hq + hq) * p.Sq_pad + i;
  if (i >= p.Sq) {
    if (t == 0) p.stats[li] = make_float2(__builtin_inff(), 0.f);
    return;
  }
  const long long r = ((long long)b * p.Sq + i) * p.Hq + hq;        // token-major row of o, dO
  const vec8 x = *(const vec8*)((const T*)p.o + r * D + 8 * t);
  const vec8 y = *(const vec8*)((const T*)p.dout + r * D + 8 * t);
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)x[e], (float)y[e], acc);
#pragma unroll
  for (int o = TPR / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, TPR);
  if (t != 0) return;
  const long long lo = ((long long)b * p.Hq + hq) * p.Sq + i;       // index in lse, dlse
  if (p.dlse != nullptr) acc -= p.dlse[lo];
  const float l = p.lse[lo];
  // a row that saw no key has LSE = -inf and P = 0: +inf makes exp2 give 0
  const float l2 = (l == -__builtin_inff()) ? __builtin_inff() : l * 1.4426950408889634f;
  p.stats[li] = make_float2(l2, acc);
}

// ---------------------------------------------------------------- launch
template <typename T, int D, bool CAUSAL, bool VARLEN>
static hipError_t launch_bwd_t(const BwdParams& p, hipStream_t s) {
  // the preprocess sees a varlen batch as one sequence of T tokens ([Hq, T])
  BwdParams pp = p;
  if (VARLEN) {
    pp.B = 1;
    pp.Sq_pad = p.Sq;
  }
  const long long threads = ((long long)pp.B * pp.Sq_pad * pp.Hq + 32) * (D / 8);
  hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, pp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_bwd_dkdv(p, std::is_same<T, __bf16>::value ? 0 : 1, D, CAUSAL, VARLEN, s);
  if (e != hipSuccess) return e;
  return launch_bwd_dq(p, std::is_same<T, __bf16>::value ? 0 : 1, D, CAUSAL, VARLEN, s);
}

template <typename T, int D>
static hipError_t launch_bwd_v(const BwdParams& p, int causal, int varlen, hipStream_t s) {
  if (varlen) return causal ? launch_bwd_t<T, D, true, true>(p, s) : launch_bwd_t<T, D, false, true>(p, s);
  return causal ? launch_bwd_t<T, D, true, false>(p, s) : launch_bwd_t<T, D, false, false>(p, s);
}

hipError_t launch_bwd(const BwdParams& p, int dtype, int d, int causal, int varlen, hipStream_t s) {
  if (dtype == 0) return d == 128 ? launch_bwd_v<__bf16, 128>(p, causal, varlen, s) : launch_bwd_v<__bf16, 64>(p, causal, varlen, s);
  return d == 128 ? launch_bwd_v<_Float16, 128>(p, causal, varlen, s) : launch_bwd_v<_Float16, 64>(p, causal, varlen, s);
}

}  // namespace attn
