// bwd_regs.h -- inline-assembly pieces of the backward kernels that keep
// their accumulators and fixed MFMA operands in named AGPRs
// (attn_bwd_dkdv.hip, attn_bwd_dq.hip).  As in the forward's wide kernel
// (wide_regs.h): the compiler does not read the assembly text, so a zeroing
// statement at kernel start clobbers the AGPRs a map uses, and the build
// checks that the compiler itself touches no AGPR in these files.
#pragma once

#include <hip/hip_runtime.h>

#include <utility>

#include "kernel_common.h"
#include "wide_regs.h"

namespace attn {
namespace breg {

using wide::Asm;

template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  [&]<int... I>(std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
  }(std::make_integer_sequence<int, N>{});
}

// 16 bytes from global memory -> a[BASE + 4 KK : + 4]
template <int BASE, int KK>
constexpr Asm frag_load_text() {
  Asm t;
  t.s("global_load_dwordx4 ").a(BASE + 4 * KK, 4).s(", %0, off");
  return t;
}
template <int BASE, int KK>
__device__ __forceinline__ void frag_load(const void* ptr) {
  asm volatile((frag_load_text<BASE, KK>())::"v"(ptr) : "memory");
}

#define BREG_CLOBBER_AGPRS_64                                                                             \
  "a0", "a1", "a2", "a3", "a4", "a5", "a6", "a7", "a8", "a9", ATTN_AGPRS_10(1), ATTN_AGPRS_10(2),         \
      ATTN_AGPRS_10(3), ATTN_AGPRS_10(4), ATTN_AGPRS_10(5), "a60", "a61", "a62", "a63"
#define BREG_CLOBBER_AGPRS_96                                                                             \
  "a0", "a1", "a2", "a3", "a4", "a5", "a6", "a7", "a8", "a9", ATTN_AGPRS_10(1), ATTN_AGPRS_10(2),         \
      ATTN_AGPRS_10(3), ATTN_AGPRS_10(4), ATTN_AGPRS_10(5), ATTN_AGPRS_10(6), ATTN_AGPRS_10(7), ATTN_AGPRS_10(8), \
      "a90", "a91", "a92", "a93", "a94", "a95"

// a[0 : N) = 0, reserving a[0 : USED) (64, 96, or the whole file)
template <int N>
constexpr Asm zero_text() {
  Asm t;
  for (int r = 0; r < N; ++r) t.s("v_accvgpr_write_b32 a").i(r).s(", 0\n\t");
  return t;
}
// At a three-waves-per-SIMD budget (d = 64 dK/dV) the compiler's own AGPR
// share is 84 of the 168 registers, so it calls a84..a95 of this list
// reserved and warns: it then never allocates them, and the kernel
// descriptor still counts every AGPR the assembly names (build.py fails the
// build if a named AGPR lies outside the descriptor's allocation).
template <int N, int USED>
__device__ __forceinline__ void acc_zero() {
  static_assert(N <= USED, "");
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  if constexpr (USED == 64) asm volatile((zero_text<N>())::: BREG_CLOBBER_AGPRS_64);
  else if constexpr (USED == 96) asm volatile((zero_text<N>())::: BREG_CLOBBER_AGPRS_96);
  else asm volatile((zero_text<N>())::: ATTN_CLOBBER_AGPRS);
#pragma clang diagnostic pop
}

// acc (VGPRs) = / += A (VGPR) x fragment k-step KK at a[BASE + 4 KK] (B operand)
template <typename T, int BASE, int KK, bool FIRST>
constexpr Asm first_text() {
  Asm t;
  t.s(wide::mfma_name<T>()).s("%0, %1, ").a(BASE + 4 * KK, 4).s(FIRST ? ", 0" : ", %0");
  return t;
}
template <typename T, int BASE, int KK, bool FIRST, typename V8>
__device__ __forceinline__ void mfma_first(f32x16& acc, const V8& a) {
  if constexpr (FIRST) asm volatile((first_text<T, BASE, KK, true>()) : "=&v"(acc) : "v"(a));
  else asm volatile((first_text<T, BASE, KK, false>()) : "+v"(acc) : "v"(a));
}

// accumulator block a[ACC : + 16] += A (VGPR) x B (VGPR)
template <typename T, int ACC>
constexpr Asm acc_text() {
  Asm t;
  t.s(wide::mfma_name<T>()).a(ACC, 16).s(", %0, %1, ").a(ACC, 16);
  return t;
}
template <typename T, int ACC, typename V8>
__device__ __forceinline__ void mfma_acc(const V8& a, const V8& b) {
  asm volatile((acc_text<T, ACC>())::"v"(a), "v"(b));
}

// s_nop run after MFMAs before their results are read by vector code
__device__ __forceinline__ void pad2(f32x16& x, f32x16& y) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(x), "+v"(y));
}

template <int ACC>
constexpr Asm read_text() {
  Asm t;
  for (int e = 0; e < 16; ++e) {
    t.s("v_accvgpr_read_b32 %").i(e).s(", a").i(ACC + e);
    if (e < 15) t.s("\n\t");
  }
  return t;
}
// a[ACC : + 16] -> VGPRs (after an s_nop run behind the last MFMA)
template <int ACC>
__device__ __forceinline__ f32x16 acc_read() {
  float x0, x1, x2, x3, x4, x5, x6, x7, x8, x9, x10, x11, x12, x13, x14, x15;
  asm volatile((read_text<ACC>())
               : "=v"(x0), "=v"(x1), "=v"(x2), "=v"(x3), "=v"(x4), "=v"(x5), "=v"(x6), "=v"(x7), "=v"(x8),
                 "=v"(x9), "=v"(x10), "=v"(x11), "=v"(x12), "=v"(x13), "=v"(x14), "=v"(x15));
  return f32x16{x0, x1, x2, x3, x4, x5, x6, x7, x8, x9, x10, x11, x12, x13, x14, x15};
}

}  // namespace breg
}  // namespace attn
