// wide_regs.h -- register-level building blocks of the one-wave-per-SIMD
// forward kernel (attn_fwd_wide.hip).
//
// The kernel's key loop keeps its long-lived matrix operands in fixed
// accumulation registers (AGPRs), addressed by name in inline assembly:
//
//   a[  0:127]  O accumulators, block (qb, db) at a[16 (4 qb + db)]
//   a[128:159]  V fragments, buffer c, channel block db at a[128 + 4 (4 c + db)]
//   a[160:223]  Q fragments, block qb, k-step kk at a[160 + 4 (8 qb + kk)]
//   a[224:247]  K fragments, ring slot r, key block bb at a[224 + 4 (2 r + bb)]
//
// and leaves the vector registers (scores S, probabilities P, addresses,
// softmax state) to the compiler.  Naming the registers is what keeps the
// accumulators in place: left to its heuristics the compiler moves them
// between the two register files inside the loop.  The zeroing of O at the
// start lists every AGPR as clobbered, which makes the kernel reserve the
// whole AGPR file; the statements of the loop list none (a clobber list makes
// the compiler put a wait state after each statement).  The compiler itself
// must then never place a value in an AGPR: the build checks the generated
// code for that (no AGPR outside these statements, no spills).
//
// The compiler does not see inside these statements, so the hazards it would
// otherwise resolve are the caller's: all statements are volatile (program
// order is kept), a score block written by an MFMA is read by vector
// instructions only after eight further MFMA issues or an s_nop run, LDS and
// global results are consumed after an explicit s_waitcnt, and O is read only
// after an s_nop run (acc_read_pad).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kernel_common.h"

namespace attn {
namespace wide {

// Compile-time assembly text.
struct Asm {
  char buf[4096] = {};
  unsigned n = 0;
  constexpr Asm& s(const char* p) {
    while (*p) buf[n++] = *p++;
    return *this;
  }
  constexpr Asm& i(int v) {
    char t[12] = {};
    int k = 0;
    if (v == 0) t[k++] = '0';
    while (v > 0) {
      t[k++] = (char)('0' + v % 10);
      v /= 10;
    }
    while (k > 0) buf[n++] = t[--k];
    return *this;
  }
  // a[lo:lo+cnt-1]
  constexpr Asm& a(int lo, int cnt) { return s("a[").i(lo).s(":").i(lo + cnt - 1).s("]"); }
  constexpr const char* data() const { return buf; }
  constexpr unsigned size() const { return n; }
};

constexpr int kO = 0, kV = 128, kQ = 160, kK = 224;
constexpr int o_reg(int qb, int db) { return kO + 16 * (4 * qb + db); }
constexpr int v_reg(int c, int db) { return kV + 4 * (4 * c + db); }
constexpr int q_reg(int qb, int kk) { return kQ + 4 * (8 * qb + kk); }
constexpr int k_reg(int r, int bb) { return kK + 4 * (2 * r + bb); }

#define ATTN_AGPRS_10(b)                                                                          \
  "a" #b "0", "a" #b "1", "a" #b "2", "a" #b "3", "a" #b "4", "a" #b "5", "a" #b "6", "a" #b "7", \
      "a" #b "8", "a" #b "9"
#define ATTN_CLOBBER_AGPRS                                                                                   \
  "a0", "a1", "a2", "a3", "a4", "a5", "a6", "a7", "a8", "a9", ATTN_AGPRS_10(1), ATTN_AGPRS_10(2), ATTN_AGPRS_10(3), \
      ATTN_AGPRS_10(4), ATTN_AGPRS_10(5), ATTN_AGPRS_10(6), ATTN_AGPRS_10(7), ATTN_AGPRS_10(8), ATTN_AGPRS_10(9),         \
      ATTN_AGPRS_10(10), ATTN_AGPRS_10(11), ATTN_AGPRS_10(12), ATTN_AGPRS_10(13), ATTN_AGPRS_10(14), ATTN_AGPRS_10(15),   \
      ATTN_AGPRS_10(16), ATTN_AGPRS_10(17), ATTN_AGPRS_10(18), ATTN_AGPRS_10(19), ATTN_AGPRS_10(20), ATTN_AGPRS_10(21),   \
      ATTN_AGPRS_10(22), ATTN_AGPRS_10(23), ATTN_AGPRS_10(24), "a250", "a251", "a252", "a253", "a254", "a255"

template <typename T>
constexpr const char* mfma_name() {
  return std::is_same<T, __bf16>::value ? "v_mfma_f32_32x32x16_bf16 " : "v_mfma_f32_32x32x16_f16 ";
}

// ---------------------------------------------------------------- O
// a[0:127] = 0
constexpr Asm o_zero_text() {
  Asm t;
  for (int r = 0; r < 128; ++r) t.s("v_accvgpr_write_b32 a").i(r).s(", 0\n\t");
  return t;
}
__device__ __forceinline__ void o_zero() { asm volatile((o_zero_text())::: ATTN_CLOBBER_AGPRS); }

// O block += V fragment x P (P: B operand in VGPRs)
template <typename T, int QB, int DB, int C>
constexpr Asm mfma_o_text() {
  Asm t;
  t.s(mfma_name<T>()).a(o_reg(QB, DB), 16).s(", ").a(v_reg(C, DB), 4).s(", %0, ").a(o_reg(QB, DB), 16);
  return t;
}
template <typename T, int QB, int DB, int C, typename P8>
__device__ __forceinline__ void mfma_o(const P8& p) {
  asm volatile((mfma_o_text<T, QB, DB, C>())::"v"(p));
}

// O block (qb, db) *= f.  The leading s_nops cover the MFMA-write ->
// accvgpr-read distance, the trailing one the accvgpr-write -> MFMA-read one.
template <int QB, int DB>
constexpr Asm acc_scale_text() {
  Asm t;
  t.s("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\t");
  for (int r = o_reg(QB, DB); r < o_reg(QB, DB) + 16; ++r) {
    t.s("v_accvgpr_read_b32 %0, a").i(r).s("\n\tv_mul_f32 %0, %1, %0\n\tv_accvgpr_write_b32 a").i(r).s(", %0\n\t");
  }
  t.s("s_nop 7");
  return t;
}
template <int QB, int DB>
__device__ __forceinline__ void acc_scale(float f) {
  float tmp;
  asm volatile((acc_scale_text<QB, DB>()) : "=&v"(tmp) : "v"(f));
}

// s_nop run after the last MFMA, before O is read
__device__ __forceinline__ void acc_read_pad() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

// O block (qb, db) -> 16 floats
template <int QB, int DB>
constexpr Asm acc_read_text() {
  Asm t;
  for (int e = 0; e < 16; ++e) {
    t.s("v_accvgpr_read_b32 %").i(e).s(", a").i(o_reg(QB, DB) + e);
    if (e < 15) t.s("\n\t");
  }
  return t;
}
template <int QB, int DB>
__device__ __forceinline__ f32x16 acc_read() {
  float x0, x1, x2, x3, x4, x5, x6, x7, x8, x9, x10, x11, x12, x13, x14, x15;
  asm volatile((acc_read_text<QB, DB>())
               : "=v"(x0), "=v"(x1), "=v"(x2), "=v"(x3), "=v"(x4), "=v"(x5), "=v"(x6), "=v"(x7), "=v"(x8),
                 "=v"(x9), "=v"(x10), "=v"(x11), "=v"(x12), "=v"(x13), "=v"(x14), "=v"(x15));
  return f32x16{x0, x1, x2, x3, x4, x5, x6, x7, x8, x9, x10, x11, x12, x13, x14, x15};
}

// ---------------------------------------------------------------- Q
template <int QB, int KK>
constexpr Asm q_load_text() {
  Asm t;
  t.s("global_load_dwordx4 ").a(q_reg(QB, KK), 4).s(", %0, off");
  return t;
}
template <int QB, int KK>
__device__ __forceinline__ void q_load(const void* ptr) {
  asm volatile((q_load_text<QB, KK>())::"v"(ptr) : "memory");
}

// ---------------------------------------------------------------- K, V reads
template <int R, int BB, int OFF>
constexpr Asm k_read_text() {
  Asm t;
  t.s("ds_read_b128 ").a(k_reg(R, BB), 4).s(", %0 offset:").i(OFF);
  return t;
}
template <int R, int BB, int OFF>
__device__ __forceinline__ void k_read(uint32_t addr) {
  asm volatile((k_read_text<R, BB, OFF>())::"v"(addr));
}

// V fragment (c, db): two transposing reads, rows r and r + 4 of the chunk
template <int C, int DB, int OFF, int OFF2>
constexpr Asm v_read_text() {
  Asm t;
  t.s("ds_read_b64_tr_b16 ").a(v_reg(C, DB), 2).s(", %0 offset:").i(OFF);
  t.s("\n\tds_read_b64_tr_b16 ").a(v_reg(C, DB) + 2, 2).s(", %0 offset:").i(OFF + OFF2);
  return t;
}
template <int C, int DB, int OFF, int OFF2>
__device__ __forceinline__ void v_read(uint32_t addr) {
  asm volatile((v_read_text<C, DB, OFF, OFF2>())::"v"(addr));
}

// V fragment (c, db) from a column-major V tile: one plain 16-byte read of
// 8 consecutive keys of one channel row
template <int C, int DB, int OFF>
constexpr Asm vcol_read_text() {
  Asm t;
  t.s("ds_read_b128 ").a(v_reg(C, DB), 4).s(", %0 offset:").i(OFF);
  return t;
}
template <int C, int DB, int OFF>
__device__ __forceinline__ void vcol_read(uint32_t addr) {
  asm volatile((vcol_read_text<C, DB, OFF>())::"v"(addr));
}

// at most N LDS operations outstanding
template <int N>
__device__ __forceinline__ void lgkm_wait() {
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N) : "memory");
}

// ---------------------------------------------------------------- S
// S block (VGPRs) = / += K fragment x Q fragment
template <typename T, bool FIRST, int R, int BB, int QB, int KK>
constexpr Asm mfma_s_text() {
  Asm t;
  t.s(mfma_name<T>()).s("%0, ").a(k_reg(R, BB), 4).s(", ").a(q_reg(QB, KK), 4).s(FIRST ? ", 0" : ", %0");
  return t;
}
template <typename T, bool FIRST, int R, int BB, int QB, int KK>
__device__ __forceinline__ void mfma_s(f32x16& s) {
  if constexpr (FIRST) asm volatile((mfma_s_text<T, true, R, BB, QB, KK>()) : "=v"(s) :);
  else asm volatile((mfma_s_text<T, false, R, BB, QB, KK>()) : "+v"(s) :);
}

// Orders vector reads of S after this point (no instructions)
__device__ __forceinline__ void tie_s(f32x16 (&s)[2][2]) {
  asm volatile("" : "+v"(s[0][0]), "+v"(s[0][1]), "+v"(s[1][0]), "+v"(s[1][1]));
}
// Same, after an s_nop run long enough for the MFMA results to land
__device__ __forceinline__ void pad_s(f32x16 (&s)[2][2]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s[0][0]), "+v"(s[0][1]), "+v"(s[1][0]), "+v"(s[1][1]));
}

}  // namespace wide
}  // namespace attn
