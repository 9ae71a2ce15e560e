// kernel_common.h -- device helpers shared by the attention kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

#define LDS_AS __attribute__((address_space(3)))

// Word 3 of a raw buffer resource on gfx9-family parts: 32-bit data format,
// no swizzle, no stride; out-of-range reads return zero.
constexpr int kBufferFlags = 0x00020000;

// Row order of keys in the first MFMA: MFMA row r reads key pi(r) of its
// 32-key block, pi swapping bits 2 and 3.
__device__ __forceinline__ int key_perm(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

__device__ __forceinline__ float wave_half_swap(float x) {
  // value of lane l ^ 32
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  const int lane = threadIdx.x & 63;
  return __int_as_float(lane < 32 ? r[1] : r[0]);
}

// N direct-to-LDS copies of 16 bytes per lane (buffer_load_dwordx4 ... lds):
// copy i writes LDS bytes [dst + 1024 i, dst + 1024 (i + 1)), lane L the 16
// bytes at offset 16 L, fetched from base + off[i].  Reads at or past `bytes`
// return zeros (the buffer range check).
template <int N>
__device__ __forceinline__ void copy_rows_to_lds(const void* base, uint32_t bytes, char* dst,
                                                 const uint32_t (&off)[N]) {
#if defined(__HIP_DEVICE_COMPILE__)
  // (the buffer-resource type exists only in the device pass of the compiler)
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferFlags);
#pragma unroll
  for (int i = 0; i < N; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (LDS_AS void*)(dst + i * 1024), 16, off[i], 0, 0, 0);
#endif
}

// Empty uses that pin a computed value at this point of the program: without
// them the compiler sinks the exponentials of one MFMA stretch down to their
// first use in a later stretch, undoing the interleave.
__device__ __forceinline__ void keep(float x) { asm volatile("" ::"v"(x)); }
template <typename V>
__device__ __forceinline__ void keep_vec(const V& x) {
  asm volatile("" ::"v"(x));
}

// Transposing LDS read (ds_read_b64_tr_b16) issued as inline assembly: the
// compiler does not see it as an LDS access, so it does not make it wait for
// the K/V copies of the next tile that are still in flight.  The caller waits
// for the result with lds_wait().
template <int OFF>
__device__ __forceinline__ i16x4 lds_tr16(uint32_t addr) {
  i16x4 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}

// Wait until at most LEFT LDS operations are outstanding, then consider r
// valid.  LDS operations complete in order, so with LEFT = the number of LDS
// reads issued after r's, r is complete.
template <int LEFT, int N>
__device__ __forceinline__ void lds_wait(i16x4 (&r)[N]) {
  if constexpr (N == 8) {
    asm volatile("s_waitcnt lgkmcnt(%8)"
                 : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]), "+v"(r[6]),
                   "+v"(r[7])
                 : "n"(LEFT));
  } else {
    static_assert(N == 4, "");
    asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]) : "n"(LEFT));
  }
}


}  // namespace attn
