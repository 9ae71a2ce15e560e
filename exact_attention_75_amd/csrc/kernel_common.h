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
typedef int i32x4 __attribute__((ext_vector_type(4)));

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

// Debug build (-DATTN_DEBUG_POISON): every copy into an LDS stage first
// fills the bytes it is about to write with 0xFF (NaN in bf16, fp16 and e4m3)
// and waits for that write.  A copy is issued only once its stage has been
// released (the barrier that ends the stage's last reads), so a read of a
// stage after its release sees NaN at once, where the normal build would
// still return the old tile's values until the copy lands.  Without such a
// read the results are bit-identical to the normal build's; only the timing
// moves.
template <int N>
__device__ __forceinline__ void poison_stage(char* dst) {
#if defined(ATTN_DEBUG_POISON) && defined(__HIP_DEVICE_COMPILE__)
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < N; ++i) *(LDS_AS i32x4*)(dst + i * 1024 + 16 * lane) = i32x4{-1, -1, -1, -1};
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#endif
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
  // base and size are uniform; saying so keeps the resource in SGPRs even
  // when they were computed with vector instructions
  const uint64_t b64 = (uint64_t)(uintptr_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b64);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b64 >> 32));
  void* const ub = (void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      ub, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), kBufferFlags);
  poison_stage<N>(dst);
#pragma unroll
  for (int i = 0; i < N; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (LDS_AS void*)(dst + i * 1024), 16, off[i], 0, 0, 0);
#endif
}

// One direct-to-LDS copy of 16 bytes per lane: LDS bytes [dst, dst + 1024),
// lane L the 16 bytes at offset 16 L, fetched from base + off (zeros at or
// past `bytes`).
__device__ __forceinline__ void copy_row_to_lds(const void* base, uint32_t bytes, char* dst, uint32_t off) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint64_t b64 = (uint64_t)(uintptr_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b64);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b64 >> 32));
  void* const ub = (void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      ub, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), kBufferFlags);
  poison_stage<1>(dst);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (LDS_AS void*)dst, 16, off, 0, 0, 0);
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
  } else if constexpr (N == 4) {
    asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]) : "n"(LEFT));
  } else {
    static_assert(N == 2, "");
    asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(r[0]), "+v"(r[1]) : "n"(LEFT));
  }
}

// 8-byte LDS read issued as inline assembly (ds_read_b64), waited for like
// lds_tr16.
template <int OFF>
__device__ __forceinline__ i16x4 lds_rd64(uint32_t addr) {
  i16x4 r;
  asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}


// 16-byte LDS read issued as inline assembly (ds_read_b128), for the same
// reason as lds_tr16; wait for it with lds_wait().
template <int OFF>
__device__ __forceinline__ i32x4 lds_rd128(uint32_t addr) {
  i32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}

template <int LEFT>
__device__ __forceinline__ void lds_wait(i32x4 (&r)[2]) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(r[0]), "+v"(r[1]) : "n"(LEFT));
}

// MFMA 32x32x16 with fp32 accumulation for the two 16-bit input types.
template <typename T>
struct Mma;

template <>
struct Mma<__bf16> {
  typedef bf16x8 vec8;
  static __device__ __forceinline__ f32x16 run(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Mma<_Float16> {
  typedef f16x8 vec8;
  static __device__ __forceinline__ f32x16 run(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

// Ragged batches: the workgroup of rank r among the (sequence, block)
// entries of a batch of B sequences packed by cu (blocks of BM rows), ranked
// longest first.  Causal: a block at level m costs about m + 1 block-widths
// of work (the query block m of the forward and of dQ, the key block
// nb - 1 - m of dK/dV), so the entries run over m descending, sequences
// ascending within one m; lane m counts the entries at level >= m and a
// ballot finds the level of rank r.  Full attention: every block of a
// sequence costs the sequence's length, so whole sequences go longest first
// (ties by index) and level = the block's index in its sequence.  Lane l reads
// sequence l's bounds (one coalesced load).  Handles up to 64 sequences of up
// to 64 blocks and then returns true, with seq = -1 when r is past the last
// entry; otherwise returns false and the caller walks the batch.  Results are
// wave-uniform.
struct VarlenEntry {
  int seq, level, start, len;
};
template <int BM, bool CAUSAL>
__device__ __forceinline__ bool varlen_rank(const int32_t* cu, int B, int r, VarlenEntry& e) {
  if (B > 64) return false;
  const int lane = threadIdx.x & 63;
  const int c0 = lane < B ? cu[lane] : 0;
  const int c1 = lane < B ? cu[lane + 1] : 0;
  const int nb_l = (c1 - c0 + BM - 1) / BM;
  e.seq = -1;
  e.level = 0;
  if constexpr (CAUSAL) {
    int cnt = 0, mx = 0;
    for (int j = 0; j < B; ++j) {
      const int nbj = __builtin_amdgcn_readlane(nb_l, j);
      mx = max(mx, nbj);
      cnt += max(0, nbj - lane);
    }
    if (mx > 64) return false;
    const int m = __builtin_popcountll(__builtin_amdgcn_ballot_w64(cnt > r)) - 1;   // -1: no entry
    if (m >= 0) {
      const int k = r - (m + 1 < 64 ? __builtin_amdgcn_readlane(cnt, m + 1) : 0);
      const bool has = lane < B && nb_l > m;
      const uint64_t hb = __builtin_amdgcn_ballot_w64(has);
      const int below = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(hb >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)hb, 0u));
      e.seq = (int)__builtin_ctzll(__builtin_amdgcn_ballot_w64(has && below == k));
      e.level = m;
    }
  } else {
    int base = 0;
    for (int j = 0; j < B; ++j) {
      const int nbj = __builtin_amdgcn_readlane(nb_l, j);
      base += (nbj > nb_l || (nbj == nb_l && j < lane)) ? nbj : 0;
    }
    const uint64_t hit = __builtin_amdgcn_ballot_w64(lane < B && r >= base && r < base + nb_l);
    if (hit != 0) {
      e.seq = (int)__builtin_ctzll(hit);
      e.level = r - __builtin_amdgcn_readlane(base, e.seq);
    }
  }
  if (e.seq >= 0) {
    e.start = __builtin_amdgcn_readlane(c0, e.seq);
    e.len = __builtin_amdgcn_readlane(c1, e.seq) - e.start;
  }
  return true;
}

// Swizzle of 16-byte chunks inside one LDS row of the K tile: chunk c of row
// r is stored at position c ^ swz_k(r).  16 consecutive rows (the lanes that
// read one chunk column together) land on 16 different 16-byte bank groups
// of the 256-byte bank space: a 256-byte row has 16 chunk positions; a
// 128-byte row puts odd rows in the upper half, so rows r and r ^ 1 share a
// position and r >> 1 picks it.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  return (D == 128) ? (r & 15) : ((r >> 1) & 7);
}

// Swizzle of the V tile.  A transposing read covers 4 consecutive rows x 64
// bytes (chunks 4j..4j+3); the XOR moves each of those rows to a different
// 64-byte quarter of the bank space.
template <int D>
__device__ __forceinline__ int swz_v(int r) {
  return (D == 128) ? ((r & 3) << 2) : (((r >> 1) & 1) << 2);
}

}  // namespace attn
