// attn_fwd.hip -- fused exact-attention forward for gfx950 (MI355X), bf16/fp16.
//
// What is computed: O = softmax(scale * Q K^T + mask) V and the per-row
// natural-log LSE ("FlashAttention-3 Deep Dive", introduction formula; Hopper
// tag page contents 4.2 and 4.6 for the streaming state and the LSE), tile by
// tile so that the score matrix stays on chip.
//
// Mapping onto CDNA4 (the pages' Hopper schedule is prior art, not a plan):
//
//  * A workgroup is 4 waves (256 threads) and owns BM = 128 query rows of one
//    (batch, head); each wave owns 32 of them.  Two workgroups share a CU, so
//    each SIMD runs two waves: while one wave is in its softmax (VALU) the
//    other issues MFMA -- the role the pages give to ping-pong warpgroups
//    ("flash-attention-3", "Why a schedule"), here obtained from the
//    hardware's wave interleaving instead of named barriers.
//  * Both GEMMs run on v_mfma_f32_32x32x16_{bf16,f16} with fp32 accumulation.
//    The first is computed transposed, S^T = K Q^T: the accumulator then
//    holds one query per lane (column) and 16 of the tile's keys per lane, so
//    the row max and row sum are in-lane, plus one exchange between the two
//    lane halves (v_permlane32_swap).  The second is O^T = V^T P^T: the
//    probabilities P^T are already in the lane layout of the MFMA B operand
//    and never leave registers (the pages' "P stays in registers" rule), and
//    the O accumulator also holds one query per lane, so the per-row
//    rescale and the final 1/l are lane scalars.
//  * Keys are fed to the first MFMA in a permuted row order (bits 2 and 3 of
//    the row index swapped) so that each lane half's 16 probabilities of a
//    16-key chunk are 8 consecutive keys -- exactly the K-operand order of the
//    second MFMA, with no shuffle.
//  * K/V tiles of BN keys are copied global -> LDS by the direct-to-LDS loads
//    (global_load_lds_dwordx4), double-buffered: tile t+1 streams in while
//    tile t is computed (the pages' producer role, done by the memory
//    pipeline rather than a producer warpgroup).  16-byte chunks are XOR
//    swizzled per row; the swizzle is expressed through the global address
//    each lane fetches, since the LDS side of the copy is lane-linear.
//  * The V operand of the second GEMM needs 8 consecutive keys per lane for a
//    fixed head-dim column; ds_read_b64_tr_b16 (gfx950's transposing LDS
//    read) delivers that from the row-major V tile.
//  * Online softmax in the exp2 domain with scale*log2(e) folded into one
//    FMA, and a lazy rescale: the running max is only moved (and O, l
//    rescaled) when a row's new max exceeds it by more than 2^8 in
//    probability, which is exact arithmetic (any reference point cancels in
//    O = sum P V / sum P) and keeps P <= 256.
//  * Causal: a wave skips key tiles entirely above its diagonal; only tiles
//    that cross the diagonal or the sequence end are masked (the pages' split
//    loop, Hopper tag page contents 4.7).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <utility>

#include "kernels.h"

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

template <typename T>
struct Mma;

template <>
struct Mma<__bf16> {
  typedef bf16x8 vec8;
  typedef __bf16 vec2 __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ f32x16 run(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // Row-sum share of one 8-key chunk.  bf16 keeps 8 significant bits, so a
  // sum of rounded probabilities can be off by 2^-9 relative (a 2e-3 error
  // in LSE when one key dominates): the sum is taken over the fp32 values.
  static constexpr bool kSumRounded = false;
  static __device__ __forceinline__ float sum8(vec8, const float (&pf)[8], float acc) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += pf[e];
    return acc;
  }
};

template <>
struct Mma<_Float16> {
  typedef f16x8 vec8;
  typedef _Float16 vec2 __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ f32x16 run(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  // fp16 keeps 11 significant bits: summing the rounded probabilities (two
  // per v_dot2) errs by at most 2^-11 relative in l, i.e. < 5e-4 in LSE.
  static constexpr bool kSumRounded = true;
  static __device__ __forceinline__ float sum8(vec8 p, const float (&)[8], float acc) {
    const vec2 one = __builtin_bit_cast(vec2, 0x3C003C00u);
    acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(p, p, 0, 1), one, acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(p, p, 2, 3), one, acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(p, p, 4, 5), one, acc, false);
    return __builtin_amdgcn_fdot2(__builtin_shufflevector(p, p, 6, 7), one, acc, false);
  }
};

// Swizzle of 16-byte chunks inside one LDS row of the K tile: chunk c of row
// r is stored at position c ^ swz_k(r).  16 consecutive rows (the lanes that
// read one chunk column together) land on 16 different chunk positions.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  return (D == 128) ? (r & 15) : (r & 7);
}

// Swizzle of the V tile.  A transposing read covers 4 consecutive rows x 64
// bytes (chunks 4j..4j+3); the XOR moves each of those rows to a different
// 64-byte quarter of the bank space.
template <int D>
__device__ __forceinline__ int swz_v(int r) {
  return (D == 128) ? ((r & 3) << 2) : (((r >> 1) & 1) << 2);
}

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

template <int N>
__device__ __forceinline__ void lds_wait(i16x4 (&r)[N]) {
  if constexpr (N == 8) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]), "+v"(r[6]),
                   "+v"(r[7]));
  } else {
    static_assert(N == 4, "");
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]));
  }
}

template <typename T, int D, int BN, bool CAUSAL, bool VARLEN>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
fwd_kernel(FwdParams p) {
  typedef typename Mma<T>::vec8 vec8;
  constexpr int NW = 4;
  constexpr int BM = kBlockM;
  constexpr int CPR = D / 8;           // 16-byte chunks per row
  constexpr int KT = D / 16;           // k-steps of the first GEMM
  constexpr int NB = BN / 32;          // 32-key blocks per tile
  constexpr int NC = BN / 16;          // 16-key chunks per tile (second GEMM)
  constexpr int DB = D / 32;           // 32-column blocks of O^T
  constexpr int ROW = D * 2;           // bytes per K/V row in LDS
  constexpr int TILE = BN * ROW;       // bytes per K or V tile
  constexpr int LOADS = BN * CPR / (NW * 64);   // DMA instructions per wave per tile
  constexpr float TAU = 8.0f;          // lazy-rescale threshold, log2 units
  constexpr float NEG_INF = -__builtin_inff();
  static_assert(BN == 64 && (BN * CPR) % (NW * 64) == 0, "tile shape");

  // [K stage 0 | K stage 1 | V stage 0 | V stage 1]
  __shared__ __attribute__((aligned(16))) char smem[4 * TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
  const int h = lane >> 5;
  const int l32 = lane & 31;

  // ---------------------------------------------------------------- tile decode
  int b, hq, mblk, q_len, kv_len;
  long long q_off, kv_off;   // element offsets of token 0 of this (batch | sequence)
  long long lse_off;         // index of this head's token 0 in lse
  if (VARLEN) {
    const int pid = blockIdx.x;
    hq = pid % p.Hq;
    int r = pid / p.Hq;
    int s = 0, start = 0, len = 0, nb = 0;
    for (; s < p.B; ++s) {
      start = p.cu_seqlens[s];
      len = p.cu_seqlens[s + 1] - start;
      nb = (len + BM - 1) / BM;
      if (r < nb) break;
      r -= nb;
    }
    if (s >= p.B) return;     // beyond the last tile (uniform over the workgroup)
    mblk = nb - 1 - r;         // longest query block of the sequence first
    b = 0;
    q_len = len;
    kv_len = len;
    q_off = (long long)start * p.q_tok_stride;
    kv_off = (long long)start * p.kv_tok_stride;
    lse_off = (long long)hq * p.Sq + start;
  } else {
    tile_decode(p.tm, blockIdx.x, b, hq, mblk);
    q_len = p.Sq;
    kv_len = p.Sk;
    q_off = (long long)b * p.q_batch_stride;
    kv_off = (long long)b * p.kv_batch_stride;
    lse_off = ((long long)b * p.Hq + hq) * p.Sq;
  }
  const int hkv = hq / p.group;
  const T* Qp = (const T*)p.q + q_off + hq * D;
  const T* Kp = (const T*)p.k + kv_off + hkv * D;
  const T* Vp = (const T*)p.v + kv_off + hkv * D;
  T* Op = (T*)p.o + q_off + hq * D;
  const int qs = p.q_tok_stride;
  const int ks = p.kv_tok_stride;

  const int q0 = mblk * BM;
  const int qw = q0 + wave * 32;                       // first query row of this wave
  const int q_hi = q0 + BM < q_len ? q0 + BM : q_len;  // one past the block's last row
  const int kv_end = CAUSAL ? (kv_len < q_hi ? kv_len : q_hi) : kv_len;
  const int ntile = (kv_end + BN - 1) / BN;

  // ---------------------------------------------------------------- Q fragment
  // B operand of S^T = K Q^T: lane holds query l32, head-dim 16*kk + 8*h .. +7.
  vec8 qf[KT];
  {
    const int qrow = (qw + l32 < q_len) ? qw + l32 : q_len - 1;
    const T* qr = Qp + (long long)qrow * qs + 8 * h;
#pragma unroll
    for (int kk = 0; kk < KT; ++kk) qf[kk] = *(const vec8*)(qr + 16 * kk);
  }

  // ---------------------------------------------------------------- K/V copy
  // buffer_load ... lds: one instruction writes 64 consecutive 16-byte LDS
  // chunks, lane L fetching the global chunk that belongs at position L under
  // the swizzle.  The per-lane byte offsets relative to the tile's first row
  // are tile-invariant (computed once); each tile gets a buffer resource whose
  // base is its first row and whose size ends at the sequence end, so the
  // hardware range check returns zeros for the rows past the end of a ragged
  // last tile (their scores are masked and their P is 0).
  const int wave_u = wave;
  uint32_t kdma[LOADS], vdma[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int pos = (wave_u * LOADS + i) * 64 + lane;
    const int row = pos / CPR, phys = pos % CPR;
    kdma[i] = (uint32_t)(row * ks * 2 + ((phys ^ swz_k<D>(row)) << 4));
    vdma[i] = (uint32_t)(row * ks * 2 + ((phys ^ swz_v<D>(row)) << 4));
  }
  auto issue = [&](const T* src, int t, char* dst, bool is_v) {
    const int j0 = t * BN;
    const uint32_t bytes = (uint32_t)(kv_len - j0) * (uint32_t)ks * 2u;
    copy_rows_to_lds<LOADS>((const void*)(src + (long long)j0 * ks), bytes, dst + wave_u * LOADS * 1024,
                            is_v ? vdma : kdma);
  };

  // per-lane LDS byte offsets, invariant over tiles
  const uint32_t lds0 = (uint32_t)(uintptr_t)(LDS_AS char*)smem;
  int koff[KT];
  {
    const int r = key_perm(l32);          // block bb adds 32 rows: an immediate offset
#pragma unroll
    for (int kk = 0; kk < KT; ++kk) koff[kk] = r * ROW + (((2 * kk + h) ^ swz_k<D>(r)) << 4);
  }
  uint32_t voff[DB];
  {
    const int G = lane >> 4, i16 = lane & 15;
    const int r = 8 * h + (i16 >> 2);     // chunk cc adds 16 rows, the second read 4 rows
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int dd = 32 * db + 16 * (G & 1) + 4 * (i16 & 3);
      voff[db] = lds0 + 2 * TILE + r * ROW + ((((dd >> 3) ^ swz_v<D>(r))) << 4) + ((dd & 7) << 1);
    }
  }

  f32x16 o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) o[i] = f32x16{};
  // P of the previous tile.  Before the first tile it is zero and the V stage
  // it pairs with (stage 1) is zero-filled, so the first tile runs the same
  // interleaved code as every other tile and adds exactly zero to O.
  vec8 pA[NC], pB[NC];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) pA[cc] = vec8{};
  {
    // both V stages start as zeros (stage 1 pairs with the zero P above; a
    // ragged tile leaves zeros, never stale bit patterns, in unused rows)
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    i32x4* z = (i32x4*)(smem + 2 * TILE);
#pragma unroll
    for (int i = tid; i < 2 * TILE / 16; i += kThreads) z[i] = i32x4{};
  }
  float m_run = NEG_INF;   // running max of scale*log2(e)*s for query l32 (same in both halves)
  float l_run = 0.f;       // this lane half's share of the running sum
  float alpha_pend = 1.f;  // rescale of O owed before the next P V product
  const float c = p.scale_log2;
  const int qi = qw + l32;

  // O^T += V^T P^T for one 16-key chunk; V tile at byte offset vbase
  auto pv_chunk = [&](i16x4 (&vr)[2 * DB], const vec8& pc) {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const i16x8 w = __builtin_shufflevector(vr[2 * db], vr[2 * db + 1], 0, 1, 2, 3, 4, 5, 6, 7);
      o[db] = Mma<T>::run(__builtin_bit_cast(vec8, w), pc, o[db]);
    }
  };
  auto read_v = [&](i16x4 (&vr)[2 * DB], uint32_t vstage, auto cc_tag) {
    constexpr int CC = decltype(cc_tag)::value;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      vr[2 * db] = lds_tr16<CC * 16 * ROW>(voff[db] + vstage);
      vr[2 * db + 1] = lds_tr16<CC * 16 * ROW + 4 * ROW>(voff[db] + vstage);
    }
  };

  if (ntile > 0) issue(Kp, 0, smem, false);

  // Per tile t the workgroup waits for K_t and V_{t-1}, then starts the copies
  // of K_{t+1} and V_t into the buffers freed by tile t-1.  Every wave takes
  // part in all ntile + 1 of these rounds; a wave of a causal block stops
  // computing after its last tile below the diagonal.
  auto top = [&](int t) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (t + 1 < ntile) issue(Kp, t + 1, smem + ((t + 1) & 1) * TILE, false);
    if (t < ntile) issue(Vp, t, smem + 2 * TILE + (t & 1) * TILE, true);
  };
  // O picks up the rescale owed for the previous tile's max before the next
  // P V product (a rare, wave-uniform branch)
  auto settle_alpha = [&] {
    if (__builtin_amdgcn_ballot_w64(alpha_pend != 1.f) != 0) {
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha_pend;
    }
    alpha_pend = 1.f;
  };

  // Full step: S_t = K_t Q^T, softmax of tile t into pout, and P_{t-1} V_{t-1}
  // (pin) into O, interleaved with the exponentials.  Unrolled by two below so
  // that the two P register sets swap roles instead of being copied.
  auto step_full = [&](int t, vec8 (&pin)[NC], vec8 (&pout)[NC]) {
    top(t);
    settle_alpha();
    const int j0 = t * BN;
    const uint32_t vprev = ((t + 1) & 1) * TILE;   // V of tile t-1

    // ---- S^T = K Q^T.  k-step outer so that each pair of LDS reads feeds two
    // independent accumulators, with the reads issued two k-steps ahead of
    // their MFMAs to cover the LDS latency.
    const char* Ks = smem + (t & 1) * TILE;
    f32x16 s[NB];
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) s[bb] = f32x16{};
    {
      constexpr int AHEAD = 2;
      vec8 kr[AHEAD + 1][NB];
#pragma unroll
      for (int kk = 0; kk < AHEAD; ++kk)
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) kr[kk][bb] = *(const vec8*)(Ks + koff[kk] + bb * 32 * ROW);
#pragma unroll
      for (int kk = 0; kk < KT; ++kk) {
        if (kk + AHEAD < KT) {
#pragma unroll
          for (int bb = 0; bb < NB; ++bb)
            kr[(kk + AHEAD) % (AHEAD + 1)][bb] = *(const vec8*)(Ks + koff[kk + AHEAD] + bb * 32 * ROW);
        }
        // keep the reads ahead of the MFMAs (the scheduler would otherwise
        // sink them next to their use to save registers)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) s[bb] = Mma<T>::run(kr[kk % (AHEAD + 1)][bb], qf[kk], s[bb]);
      }
    }

    // ---- mask: element i of block bb is key j0 + 32*bb + 16*(i/8) + 8*h + i%8
    const bool edge = (j0 + BN > kv_len) || (CAUSAL && j0 + BN - 1 > qw);
    if (edge) {
#pragma unroll
      for (int bb = 0; bb < NB; ++bb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = j0 + 32 * bb + 16 * (i >> 3) + 8 * h + (i & 7);
          const bool dead = (key >= kv_len) || (CAUSAL && key > qi);
          s[bb][i] = dead ? NEG_INF : s[bb][i];
        }
    }

    // ---- row max (in-lane over 32 keys, then across the two lane halves)
    float mx = NEG_INF;
#pragma unroll
    for (int bb = 0; bb < NB; ++bb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[bb][i]);
    mx = fmaxf(mx, wave_half_swap(mx));
    // lazy rescale, decided for the whole wave and kept branch-free so that
    // the exponentials below stay in one basic block with the MFMAs
    const float m_new = fmaxf(m_run, mx * c);
    const bool moved = __builtin_amdgcn_ballot_w64(m_new > m_run + TAU) != 0;
    const float m_upd = moved ? m_new : m_run;
    const float alpha = (m_upd == m_run) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_upd);
    m_run = m_upd;
    const float msub = (m_run == NEG_INF) ? 0.f : m_run;

    // ---- P = exp2(c*s - m) for chunk cc, with its row-sum share
    float rs = 0.f;
    auto softmax_chunk = [&](int cc) {
      float pf[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pf[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[cc >> 1][8 * (cc & 1) + e], c, -msub));
        pout[cc][e] = (T)pf[e];
      }
      rs = Mma<T>::sum8(pout[cc], pf, rs);
    };

    // ---- O^T += V^T P^T of the previous tile, interleaved with this tile's exp
    [&]<int... CC>(std::integer_sequence<int, CC...>) {
      ([&] {
        i16x4 vr[2 * DB];
        read_v(vr, vprev, std::integral_constant<int, CC>{});
        softmax_chunk(CC);
        lds_wait(vr);
        pv_chunk(vr, pin[CC]);
      }(), ...);
    }(std::make_integer_sequence<int, NC>{});
    l_run = l_run * alpha + rs;
    alpha_pend = alpha;
  };

  // Closing step of a wave: the last P V product only.
  auto step_pv = [&](int t, vec8 (&pin)[NC]) {
    top(t);
    settle_alpha();
    const uint32_t vprev = ((t + 1) & 1) * TILE;
    [&]<int... CC>(std::integer_sequence<int, CC...>) {
      ([&] {
        i16x4 vr[2 * DB];
        read_v(vr, vprev, std::integral_constant<int, CC>{});
        lds_wait(vr);
        pv_chunk(vr, pin[CC]);
      }(), ...);
    }(std::make_integer_sequence<int, NC>{});
  };

  // tiles this wave computes (a causal wave stops at its diagonal)
  const int n_w = CAUSAL ? min(ntile, (qw + 31) / BN + 1) : ntile;
  int t = 0;
  for (; t + 1 < n_w; t += 2) {
    step_full(t, pA, pB);
    step_full(t + 1, pB, pA);
  }
  if (t < n_w) {
    step_full(t, pA, pB);
    step_pv(t + 1, pB);
    t += 2;
  } else {
    step_pv(t, pA);
    t += 1;
  }
  for (; t <= ntile; ++t) top(t);

  // ---------------------------------------------------------------- epilogue
  const float l_tot = l_run + wave_half_swap(l_run);
  if (qi < q_len) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    T* orow = Op + (long long)qi * qs;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        typedef T T4 __attribute__((ext_vector_type(4)));
        T4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (T)(o[db][4 * g + e] * inv);
        *(T4*)(orow + 32 * db + 8 * g + 4 * h) = w;
      }
    if (p.lse != nullptr && h == 0) {
      const float lse = l_tot > 0.f ? (m_run + log2f(l_tot)) * 0.69314718055994530942f : NEG_INF;
      p.lse[lse_off + qi] = lse;
    }
  }
}

template <typename T, int D, int BN>
static hipError_t launch_t(const FwdParams& p, int causal, int varlen, hipStream_t s) {
  dim3 grid(p.grid), block(kThreads);
  if (varlen) {
    if (causal) hipLaunchKernelGGL((fwd_kernel<T, D, BN, true, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((fwd_kernel<T, D, BN, false, true>), grid, block, 0, s, p);
  } else {
    if (causal) hipLaunchKernelGGL((fwd_kernel<T, D, BN, true, false>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((fwd_kernel<T, D, BN, false, false>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdParams& p, int dtype, int d, int causal, int varlen, hipStream_t s) {
  if (dtype == 0) {
    return d == 128 ? launch_t<__bf16, 128, 64>(p, causal, varlen, s)
                    : launch_t<__bf16, 64, 64>(p, causal, varlen, s);
  }
  return d == 128 ? launch_t<_Float16, 128, 64>(p, causal, varlen, s)
                  : launch_t<_Float16, 64, 64>(p, causal, varlen, s);
}

}  // namespace attn
