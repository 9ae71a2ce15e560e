// attn_bwd_dkdv.hip -- dK and dV of the attention backward (bf16 / fp16,
// d in {64, 128}, dense or varlen, causal or not, GQA).
//
// Gradient math (Hopper tag page, contents 7.1): with P recomputed from the
// forward's LSE, dV = P^T dO and dK = scale dS^T Q, dS = P (dP - delta),
// dP = dO V^T.
//
// Workgroup = (batch, KV head, 128 keys) -- varlen: (KV head, sequence, key
// block), found by a scan of the offsets -- in ascending key-block order (the
// first blocks see the most queries under a causal mask: longest first).
// Each of the 4 waves owns 32 keys and walks 32-query steps of every query
// head of the KV group (GQA sums in registers, no atomics):
//   S = Q K^T, dP = dO V^T   (query rows x keys; the rows are permuted by
//                             key_perm so each accumulator, 8 registers at a
//                             time, is the B operand of the next MFMAs)
//   P = exp2(c S - lse2), dS = P (dP - delta)          (vector units)
//   dV^T += dO^T P, dK^T += Q^T dS  (A operands by ds_read_b64_tr_b16)
//
// Registers are assigned by name, as in the forward's wide kernel: the dK^T
// and dV^T accumulators and the wave's K and V fragments (the B operands of
// the first two GEMMs) live in fixed AGPRs and every MFMA is inline assembly
// that names them; S and dP are written straight to VGPRs, where the vector
// code reads them.  Left to itself the compiler placed S and dP in AGPRs and
// copied them out (and zeroed them) on every step.  The build checks that the
// compiler uses no AGPR in this file and spills nothing.
//
// AGPR map (DB = D / 32 channel blocks, KT = D / 16 k-steps):
//   a[0 : 16 DB)              dV^T, block db at 16 db
//   a[16 DB : 32 DB)          dK^T, block db at 16 DB + 16 db
//   a[32 DB : 32 DB + 4 KT)   K fragments, k-step kk at 32 DB + 4 kk
//   a[... : + 4 KT)           V fragments
// Hazards the compiler cannot see are kept by the order of the statements:
// S and dP are read after an s_nop run behind their last MFMA; each dV/dK
// MFMA has another MFMA between it and the next one on the same block; the
// accumulators are read after an s_nop run.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <utility>

#include "bwd_common.h"
#include "kernel_common.h"
#include "kernels.h"
#include "bwd_regs.h"
#include "wide_regs.h"

namespace attn {
namespace dkdv {

using namespace breg;

// AGPR map (DB = D / 32 channel blocks, KT = D / 16 k-steps)
template <int D>
struct Map {
  static constexpr int DB = D / 32, KT = D / 16;
  static constexpr int DV = 0, DK = 16 * DB, KF = 32 * DB, VF = 32 * DB + 4 * KT;
  static constexpr int USED = VF + 4 * KT;
};
static_assert(Map<64>::USED == 96, "d = 64 register map");
static_assert(Map<128>::USED <= 256, "d = 128 register map");

// accumulators a[0 : 32 DB) = 0, reserving the AGPRs the map uses: all 256
// for d = 128, a0..a95 for d = 64 (room for two waves per SIMD)
template <int D>
__device__ __forceinline__ void acc_zero() {
  breg::acc_zero<32 * Map<D>::DB, D == 64 ? 96 : 256>();
}

}  // namespace dkdv

// VARLEN: p.B sequences packed along the token axis (cu_seqlens); the
// statistics are then read from global memory (their per-sequence rows are
// not 16-byte aligned for the copy).
// Register budget (waves per SIMD): d = 128 one; d = 64 three (the 96 named
// AGPRs plus at most 72 VGPRs), except full attention over ragged batches,
// whose instance needs 76 VGPRs and gets two.
constexpr int dkdv_waves_per_simd(int D, bool CAUSAL, bool VARLEN) {
  return D == 128 ? 1 : (!CAUSAL && VARLEN) ? 2 : 3;
}
template <typename T, int D, bool CAUSAL, bool VARLEN>
__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(dkdv_waves_per_simd(D, CAUSAL, VARLEN), dkdv_waves_per_simd(D, CAUSAL, VARLEN))))
bwd_dkdv_kernel(BwdParams p) {
  using namespace dkdv;
  typedef typename Mma<T>::vec8 vec8;
  using M = Map<D>;
  constexpr int BMQ = 32;                 // query rows per step
  constexpr int KT = M::KT;
  constexpr int DB = M::DB;
  constexpr int ROW = 2 * D;
  constexpr int QT = BMQ * ROW;           // one 32-row tile
  constexpr int STAT = 1024;              // (lse2, delta) of 32 rows, in a 1 KiB slot
  // stage: [Q row-swizzled | Q transposed-swizzled | dO row | dO transposed | stats]
  constexpr int STAGE = 4 * QT + STAT;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int l32 = lane & 31;

  int b, hkv, nblk, q_len, k_len;
  long long q_tok0, k_tok0;               // token index of the sequence's first query / key
  if constexpr (VARLEN) {
    hkv = blockIdx.x % p.Hkv;
    int r = blockIdx.x / p.Hkv, sq = 0, start = 0, len = 0;
    // longest blocks first over the whole batch: causal, key block j of nb
    // is seen by the queries from j on, level nb - 1 - j
    VarlenEntry ve;
    if (varlen_rank<kBwdBlockN, CAUSAL>(p.cu_seqlens, p.B, r, ve)) {
      if (ve.seq < 0) return;             // beyond the last block (uniform over the workgroup)
      start = ve.start;
      len = ve.len;
      nblk = CAUSAL ? (len + kBwdBlockN - 1) / kBwdBlockN - 1 - ve.level : ve.level;
    } else {
      for (; sq < p.B; ++sq) {
        start = p.cu_seqlens[sq];
        len = p.cu_seqlens[sq + 1] - start;
        const int nb = (len + kBwdBlockN - 1) / kBwdBlockN;
        if (r < nb) break;
        r -= nb;
      }
      if (sq >= p.B) return;              // beyond the last block (uniform over the workgroup)
      nblk = r;
    }
    b = 0;
    q_len = k_len = len;
    q_tok0 = k_tok0 = start;
  } else {
    const int G = p.B * p.Hkv;
    nblk = blockIdx.x / G;
    const int gi = blockIdx.x % G;
    b = gi / p.Hkv;
    hkv = gi % p.Hkv;
    q_len = p.Sq;
    k_len = p.Sk;
    q_tok0 = (long long)b * p.Sq;
    k_tok0 = (long long)b * p.Sk;
  }
  const int k0 = nblk * kBwdBlockN;
  const int key = k0 + wave * 32 + l32;   // this lane's key (column of S), sequence position
  const int qs = p.Hq * D;                // token stride of q, o, dO, dQ

  acc_zero<D>();
  // K and V of the lane's key (B operands, k = head dimension) into their
  // AGPRs; rows past the end read a valid row and are masked
  {
    const long long row = (k_tok0 + min(key, k_len - 1)) * p.Hkv + hkv;
    const T* kr = (const T*)p.k + row * D + 8 * h;
    const T* vr = (const T*)p.v + row * D + 8 * h;
    static_for<KT>([&](auto kk) {
      frag_load<M::KF, decltype(kk)::value>(kr + 16 * kk);
      frag_load<M::VF, decltype(kk)::value>(vr + 16 * kk);
    });
  }

  const int nM = (q_len + BMQ - 1) / BMQ;
  const int m_begin = CAUSAL ? min(k0 / BMQ, nM) : 0;   // queries before k0 see none of these keys
  const int per_head = nM - m_begin;
  const int nsteps = p.group * per_head;

  const TileCopy<D, BMQ, 4> cp(wave, lane, qs);
  const TileReads<D> rd(lane);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(LDS_AS char*)smem;

  auto step_coords = [&](int s, int& hq, int& q0) {
    const int hg = s / per_head;
    hq = hkv * p.group + hg;
    q0 = (m_begin + s % per_head) * BMQ;
  };
  // varlen: a step's 32 (lse2, delta) pairs, one per lane of wave 0's first
  // half, loaded with the step's copies (8-byte loads from [Hq, T]; the array
  // has 32 spare pairs past its end, so a step's rows past the last token of
  // the last head still read allocated, initialised memory) and written into
  // the stage's statistics slot at the top of the step
  float2 st_pre = make_float2(0.f, 0.f);
  auto issue = [&](int s) {
    int hq, q0;
    step_coords(s, hq, q0);
    if (VARLEN && wave == 0 && lane < 32) st_pre = p.stats[(long long)hq * p.Sq + q_tok0 + q0 + lane];
    char* st = smem + (s & 1) * STAGE;
    const long long off = (q_tok0 + q0) * qs + hq * D;
    const uint32_t bytes = (uint32_t)(q_len - q0) * (uint32_t)qs * 2u;
    const T* qb = (const T*)p.q + off;
    const T* gb = (const T*)p.dout + off;
    constexpr int L = TileCopy<D, BMQ, 4>::LOADS;
    copy_rows_to_lds<L>(qb, bytes, st + 0 * QT + wave * L * 1024, cp.k);
    copy_rows_to_lds<L>(qb, bytes, st + 1 * QT + wave * L * 1024, cp.v);
    copy_rows_to_lds<L>(gb, bytes, st + 2 * QT + wave * L * 1024, cp.k);
    copy_rows_to_lds<L>(gb, bytes, st + 3 * QT + wave * L * 1024, cp.v);
    if (!VARLEN && wave == 0) {
      // 32 (lse2, delta) pairs = 16 lanes x 16 bytes (the array is padded to
      // 32 rows per head, so no 16-byte read straddles its end); the other
      // lanes' offsets are out of range and write zeros past the pairs
      const float2* sb = p.stats + ((long long)b * p.Hq + hq) * p.Sq_pad + q0;
      copy_row_to_lds(sb, (uint32_t)(p.Sq_pad - q0) * 8u, st + 4 * QT, lane < 16 ? (uint32_t)lane * 16u : 0x40000000u);
    }
  };

  const float c = p.scale_log2;
  if (nsteps > 0) issue(0);
  for (int s = 0; s < nsteps; ++s) {
    if constexpr (VARLEN) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (wave == 0 && lane < 32) {
        // rows past the sequence take (+inf, 0): P = 0 there
        int hq_s, q0_s;
        step_coords(s, hq_s, q0_s);
        const float2 v = q0_s + lane < q_len ? st_pre : make_float2(__builtin_inff(), 0.f);
        *(float2*)(smem + (s & 1) * STAGE + 4 * QT + 8 * lane) = v;
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    }
    if (s + 1 < nsteps) issue(s + 1);
    int hq, q0;
    step_coords(s, hq, q0);
    const char* st = smem + (s & 1) * STAGE;
    const uint32_t stl = lds0 + (s & 1) * STAGE;

    // S = Q K^T and dP = dO V^T: row m of the MFMA is query key_perm(m)
    f32x16 sacc, pacc;
    static_for<KT>([&](auto kkc) {
      constexpr int kk = decltype(kkc)::value;
      const vec8 qa = *(const vec8*)(st + 0 * QT + rd.koff(kk));
      const vec8 ga = *(const vec8*)(st + 2 * QT + rd.koff(kk));
      mfma_first<T, M::KF, kk, kk == 0>(sacc, qa);
      mfma_first<T, M::VF, kk, kk == 0>(pacc, ga);
    });
    pad2(sacc, pacc);
    // register r = 4 g + i holds query 16 (g >> 1) + 8 h + 4 (g & 1) + i:
    // 4 consecutive queries per g, read as 2 x 16 bytes of (lse2, delta)
    // (rows past the sequence: (+inf, 0), and their Q and dO are zero)
    const float* sp = (const float*)(st + 4 * QT);
    vec8 pv[2], dsv[2];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int qr = 16 * (g >> 1) + 8 * h + 4 * (g & 1);
      float l2[4], dl[4];
      {
        const float4 s01 = *(const float4*)(sp + 2 * qr);
        const float4 s23 = *(const float4*)(sp + 2 * qr + 4);
        l2[0] = s01.x; l2[1] = s01.z; l2[2] = s23.x; l2[3] = s23.z;
        dl[0] = s01.y; dl[1] = s01.w; dl[2] = s23.y; dl[3] = s23.w;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * g + i;
        const int qrow = q0 + qr + i;
        const bool dead = (key >= k_len) || (CAUSAL && key > qrow);
        const float pr = dead ? 0.f : __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], c, -l2[i]));
        const float ds = pr * (pacc[r] - dl[i]);
        pv[g >> 1][4 * (g & 1) + i] = (T)pr;
        dsv[g >> 1][4 * (g & 1) + i] = (T)ds;
      }
    }
    // dV^T += dO^T P, dK^T += Q^T dS (k = 16 queries per step); the eight
    // transposed reads of block db + 1 are in flight during block db's MFMAs.
    // Read pairs 0, 1 are dO^T, 2, 3 are Q^T; waiting for pair 2 covers 1.
    __builtin_amdgcn_sched_barrier(0);
    i16x4 tr[2][8];
    tr_issue8<D>(stl + 3 * QT + rd.voff(0), stl + 1 * QT + rd.voff(0), tr[0]);
    static_for<DB>([&](auto dbc) {
      constexpr int db = decltype(dbc)::value;
      i16x4(&cur)[8] = tr[db & 1];
      constexpr int DVB = M::DV + 16 * db, DKB = M::DK + 16 * db;
      if constexpr (db + 1 < DB) {
        tr_issue8<D>(stl + 3 * QT + rd.voff(db + 1), stl + 1 * QT + rd.voff(db + 1), tr[(db + 1) & 1]);
        lds_wait<14>(cur);
        mfma_acc<T, DVB>(tr_pair<vec8>(cur, 0), pv[0]);
        lds_wait<10>(cur);
        mfma_acc<T, DKB>(tr_pair<vec8>(cur, 2), dsv[0]);
        mfma_acc<T, DVB>(tr_pair<vec8>(cur, 1), pv[1]);
        lds_wait<8>(cur);
        mfma_acc<T, DKB>(tr_pair<vec8>(cur, 3), dsv[1]);
      } else {
        lds_wait<6>(cur);
        mfma_acc<T, DVB>(tr_pair<vec8>(cur, 0), pv[0]);
        lds_wait<2>(cur);
        mfma_acc<T, DKB>(tr_pair<vec8>(cur, 2), dsv[0]);
        mfma_acc<T, DVB>(tr_pair<vec8>(cur, 1), pv[1]);
        lds_wait<0>(cur);
        mfma_acc<T, DKB>(tr_pair<vec8>(cur, 3), dsv[1]);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  }

  // dK^T, dV^T: lane holds key `key` and channels 32 db + 8 g + 4 h + 0..3
  wide::acc_read_pad();
  if (key < k_len) {
    const long long row = (k_tok0 + key) * p.Hkv + hkv;
    T* dkr = (T*)p.dk + row * D;
    T* dvr = (T*)p.dv + row * D;
    typedef T T4 __attribute__((ext_vector_type(4)));
    static_for<DB>([&](auto dbc) {
      constexpr int db = decltype(dbc)::value;
      const f32x16 dkx = acc_read<M::DK + 16 * db>();
      const f32x16 dvx = acc_read<M::DV + 16 * db>();
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        T4 wk, wv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          wk[e] = (T)(dkx[4 * g + e] * p.scale);
          wv[e] = (T)dvx[4 * g + e];
        }
        *(T4*)(dkr + 32 * db + 8 * g + 4 * h) = wk;
        *(T4*)(dvr + 32 * db + 8 * g + 4 * h) = wv;
      }
    });
  }
}

// ---------------------------------------------------------------- pipelined
// The same work per step as bwd_dkdv_kernel, reordered so that the vector
// work of step s (P and dS from S_s, dP_s) runs under MFMAs: query rows 0-15
// of the step under dV/dK of step s - 1, rows 16-31 under S, dP of step s + 1.
// LDS ring of four stages; in iteration s, stage s - 1 feeds the transposed
// reads of dV/dK(s - 1), stage s + 1 the row reads of S, dP(s + 1) and the
// statistics of step s + 1, and stage s + 2 is being copied (the barrier at
// the top of iteration s frees it: every wave has finished iteration s - 1).
// The first transposed reads of an iteration and the statistics it needs are
// issued at the end of the one before, so the first MFMA follows the barrier
// at once; the copy of stage s + 2 is issued after that MFMA.  LDS reads are
// inline assembly waited for with explicit lgkmcnt values (reads complete in
// order); the vector code is pinned between MFMAs with scheduling barriers.
// Dense batches only (the statistics come with the LDS copies).
template <typename T, int D, bool CAUSAL>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
bwd_dkdv_pipe_kernel(BwdParams p) {
  using namespace dkdv;
  typedef typename Mma<T>::vec8 vec8;
  using M = Map<D>;
  constexpr int BMQ = 32;                 // query rows per step
  constexpr int KT = M::KT;
  constexpr int DB = M::DB;
  constexpr int ROW = 2 * D;
  constexpr int QT = BMQ * ROW;
  constexpr int STAT = 1024;
  // stage: [Q row-swizzled | Q transposed-swizzled | dO row | dO transposed | stats]
  constexpr int STAGE = 4 * QT + STAT;
  constexpr int HEAD = KT < 4 ? KT : 4;   // row-read batches in flight in S, dP
  static_assert(KT % 4 == 0 && (4 % DB == 0 || DB % 4 == 0), "vector work placement");
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int l32 = lane & 31;

  const int G = p.B * p.Hkv;
  const int nblk = blockIdx.x / G;
  const int b = (blockIdx.x % G) / p.Hkv;
  const int hkv = (blockIdx.x % G) % p.Hkv;
  const int q_len = p.Sq, k_len = p.Sk;
  const long long q_tok0 = (long long)b * p.Sq;
  const long long k_tok0 = (long long)b * p.Sk;
  const int k0 = nblk * kBwdBlockN;
  const int key = k0 + wave * 32 + l32;
  const int qs = p.Hq * D;

  acc_zero<D>();
  {
    const long long row = (k_tok0 + min(key, k_len - 1)) * p.Hkv + hkv;
    const T* kr = (const T*)p.k + row * D + 8 * h;
    const T* vr = (const T*)p.v + row * D + 8 * h;
    static_for<KT>([&](auto kk) {
      frag_load<M::KF, decltype(kk)::value>(kr + 16 * kk);
      frag_load<M::VF, decltype(kk)::value>(vr + 16 * kk);
    });
  }

  const int nM = (q_len + BMQ - 1) / BMQ;
  const int m_begin = CAUSAL ? min(k0 / BMQ, nM) : 0;
  const int per_head = nM - m_begin;
  const int nsteps = p.group * per_head;

  const TileCopy<D, BMQ, 4> cp(wave, lane, qs);
  const TileReads<D> rd(lane);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(LDS_AS char*)smem;
  auto stage = [&](int s) { return lds0 + (uint32_t)(s & 3) * STAGE; };

  // Step order: first the query blocks a mask reaches (nd per head: the
  // causal diagonal, every block of a ragged key block) of every head, then
  // the other blocks of every head; steps [0, nmask) need the mask.
  // StepIt = (query head hkv * group + hg, query block qb) of one step,
  // advanced one step at a time over blocks [lo, hi) of each head.
  const bool ragged = k0 + kBwdBlockN > k_len;
  const int nd = ragged ? per_head : (CAUSAL ? min(per_head, 4) : 0);
  const bool two_phase = nd > 0 && nd < per_head;
  const int nmask = nd == 0 ? 0 : (two_phase ? p.group * nd : nsteps);
  struct StepIt {
    int hg, qb, lo, hi;
  };
  auto advance = [&](StepIt& it) {
    if (++it.qb < it.hi) return;
    if (++it.hg < p.group) {
      it.qb = it.lo;
      return;
    }
    if (it.hi != nM) {                    // end of the first phase
      it.hg = 0;
      it.lo = it.qb = it.hi;
      it.hi = nM;
    }
  };

  auto issue = [&](int s, const StepIt& it) {
    const int hq = hkv * p.group + it.hg, q0 = it.qb * BMQ;
    char* st = smem + (s & 3) * STAGE;
    const long long off = (q_tok0 + q0) * qs + hq * D;
    const uint32_t bytes = (uint32_t)(q_len - q0) * (uint32_t)qs * 2u;
    const T* qb = (const T*)p.q + off;
    const T* gb = (const T*)p.dout + off;
    constexpr int L = TileCopy<D, BMQ, 4>::LOADS;
    copy_rows_to_lds<L>(qb, bytes, st + 0 * QT + wave * L * 1024, cp.k);
    copy_rows_to_lds<L>(qb, bytes, st + 1 * QT + wave * L * 1024, cp.v);
    copy_rows_to_lds<L>(gb, bytes, st + 2 * QT + wave * L * 1024, cp.k);
    copy_rows_to_lds<L>(gb, bytes, st + 3 * QT + wave * L * 1024, cp.v);
    if (wave == 0) {
      const float2* sb = p.stats + ((long long)b * p.Hq + hq) * p.Sq_pad + q0;
      copy_row_to_lds(sb, (uint32_t)(p.Sq_pad - q0) * 8u, st + 4 * QT, lane < 16 ? (uint32_t)lane * 16u : 0x40000000u);
    }
  };

  // statistics of a step: st[2 g + j] = (lse2, delta) of query rows
  // qr + 2 j and qr + 2 j + 1, qr = 16 (g >> 1) + 8 h + 4 (g & 1)
  auto stats_lds = [&](uint32_t sb, f32x4 (&st)[8]) {
    const uint32_t a = sb + 4 * QT + 64 * h;
    i32x4 r[8];
    r[0] = lds_rd128<0>(a);
    r[1] = lds_rd128<16>(a);
    r[2] = lds_rd128<32>(a);
    r[3] = lds_rd128<48>(a);
    r[4] = lds_rd128<128>(a);
    r[5] = lds_rd128<144>(a);
    r[6] = lds_rd128<160>(a);
    r[7] = lds_rd128<176>(a);
#pragma unroll
    for (int j = 0; j < 8; ++j) st[j] = __builtin_bit_cast(f32x4, r[j]);
  };

  const float c = p.scale_log2;
  // element (g, i) of a step at q0 is masked iff tl - q0 > 16 (g >> 1) + 4 (g & 1) + i
  // (causal: the key is past the query row; any: the key is past the end)
  constexpr int BIG = 1 << 30;
  const int tl = key >= k_len ? BIG : (CAUSAL ? key - 8 * h : -BIG);

  // P and dS of elements E, E + 1 (E even; register r = 4 g + i holds query
  // row 16 (g >> 1) + 8 h + 4 (g & 1) + i) into the 16-bit B operands
  auto pair = [&](auto ec, auto maskc, const f32x16& sc, const f32x16& pc, const f32x4 (&st)[8], int t,
                  vec8 (&pvc)[2], vec8 (&dsc)[2]) {
    constexpr int E = decltype(ec)::value;
    constexpr bool MASK = decltype(maskc)::value;
    constexpr int g = E >> 2, i = E & 3;
    constexpr int cr = 16 * (g >> 1) + 4 * (g & 1) + i;
    const f32x4 sv = st[2 * g + (i >> 1)];
    float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[E], c, -sv.x));
    float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[E + 1], c, -sv.z));
    if constexpr (MASK) {
      p0 = t > cr ? 0.f : p0;
      p1 = t > cr + 1 ? 0.f : p1;
    }
    const float d0 = p0 * (pc[E] - sv.y);
    const float d1 = p1 * (pc[E + 1] - sv.w);
    constexpr int v = g >> 1, o = 4 * (g & 1) + i;
    typedef T T2 __attribute__((ext_vector_type(2)));
    const T2 pp = {(T)p0, (T)p1};
    const T2 dd = {(T)d0, (T)d1};
    // pinned here: otherwise the compiler sinks the whole computation to the
    // first use (the next iteration's MFMAs), undoing the interleave
    keep_vec(pp);
    keep_vec(dd);
    pvc[v][o] = pp[0];
    pvc[v][o + 1] = pp[1];
    dsc[v][o] = dd[0];
    dsc[v][o + 1] = dd[1];
  };

  // row reads of S, dP: batch kk = (Q, dO) 16 bytes each at the lane's offset
  auto rowread = [&](auto kkc, uint32_t sb, i32x4 (&qg)[KT][2]) {
    constexpr int kk = decltype(kkc)::value;
    const uint32_t a = sb + (uint32_t)rd.koff(kk);
    qg[kk][0] = lds_rd128<0>(a);
    qg[kk][1] = lds_rd128<2 * QT>(a);
  };
  auto rowread_head = [&](uint32_t sb, i32x4 (&qg)[KT][2]) {
    static_for<HEAD>([&](auto kk) { rowread(kk, sb, qg); });
  };

  // S = Q K^T, dP = dO V^T of the step in stage sb (its first HEAD batches
  // already issued); HOOK(kk) runs after k-step kk's MFMAs
  auto sdp = [&](uint32_t sb, f32x16& sn, f32x16& pn, i32x4 (&qg)[KT][2], auto&& hook) {
    static_for<KT>([&](auto kkc) {
      constexpr int kk = decltype(kkc)::value;
      constexpr int after = (KT - 1 - kk) < (HEAD - 1) ? (KT - 1 - kk) : (HEAD - 1);
      lds_wait<2 * after>(qg[kk]);
      mfma_first<T, M::KF, kk, kk == 0>(sn, __builtin_bit_cast(vec8, qg[kk][0]));
      mfma_first<T, M::VF, kk, kk == 0>(pn, __builtin_bit_cast(vec8, qg[kk][1]));
      if constexpr (kk + HEAD < KT) rowread(std::integral_constant<int, kk + HEAD>{}, sb, qg);
      hook(kkc);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // transposed reads of channel block db of the step in stage sb: pairs 0, 1
  // = dO^T, pairs 2, 3 = Q^T (16 query rows each)
  auto tr_issue = [&](auto dbc, uint32_t sb, i16x4(&r)[8]) {
    constexpr int db = decltype(dbc)::value;
    constexpr int R = ROW;
    const uint32_t x = sb + QT + (rd.voff0 ^ (uint32_t)(db << 6));
    r[0] = lds_tr16<2 * QT>(x);
    r[1] = lds_tr16<2 * QT + 4 * R>(x);
    r[2] = lds_tr16<2 * QT + 16 * R>(x);
    r[3] = lds_tr16<2 * QT + 20 * R>(x);
    r[4] = lds_tr16<0>(x);
    r[5] = lds_tr16<4 * R>(x);
    r[6] = lds_tr16<16 * R>(x);
    r[7] = lds_tr16<20 * R>(x);
  };

  // dV^T += dO^T P, dK^T += Q^T dS of the step in stage sb.  PRE: the reads
  // of block 0 were issued by the caller (tr0).  NEXT: the first row reads of
  // the next step (stage sbn) are issued during the last channel block.
  // HOOK(m) runs after MFMA m (4 per channel block).
  auto dvdk = [&](auto prec, auto nextc, uint32_t sb, uint32_t sbn, const vec8 (&pvp)[2], const vec8 (&dsp)[2],
                  i32x4 (&qg)[KT][2], const i16x4 (&tr0)[8], auto&& hook) {
    constexpr bool PRE = decltype(prec)::value, NEXT = decltype(nextc)::value;
    i16x4 tr[2][8];
    if constexpr (PRE) {
#pragma unroll
      for (int j = 0; j < 8; ++j) tr[0][j] = tr0[j];
    } else {
      tr_issue(std::integral_constant<int, 0>{}, sb, tr[0]);
    }
    static_for<DB>([&](auto dbc) {
      constexpr int db = decltype(dbc)::value;
      i16x4(&cur)[8] = tr[db & 1];
      constexpr int DVB = M::DV + 16 * db, DKB = M::DK + 16 * db;
      constexpr int nb = (db + 1 < DB) ? 8 : (NEXT ? 2 * HEAD : 0);
      if constexpr (db + 1 < DB) tr_issue(std::integral_constant<int, db + 1>{}, sb, tr[(db + 1) & 1]);
      else if constexpr (NEXT) rowread_head(sbn, qg);
      lds_wait<6 + nb>(cur);
      mfma_acc<T, DVB>(tr_pair<vec8>(cur, 0), pvp[0]);
      hook(std::integral_constant<int, 4 * db + 0>{});
      __builtin_amdgcn_sched_barrier(0);
      lds_wait<2 + nb>(cur);
      mfma_acc<T, DKB>(tr_pair<vec8>(cur, 2), dsp[0]);
      hook(std::integral_constant<int, 4 * db + 1>{});
      __builtin_amdgcn_sched_barrier(0);
      mfma_acc<T, DVB>(tr_pair<vec8>(cur, 1), pvp[1]);
      hook(std::integral_constant<int, 4 * db + 2>{});
      __builtin_amdgcn_sched_barrier(0);
      lds_wait<0 + nb>(cur);
      mfma_acc<T, DKB>(tr_pair<vec8>(cur, 3), dsp[1]);
      hook(std::integral_constant<int, 4 * db + 3>{});
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  auto no_hook = [](auto) {};

  // one iteration: P, dS of step s (from sc, pc, st) into pvc, dsc, under
  // dV/dK of step s - 1 (pvp, dsp; its first reads in trn) and S, dP of step
  // s + 1 (into sn, pn).  With NEXT, ends by issuing the statistics of step
  // s + 1 (into st, after their last use for step s) and the first
  // transposed reads of dV/dK(s) (into trn).  it: step s; it2: step s + 2
  // (copy); each advanced by one.
  auto body = [&](auto prevc, auto nextc, auto maskc, int s, f32x16& sc, f32x16& pc, f32x16& sn, f32x16& pn,
                  const vec8 (&pvp)[2], const vec8 (&dsp)[2], vec8 (&pvc)[2], vec8 (&dsc)[2],
                  f32x4 (&st)[8], i16x4 (&trn)[8], StepIt& it, StepIt& it2) {
    constexpr bool PREV = decltype(prevc)::value, NEXT = decltype(nextc)::value;
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    const uint32_t sbn = stage(s + 1);
    const int t = tl - it.qb * BMQ;
    i32x4 qg[KT][2];
    auto copy_next = [&]() {
      if (s + 2 < nsteps) issue(s + 2, it2);
    };
    // The vector work reads S and dP through this tie, placed after the wait
    // that covers the statistics reads: its inputs are otherwise available
    // (to the compiler) at the end of the previous iteration, and it may
    // hoist the pure arithmetic there, ahead of the waits and of the MFMA
    // results.  (Tying the statistics as well gave wrong dV in measurement;
    // the tie on S and dP alone already orders every use.)
    f32x16& scx = sc;
    f32x16& pcx = pc;
    auto tie = [&]() { asm volatile("" : "+v"(scx), "+v"(pcx)); };
    // rows 0-15: pairs 0..3
    if constexpr (PREV) {
      dvdk(std::true_type{}, nextc, stage(s - 1), sbn, pvp, dsp, qg, trn, [&](auto mc) {
        constexpr int m = decltype(mc)::value;
        if constexpr (m == 0) {
          tie();
          copy_next();
        }
        if constexpr ((m + 1) % DB == 0)
          pair(std::integral_constant<int, 2 * ((m + 1) / DB - 1)>{}, maskc, scx, pcx, st, t, pvc, dsc);
      });
    } else {
      tie();
      copy_next();
      if constexpr (NEXT) rowread_head(sbn, qg);
      static_for<4>([&](auto e) {
        pair(std::integral_constant<int, 2 * decltype(e)::value>{}, maskc, scx, pcx, st, t, pvc, dsc);
      });
      __builtin_amdgcn_sched_barrier(0);
    }
    // rows 16-31: pairs 4..7
    if constexpr (NEXT) {
      sdp(sbn, sn, pn, qg, [&](auto kkc) {
        constexpr int kk = decltype(kkc)::value;
        constexpr int per = KT / 4;
        if constexpr ((kk + 1) % per == 0)
          pair(std::integral_constant<int, 8 + 2 * ((kk + 1) / per - 1)>{}, maskc, scx, pcx, st, t, pvc, dsc);
      });
      stats_lds(sbn, st);
      tr_issue(std::integral_constant<int, 0>{}, stage(s), trn);
    } else {
      static_for<4>([&](auto e) {
        pair(std::integral_constant<int, 8 + 2 * decltype(e)::value>{}, maskc, scx, pcx, st, t, pvc, dsc);
      });
    }
    advance(it);
    advance(it2);
  };

  const std::integral_constant<bool, true> yes;
  const std::integral_constant<bool, false> no;
  f32x16 sa, pa, sb2, pb2;
  vec8 px[2], dx[2], py[2], dy[2];
  f32x4 st[8];
  i16x4 trn[8];
  i32x4 qg0[KT][2];
  if (nsteps > 0) {
    const StepIt it0{0, m_begin, m_begin, two_phase ? m_begin + nd : nM};
    StepIt it = it0, it2 = it0;
    issue(0, it2);
    advance(it2);
    if (nsteps > 1) issue(1, it2);
    advance(it2);
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    stats_lds(stage(0), st);
    rowread_head(stage(0), qg0);
    sdp(stage(0), sa, pa, qg0, no_hook);
    pad2(sa, pa);
    // step s consumes S set s % 2 (a, b) and produces P set s % 2 (x, y);
    // the first and the last steps, and pairs that start below nmask, run
    // with the mask
    if (nsteps == 1) {
      body(no, no, yes, 0, sa, pa, sb2, pb2, py, dy, px, dx, st, trn, it, it2);
      dvdk(no, no, stage(0), 0, px, dx, qg0, trn, no_hook);
    } else {
      body(no, yes, yes, 0, sa, pa, sb2, pb2, py, dy, px, dx, st, trn, it, it2);
      int s = 1;
      for (; s + 2 < nsteps && s < nmask; s += 2) {
        body(yes, yes, yes, s, sb2, pb2, sa, pa, px, dx, py, dy, st, trn, it, it2);
        body(yes, yes, yes, s + 1, sa, pa, sb2, pb2, py, dy, px, dx, st, trn, it, it2);
      }
      for (; s + 2 < nsteps; s += 2) {
        body(yes, yes, no, s, sb2, pb2, sa, pa, px, dx, py, dy, st, trn, it, it2);
        body(yes, yes, no, s + 1, sa, pa, sb2, pb2, py, dy, px, dx, st, trn, it, it2);
      }
      if (s + 1 < nsteps) {
        body(yes, yes, yes, s, sb2, pb2, sa, pa, px, dx, py, dy, st, trn, it, it2);
        body(yes, no, yes, s + 1, sa, pa, sb2, pb2, py, dy, px, dx, st, trn, it, it2);
        dvdk(no, no, stage(s + 1), 0, px, dx, qg0, trn, no_hook);
      } else {
        body(yes, no, yes, s, sb2, pb2, sa, pa, px, dx, py, dy, st, trn, it, it2);
        dvdk(no, no, stage(s), 0, py, dy, qg0, trn, no_hook);
      }
    }
  }

  wide::acc_read_pad();
  if (key < k_len) {
    const long long row = (k_tok0 + key) * p.Hkv + hkv;
    T* dkr = (T*)p.dk + row * D;
    T* dvr = (T*)p.dv + row * D;
    typedef T T4 __attribute__((ext_vector_type(4)));
    static_for<DB>([&](auto dbc) {
      constexpr int db = decltype(dbc)::value;
      const f32x16 dkx = acc_read<M::DK + 16 * db>();
      const f32x16 dvx = acc_read<M::DV + 16 * db>();
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        T4 wk, wv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          wk[e] = (T)(dkx[4 * g + e] * p.scale);
          wv[e] = (T)dvx[4 * g + e];
        }
        *(T4*)(dkr + 32 * db + 8 * g + 4 * h) = wk;
        *(T4*)(dvr + 32 * db + 8 * g + 4 * h) = wv;
      }
    });
  }
}

template <typename T, int D, bool CAUSAL, bool VARLEN>
static hipError_t launch_dkdv_t(const BwdParams& p, hipStream_t s) {
  if constexpr (D == 128 && !VARLEN) {
    constexpr int lds = 4 * (4 * 32 * 2 * D + 1024);
    static const hipError_t attr = hipFuncSetAttribute((const void*)bwd_dkdv_pipe_kernel<T, D, CAUSAL>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((bwd_dkdv_pipe_kernel<T, D, CAUSAL>), dim3(p.grid_dkdv), dim3(256), lds, s, p);
  } else {
    constexpr int lds = 2 * (4 * 32 * 2 * D + 1024);
    static const hipError_t attr = hipFuncSetAttribute((const void*)bwd_dkdv_kernel<T, D, CAUSAL, VARLEN>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, CAUSAL, VARLEN>), dim3(p.grid_dkdv), dim3(256), lds, s, p);
  }
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_dkdv_v(const BwdParams& p, int causal, int varlen, hipStream_t s) {
  if (varlen) return causal ? launch_dkdv_t<T, D, true, true>(p, s) : launch_dkdv_t<T, D, false, true>(p, s);
  return causal ? launch_dkdv_t<T, D, true, false>(p, s) : launch_dkdv_t<T, D, false, false>(p, s);
}

hipError_t launch_bwd_dkdv(const BwdParams& p, int dtype, int d, int causal, int varlen, hipStream_t s) {
  if (dtype == 0)
    return d == 128 ? launch_dkdv_v<__bf16, 128>(p, causal, varlen, s) : launch_dkdv_v<__bf16, 64>(p, causal, varlen, s);
  return d == 128 ? launch_dkdv_v<_Float16, 128>(p, causal, varlen, s) : launch_dkdv_v<_Float16, 64>(p, causal, varlen, s);
}

}  // namespace attn
