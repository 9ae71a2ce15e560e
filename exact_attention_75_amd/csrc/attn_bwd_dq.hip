// attn_bwd_dq.hip -- dQ of the attention backward (bf16 / fp16, d in
// {64, 128}, dense or varlen, causal or not, GQA).
//
// Gradient math (Hopper tag page, contents 7.1): dQ = scale dS K with
// dS = P (dP - delta), P = exp2(c S - lse2) and dP = dO V^T recomputed per
// key tile (the pages' kernel accumulates dQ across key blocks with atomics;
// here dQ has a kernel of its own, deterministic).
//
// Workgroup = (batch, query head, 128 rows) in the forward's tile order
// (varlen: (query head, sequence, query block), longest block of a sequence
// first); each of the 4 waves owns 32 queries and walks the 64-key tiles up
// to its diagonal.  A lane owns one query (the column of the transposed
// products), so LSE and delta are lane scalars:
//   S^T = K Q^T, dP^T = V dO^T   (two 32-key blocks; key rows permuted by
//                                 key_perm so each accumulator, 8 registers
//                                 at a time, is the B operand of dQ)
//   dS^T = P^T (dP^T - delta)     (vector units)
//   dQ^T += K^T dS^T              (K^T by ds_read_b64_tr_b16 of a second,
//                                 transpose-swizzled copy of the K tile)
// Pipeline: the MFMAs of S^T, dP^T of tile t + 1 carry the vector work of
// tile t; three LDS stages (tile t + 2 being copied).
//
// Registers are named as in the dK/dV kernel: dQ^T and the wave's Q and dO
// fragments (the B operands of S^T and dP^T) sit in fixed AGPRs, every MFMA
// is inline assembly that names them, S^T and dP^T go straight to VGPRs.
// AGPR map (DB = D / 32, KT = D / 16): dQ^T block db at 16 db, Q k-step kk at
// 16 DB + 4 kk, dO k-step kk at 16 DB + 4 KT + 4 kk.  LDS reads are inline
// assembly waited for with explicit lgkmcnt values; one wave per SIMD (the
// two S / dP register sets alone take 128 VGPRs).  Tiles that no mask
// reaches (all keys at or below every query of the wave and inside the
// sequence) run without the mask arithmetic.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <utility>

#include "bwd_common.h"
#include "bwd_regs.h"
#include "kernel_common.h"
#include "kernels.h"
#include "tile_sched.h"

namespace attn {
namespace dqr {

using namespace breg;

template <int D>
struct Map {
  static constexpr int DB = D / 32, KT = D / 16;
  static constexpr int DQ = 0, QF = 16 * DB, GF = 16 * DB + 4 * KT;
  static constexpr int USED = GF + 4 * KT;
};
static_assert(Map<64>::USED == 64 && Map<128>::USED == 128, "register map");

}  // namespace dqr

template <typename T, int D, bool CAUSAL, bool VARLEN>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
bwd_dq_pipe_kernel(BwdParams p) {
  using namespace dqr;
  typedef typename Mma<T>::vec8 vec8;
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  using M = Map<D>;
  constexpr int BN = 64;                  // keys per tile (two 32-key blocks)
  constexpr int KT = M::KT;
  constexpr int DB = M::DB;
  constexpr int ROW = 2 * D;
  constexpr int TILE = BN * ROW;
  // stage: [K row-swizzled | K transposed-swizzled | V row-swizzled]
  constexpr int STAGE = 3 * TILE;
  constexpr int HEAD = KT >= 8 ? 3 : 2;   // row-read batches (4 reads each) in flight
  constexpr int EPS = 32 / KT;            // dS elements per k-step of the next tile's MFMAs
  static_assert(KT >= HEAD && EPS % 2 == 0, "pipeline shape");
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int l32 = lane & 31;

  int b, hq, mblk, q_len, k_len;
  long long q_tok0, k_tok0, stat0;        // first query / key token; stats index of query 0
  if constexpr (VARLEN) {
    hq = blockIdx.x % p.Hq;
    int r = blockIdx.x / p.Hq, sq = 0, start = 0, len = 0, nb = 0;
    // longest blocks first over the whole batch (level = query block index)
    VarlenEntry ve;
    if (varlen_rank<kBwdBlockM, CAUSAL>(p.cu_seqlens, p.B, r, ve)) {
      if (ve.seq < 0) return;             // beyond the last block (uniform over the workgroup)
      mblk = ve.level;
      start = ve.start;
      len = ve.len;
    } else {
      for (; sq < p.B; ++sq) {
        start = p.cu_seqlens[sq];
        len = p.cu_seqlens[sq + 1] - start;
        nb = (len + kBwdBlockM - 1) / kBwdBlockM;
        if (r < nb) break;
        r -= nb;
      }
      if (sq >= p.B) return;              // beyond the last tile (uniform over the workgroup)
      mblk = nb - 1 - r;                  // longest query block of the sequence first
    }
    b = 0;
    q_len = k_len = len;
    q_tok0 = k_tok0 = start;
    stat0 = (long long)hq * p.Sq + start; // varlen layout [Hq, T]
  } else {
    tile_decode(p.tm, (int)blockIdx.x, b, hq, mblk);
    q_len = p.Sq;
    k_len = p.Sk;
    q_tok0 = (long long)b * p.Sq;
    k_tok0 = (long long)b * p.Sk;
    stat0 = ((long long)b * p.Hq + hq) * p.Sq_pad;
  }
  const int hkv = hq / p.group;
  const int qs = p.Hq * D;
  const int ks = p.Hkv * D;
  const int q0 = mblk * kBwdBlockM;
  const int qw = q0 + wave * 32;
  const int qi = qw + key_perm(l32);      // this lane's query (column of S^T)
  const int qc = min(qi, q_len - 1);      // rows past the end compute on a valid row, never stored
  const int q_hi = min(q0 + kBwdBlockM, q_len);
  const int kv_end = CAUSAL ? min(k_len, q_hi) : k_len;
  const int ntile = (kv_end + BN - 1) / BN;

  acc_zero<16 * DB, 256>();
  {
    const long long row = (q_tok0 + qc) * p.Hq + hq;
    const T* qr = (const T*)p.q + row * D + 8 * h;
    const T* gr = (const T*)p.dout + row * D + 8 * h;
    static_for<KT>([&](auto kk) {
      frag_load<M::QF, decltype(kk)::value>(qr + 16 * kk);
      frag_load<M::GF, decltype(kk)::value>(gr + 16 * kk);
    });
  }
  const float2 st2 = p.stats[stat0 + qc];
  const float l2 = st2.x, dl = st2.y;
  const float c = p.scale_log2;

  const TileCopy<D, BN, 4> cp(wave, lane, ks);
  const TileReads<D> rd(lane);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(LDS_AS char*)smem;
  auto stage = [&](int t) { return lds0 + (uint32_t)(t % 3) * STAGE; };
  const T* kbase = (const T*)p.k + k_tok0 * ks + hkv * D;
  const T* vbase = (const T*)p.v + k_tok0 * ks + hkv * D;
  auto issue = [&](int t) {
    char* st = smem + (t % 3) * STAGE;
    const int j0 = t * BN;
    const uint32_t bytes = (uint32_t)(k_len - j0) * (uint32_t)ks * 2u;
    constexpr int L = TileCopy<D, BN, 4>::LOADS;
    copy_rows_to_lds<L>(kbase + (long long)j0 * ks, bytes, st + 0 * TILE + wave * L * 1024, cp.k);
    copy_rows_to_lds<L>(kbase + (long long)j0 * ks, bytes, st + 1 * TILE + wave * L * 1024, cp.v);
    copy_rows_to_lds<L>(vbase + (long long)j0 * ks, bytes, st + 2 * TILE + wave * L * 1024, cp.k);
  };
  // tiles this wave computes (a causal wave stops at its diagonal); every
  // wave still takes part in every round's barrier
  const int n_w = CAUSAL ? min(ntile, (qw + 31) / BN + 1) : ntile;
  // element k of a tile (block k >> 4, register r = k & 15, g = r >> 2,
  // i = r & 3) is key j0 + 8 h + cr(k), cr = 32 (k >> 4) + 16 (g >> 1) +
  // 4 (g & 1) + i; it is masked iff that key is past lim (the lane's query
  // under the causal mask, the last key in any case)
  const int lim = CAUSAL ? min(qi, k_len - 1) : k_len - 1;
  // leading tiles no mask reaches: every key <= every lim of the wave
  const int lim_w = CAUSAL ? min(qw, k_len - 1) : k_len - 1;
  const int n_free = min(n_w, (lim_w + 1) / BN);

  // row reads of k-step kk: K and V of both 32-key blocks
  auto rowread = [&](auto kkc, uint32_t sb, i32x4 (&kv)[KT][4]) {
    constexpr int kk = decltype(kkc)::value;
    const uint32_t a = sb + (uint32_t)rd.koff(kk);
    kv[kk][0] = lds_rd128<0>(a);
    kv[kk][1] = lds_rd128<32 * ROW>(a);
    kv[kk][2] = lds_rd128<2 * TILE>(a);
    kv[kk][3] = lds_rd128<2 * TILE + 32 * ROW>(a);
  };
  auto wait4 = [](auto leftc, i32x4 (&r)[4]) {
    constexpr int LEFT = decltype(leftc)::value;
    asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]) : "n"(LEFT));
  };

  // S^T, dP^T of the tile in stage sb; HOOK(kk) runs after k-step kk's MFMAs
  auto sdp = [&](uint32_t sb, f32x16 (&sn)[2], f32x16 (&pn)[2], auto&& hook) {
    i32x4 kv[KT][4];
    static_for<HEAD>([&](auto kk) { rowread(kk, sb, kv); });
    static_for<KT>([&](auto kkc) {
      constexpr int kk = decltype(kkc)::value;
      constexpr int after = (KT - 1 - kk) < (HEAD - 1) ? (KT - 1 - kk) : (HEAD - 1);
      wait4(std::integral_constant<int, 4 * after>{}, kv[kk]);
      mfma_first<T, M::QF, kk, kk == 0>(sn[0], __builtin_bit_cast(vec8, kv[kk][0]));
      mfma_first<T, M::QF, kk, kk == 0>(sn[1], __builtin_bit_cast(vec8, kv[kk][1]));
      mfma_first<T, M::GF, kk, kk == 0>(pn[0], __builtin_bit_cast(vec8, kv[kk][2]));
      mfma_first<T, M::GF, kk, kk == 0>(pn[1], __builtin_bit_cast(vec8, kv[kk][3]));
      if constexpr (kk + HEAD < KT) rowread(std::integral_constant<int, kk + HEAD>{}, sb, kv);
      hook(kkc);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // dS^T of elements K, K + 1 into dsv (packed to 16 bits)
  auto pair = [&](auto kc, auto maskc, const f32x16 (&sc)[2], const f32x16 (&pc)[2], int u, vec8 (&dsv)[4]) {
    constexpr int K = decltype(kc)::value;
    constexpr bool MASK = decltype(maskc)::value;
    constexpr int bb = K >> 4, r = K & 15, g = r >> 2, i = r & 3;
    constexpr int cr = 32 * bb + 16 * (g >> 1) + 4 * (g & 1) + i;
    float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[bb][r], c, -l2));
    float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[bb][r + 1], c, -l2));
    if constexpr (MASK) {
      p0 = cr > u ? 0.f : p0;
      p1 = cr + 1 > u ? 0.f : p1;
    }
    typedef T T2 __attribute__((ext_vector_type(2)));
    const T2 dd = {(T)(p0 * (pc[bb][r] - dl)), (T)(p1 * (pc[bb][r + 1] - dl))};
    keep_vec(dd);                         // pinned here (the compiler would sink it to the dQ MFMAs)
    dsv[K >> 3][K & 7] = dd[0];
    dsv[K >> 3][(K & 7) + 1] = dd[1];
  };

  // dQ^T += K^T dS^T of the tile in stage sb (eight transposed reads per
  // 32-channel block, the next block's in flight during the MFMAs)
  auto dq_tile = [&](uint32_t sb, const vec8 (&dsv)[4]) {
    i16x4 tr[2][8];
    auto tr_issue = [&](auto dbc, i16x4(&r)[8]) {
      constexpr int db = decltype(dbc)::value;
      constexpr int R = ROW;
      const uint32_t x = sb + TILE + (rd.voff0 ^ (uint32_t)(db << 6));
      r[0] = lds_tr16<0>(x);
      r[1] = lds_tr16<4 * R>(x);
      r[2] = lds_tr16<16 * R>(x);
      r[3] = lds_tr16<20 * R>(x);
      r[4] = lds_tr16<32 * R>(x);
      r[5] = lds_tr16<36 * R>(x);
      r[6] = lds_tr16<48 * R>(x);
      r[7] = lds_tr16<52 * R>(x);
    };
    tr_issue(std::integral_constant<int, 0>{}, tr[0]);
    static_for<DB>([&](auto dbc) {
      constexpr int db = decltype(dbc)::value;
      i16x4(&cur)[8] = tr[db & 1];
      constexpr int nb = db + 1 < DB ? 8 : 0;
      if constexpr (db + 1 < DB) tr_issue(std::integral_constant<int, db + 1>{}, tr[(db + 1) & 1]);
      lds_wait<6 + nb>(cur);
      mfma_acc<T, M::DQ + 16 * db>(tr_pair<vec8>(cur, 0), dsv[0]);
      lds_wait<4 + nb>(cur);
      mfma_acc<T, M::DQ + 16 * db>(tr_pair<vec8>(cur, 1), dsv[1]);
      lds_wait<2 + nb>(cur);
      mfma_acc<T, M::DQ + 16 * db>(tr_pair<vec8>(cur, 2), dsv[2]);
      lds_wait<0 + nb>(cur);
      mfma_acc<T, M::DQ + 16 * db>(tr_pair<vec8>(cur, 3), dsv[3]);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // round t: all copies landed (tile t + 1), barrier, copies of tile t + 2
  auto top = [&](int t) {
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    if (t + 2 < ntile) issue(t + 2);
  };
  // one tile: S^T, dP^T of tile t + 1 (NEXT) carrying dS of tile t, then dQ
  auto tile = [&](auto maskc, auto nextc, int t, f32x16 (&sc)[2], f32x16 (&pc)[2], f32x16 (&sn)[2],
                  f32x16 (&pn)[2]) {
    constexpr bool NEXT = decltype(nextc)::value;
    top(t);
    // S^T, dP^T are read through a tie placed here: the compiler would
    // otherwise hoist the (pure) vector work above the waits of this round
    asm volatile("" : "+v"(sc[0]), "+v"(sc[1]), "+v"(pc[0]), "+v"(pc[1]));
    const int u = lim - t * BN - 8 * h;
    vec8 dsv[4];
    if constexpr (NEXT) {
      sdp(stage(t + 1), sn, pn, [&](auto kkc) {
        constexpr int kk = decltype(kkc)::value;
        static_for<EPS / 2>([&](auto e) {
          pair(std::integral_constant<int, kk * EPS + 2 * decltype(e)::value>{}, maskc, sc, pc, u, dsv);
        });
      });
      pad2(sn[0], sn[1]);
      pad2(pn[0], pn[1]);
    } else {
      static_for<16>([&](auto e) {
        pair(std::integral_constant<int, 2 * decltype(e)::value>{}, maskc, sc, pc, u, dsv);
      });
    }
    __builtin_amdgcn_sched_barrier(0);
    dq_tile(stage(t), dsv);
  };

  const std::true_type masked, yes;
  const std::false_type plain, no;
  if (ntile > 0) issue(0);
  if (ntile > 1) issue(1);
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  f32x16 sA[2], pA[2], sB[2], pB[2];
  if (n_w > 0) {
    sdp(stage(0), sA, pA, [](auto) {});
    pad2(sA[0], sA[1]);
    pad2(pA[0], pA[1]);
  }
  // unrolled by two (tile t consumes set A when t is even); mask-free tiles
  // first, an even count of them, then the rest with the mask; the last
  // tile of the wave has no next tile
  const int n_free2 = n_free & ~1;
  int t = 0;
  for (; t + 2 <= n_free2 && t + 2 < n_w; t += 2) {
    tile(plain, yes, t, sA, pA, sB, pB);
    tile(plain, yes, t + 1, sB, pB, sA, pA);
  }
  for (; t + 2 < n_w; t += 2) {
    tile(masked, yes, t, sA, pA, sB, pB);
    tile(masked, yes, t + 1, sB, pB, sA, pA);
  }
  if (t + 1 < n_w) {
    tile(masked, yes, t, sA, pA, sB, pB);
    tile(masked, no, t + 1, sB, pB, sA, pA);
    t += 2;
  } else if (t < n_w) {
    tile(masked, no, t, sA, pA, sB, pB);
    ++t;
  }
  for (; t < ntile; ++t) top(t);

  wide::acc_read_pad();
  if (qi < q_len) {
    T* dqr = (T*)p.dq + (q_tok0 + qi) * qs + hq * D;
    typedef T T4 __attribute__((ext_vector_type(4)));
    static_for<DB>([&](auto dbc) {
      constexpr int db = decltype(dbc)::value;
      const f32x16 x = acc_read<M::DQ + 16 * db>();
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        T4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (T)(x[4 * g + e] * p.scale);
        *(T4*)(dqr + 32 * db + 8 * g + 4 * h) = w;
      }
    });
  }
}

template <typename T, int D, bool CAUSAL, bool VARLEN>
static hipError_t launch_dq_t(const BwdParams& p, hipStream_t s) {
  constexpr int lds = 3 * (3 * 64 * 2 * D);
  static const hipError_t attr = hipFuncSetAttribute((const void*)bwd_dq_pipe_kernel<T, D, CAUSAL, VARLEN>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((bwd_dq_pipe_kernel<T, D, CAUSAL, VARLEN>), dim3(p.grid_dq), dim3(256), lds, s, p);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_dq_v(const BwdParams& p, int causal, int varlen, hipStream_t s) {
  if (varlen) return causal ? launch_dq_t<T, D, true, true>(p, s) : launch_dq_t<T, D, false, true>(p, s);
  return causal ? launch_dq_t<T, D, true, false>(p, s) : launch_dq_t<T, D, false, false>(p, s);
}

hipError_t launch_bwd_dq(const BwdParams& p, int dtype, int d, int causal, int varlen, hipStream_t s) {
  if (dtype == 0)
    return d == 128 ? launch_dq_v<__bf16, 128>(p, causal, varlen, s) : launch_dq_v<__bf16, 64>(p, causal, varlen, s);
  return d == 128 ? launch_dq_v<_Float16, 128>(p, causal, varlen, s) : launch_dq_v<_Float16, 64>(p, causal, varlen, s);
}

}  // namespace attn
