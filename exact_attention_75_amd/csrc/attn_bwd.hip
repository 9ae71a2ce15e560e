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
//                    7.3.1), padded to 32 rows per head.
//   bwd_dkdv_kernel  one workgroup per (batch, KV head, 128 keys); each wave
//                    owns 32 keys and keeps their K, V fragments and dK, dV
//                    accumulators in registers, and walks the query blocks of
//                    every query head of the KV group (so GQA sums in
//                    registers and no atomics are needed).  Per 32-query step:
//                    S = Q K^T and dP = dO V^T (query rows x keys, so the
//                    accumulator of each is directly the B operand of the
//                    next MFMAs), P, dS, then dV^T += dO^T P and
//                    dK^T += Q^T dS with the transposed operands read from
//                    LDS by ds_read_b64_tr_b16.
//   bwd_dq_kernel    one workgroup per (batch, query head, 128 query rows),
//                    like the forward: S^T = K Q^T, dP^T = V dO^T (a lane
//                    owns a query, so LSE and delta are lane scalars),
//                    dS^T, then dQ^T += K^T dS^T.
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

#include "bwd_common.h"
#include "kernel_common.h"
#include "kernels.h"

namespace attn {

// ---------------------------------------------------------------- preprocess
// D/8 consecutive threads own one row (16 bytes of o and dO each, one
// coalesced row per thread group) and sum their partial dot products with
// shuffles.  Rows i in [Sq, Sq_pad) of the statistics get (+inf, 0): P = 0
// there.
template <typename T, int D>
__global__ void __launch_bounds__(256) bwd_pre_kernel(BwdParams p) {
  typedef typename Mma<T>::vec8 vec8;
  constexpr int TPR = D / 8;                 // threads per row
  const long long rows = (long long)p.B * p.Sq_pad * p.Hq;
  const long long rp = ((long long)blockIdx.x * 256 + threadIdx.x) / TPR;   // (b * Sq_pad + i) * Hq + h
  const int t = threadIdx.x % TPR;
  if (rp >= rows) return;                    // whole thread groups leave together
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

// ---------------------------------------------------------------- dQ
// Per-wave software pipeline over 64-key tiles: the MFMAs of S^T_{t+1} and
// dP^T_{t+1} carry the vector work of tile t (P = exp2(c s - lse2), masked,
// dS = P (dP - delta), packed to 16 bits), then dQ^T += K_t^T dS_t^T.  Three
// LDS stages: during tile t the copies of tile t + 2 are in flight, tile
// t + 1 feeds S and dP, and tile t's transposed K copy feeds dQ.
// VARLEN: workgroup = (query head, sequence, 128-row block), longest block of
// a sequence first.
template <typename T, int D, bool CAUSAL, bool VARLEN>
__global__ void __launch_bounds__(256) bwd_dq_kernel(BwdParams p) {
  typedef typename Mma<T>::vec8 vec8;
  constexpr int BN = 64;                  // keys per tile
  constexpr int NB = BN / 32;
  constexpr int KT = D / 16;
  constexpr int DB = D / 32;
  constexpr int ROW = 2 * D;
  constexpr int TILE = BN * ROW;
  constexpr int NST = 3;                  // LDS stages
  // stage: [K row-swizzled | K transposed-swizzled | V row-swizzled]
  constexpr int STAGE = 3 * TILE;
  constexpr int EPS = 2 * 16 / KT;        // dS elements per k-step of the next tile's MFMAs
  extern __shared__ __attribute__((aligned(16))) char smem[];
  static_assert(NB == 2, "four 16-key chunks per tile");

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
    for (; sq < p.B; ++sq) {
      start = p.cu_seqlens[sq];
      len = p.cu_seqlens[sq + 1] - start;
      nb = (len + kBwdBlockM - 1) / kBwdBlockM;
      if (r < nb) break;
      r -= nb;
    }
    if (sq >= p.B) return;                // beyond the last tile (uniform over the workgroup)
    b = 0;
    mblk = nb - 1 - r;                    // longest query block of the sequence first
    q_len = k_len = len;
    q_tok0 = k_tok0 = start;
    stat0 = (long long)hq * p.Sq + start;   // varlen layout [Hq, T]
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

  // Q and dO of the lane's query as B operands (k = head dimension)
  vec8 qf[KT], gf[KT];
  {
    const long long row = (q_tok0 + qc) * p.Hq + hq;
    const T* qr = (const T*)p.q + row * D + 8 * h;
    const T* gr = (const T*)p.dout + row * D + 8 * h;
#pragma unroll
    for (int kk = 0; kk < KT; ++kk) {
      qf[kk] = *(const vec8*)(qr + 16 * kk);
      gf[kk] = *(const vec8*)(gr + 16 * kk);
    }
  }
  const float2 st2 = p.stats[stat0 + qc];
  const float l2 = st2.x, dl = st2.y;
  const float c = p.scale_log2;

  f32x16 dq[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) dq[i] = f32x16{};

  const TileCopy<D, BN, 4> cp(wave, lane, ks);
  const TileReads<D> rd(lane);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(LDS_AS char*)smem;
  const T* kbase = (const T*)p.k + k_tok0 * ks + hkv * D;
  const T* vbase = (const T*)p.v + k_tok0 * ks + hkv * D;
  auto issue = [&](int t) {
    char* st = smem + (t % NST) * STAGE;
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

  // S^T and dP^T of tile t: row m of block bb is key 64 t + 32 bb + key_perm(m).
  // step(kk) runs after the MFMAs of k-step kk.
  auto sdp = [&](int t, f32x16 (&sa)[NB], f32x16 (&pa)[NB], auto&& step) {
    const char* st = smem + (t % NST) * STAGE;
#pragma unroll
    for (int kk = 0; kk < KT; ++kk) {
      vec8 ka[NB], va[NB];
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) {
        ka[bb] = *(const vec8*)(st + 0 * TILE + rd.koff(kk) + bb * 32 * ROW);
        va[bb] = *(const vec8*)(st + 2 * TILE + rd.koff(kk) + bb * 32 * ROW);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) {
        sa[bb] = Mma<T>::run(ka[bb], qf[kk], kk == 0 ? f32x16{} : sa[bb]);
        pa[bb] = Mma<T>::run(va[bb], gf[kk], kk == 0 ? f32x16{} : pa[bb]);
      }
      step(kk);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // dS^T of tile t, flattened elements e0 .. e0 + n - 1 (element k: block
  // k >> 4, register k & 15); chunk cc of 16 keys = elements 8 cc .. 8 cc + 7
  auto ds_elems = [&](int t, const f32x16 (&sc)[NB], const f32x16 (&pc)[NB], int e0, int n, vec8 (&dsv)[2 * NB]) {
    const int j0 = t * BN;
#pragma unroll
    for (int k = e0; k < e0 + n; ++k) {
      const int bb = k >> 4, r = k & 15;
      const int g = r >> 2, i = r & 3;
      const int key = j0 + 32 * bb + 16 * (g >> 1) + 8 * h + 4 * (g & 1) + i;
      const bool dead = (key >= k_len) || (CAUSAL && key > qi);
      const float pr = dead ? 0.f : __builtin_amdgcn_exp2f(__builtin_fmaf(sc[bb][r], c, -l2));
      dsv[k >> 3][k & 7] = (T)(pr * (pc[bb][r] - dl));
    }
  };
  // dQ^T += K_t^T dS_t^T (eight transposed reads per 32-channel block, the
  // next block's in flight during the MFMAs)
  auto dq_tile = [&](int t, const vec8 (&dsv)[2 * NB]) {
    __builtin_amdgcn_sched_barrier(0);
    i16x4 tr[2][8];
    const uint32_t kt = lds0 + (t % NST) * STAGE + 1 * TILE;
    tr_issue8<D>(kt + rd.voff(0), kt + rd.voff(0) + 32 * ROW, tr[0]);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      i16x4 (&cur)[8] = tr[db & 1];
      if (db + 1 < DB) {
        tr_issue8<D>(kt + rd.voff(db + 1), kt + rd.voff(db + 1) + 32 * ROW, tr[(db + 1) & 1]);
        lds_wait<14>(cur);
        dq[db] = Mma<T>::run(tr_pair<vec8>(cur, 0), dsv[0], dq[db]);
        lds_wait<12>(cur);
        dq[db] = Mma<T>::run(tr_pair<vec8>(cur, 1), dsv[1], dq[db]);
        lds_wait<10>(cur);
        dq[db] = Mma<T>::run(tr_pair<vec8>(cur, 2), dsv[2], dq[db]);
        lds_wait<8>(cur);
        dq[db] = Mma<T>::run(tr_pair<vec8>(cur, 3), dsv[3], dq[db]);
      } else {
        lds_wait<6>(cur);
        dq[db] = Mma<T>::run(tr_pair<vec8>(cur, 0), dsv[0], dq[db]);
        lds_wait<4>(cur);
        dq[db] = Mma<T>::run(tr_pair<vec8>(cur, 1), dsv[1], dq[db]);
        lds_wait<2>(cur);
        dq[db] = Mma<T>::run(tr_pair<vec8>(cur, 2), dsv[2], dq[db]);
        lds_wait<0>(cur);
        dq[db] = Mma<T>::run(tr_pair<vec8>(cur, 3), dsv[3], dq[db]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // one tile: S^T, dP^T of tile t + 1 (when has_next) with dS of tile t, then dQ
  auto tile = [&](int t, bool has_next, const f32x16 (&sc)[NB], const f32x16 (&pc)[NB], f32x16 (&sn)[NB],
                  f32x16 (&pn)[NB]) {
    vec8 dsv[2 * NB];
    if (has_next) {
      sdp(t + 1, sn, pn, [&](int kk) { ds_elems(t, sc, pc, kk * EPS, EPS, dsv); });
    } else {
      ds_elems(t, sc, pc, 0, 32, dsv);
    }
    dq_tile(t, dsv);
  };
  // round t: all copies landed (tile t + 1), barrier, copies of tile t + 2
  auto top = [&](int t) {
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    if (t + 2 < ntile) issue(t + 2);
  };

  if (ntile > 0) issue(0);
  if (ntile > 1) issue(1);
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  f32x16 sA[NB], pA[NB], sB[NB], pB[NB];
  if (n_w > 0) sdp(0, sA, pA, [](int) {});
  int t = 0;
  for (; t + 1 < n_w; t += 2) {          // unrolled by two: the S / dP sets swap roles
    top(t);
    tile(t, true, sA, pA, sB, pB);
    top(t + 1);
    tile(t + 1, t + 2 < n_w, sB, pB, sA, pA);
  }
  if (t < n_w) {
    top(t);
    tile(t, false, sA, pA, sB, pB);
    ++t;
  }
  for (; t < ntile; ++t) top(t);

  if (qi < q_len) {
    T* dqr = (T*)p.dq + (q_tok0 + qi) * qs + hq * D;
    typedef T T4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        T4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (T)(dq[db][4 * g + e] * p.scale);
        *(T4*)(dqr + 32 * db + 8 * g + 4 * h) = w;
      }
  }
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
  const long long threads = (long long)pp.B * pp.Sq_pad * pp.Hq * (D / 8);
  hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, pp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int lds_q = 3 * (3 * 64 * 2 * D);
  static const hipError_t a2 = hipFuncSetAttribute((const void*)bwd_dq_kernel<T, D, CAUSAL, VARLEN>,
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, lds_q);
  if (a2 != hipSuccess) return a2;
  e = launch_bwd_dkdv(p, std::is_same<T, __bf16>::value ? 0 : 1, D, CAUSAL, VARLEN, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dq_kernel<T, D, CAUSAL, VARLEN>), dim3(p.grid_dq), dim3(256), lds_q, s, p);
  return hipGetLastError();
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
