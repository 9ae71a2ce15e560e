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

// Per-lane LDS byte offsets of the two read patterns over a tile of rows of
// D 16-bit elements (row stride 2 D bytes):
//   row reads  (A/B operand, 8 consecutive elements of row key_perm(l % 32)):
//              koff(kk) = koff0 ^ (kk << 5), +32 rows per 32-row block;
//   transposed (A operand: 32 columns x 16 rows, ds_read_b64_tr_b16 pairs):
//              voff(db) = voff0 ^ (db << 6), + 16 rows per chunk, second
//              read + 4 rows.
template <int D>
struct TileReads {
  static constexpr int ROW = 2 * D;
  int koff0;
  uint32_t voff0;
  __device__ __forceinline__ TileReads(int lane) {
    const int h = lane >> 5, l32 = lane & 31;
    const int r0 = key_perm(l32);
    koff0 = r0 * ROW + ((h ^ swz_k<D>(r0)) << 4);
    const int G = lane >> 4, i16 = lane & 15;
    const int r = 8 * h + (i16 >> 2);
    const int dd = 16 * (G & 1) + 4 * (i16 & 3);
    voff0 = r * ROW + (((dd >> 3) ^ swz_v<D>(r)) << 4) + ((dd & 7) << 1);
  }
  __device__ __forceinline__ int koff(int kk) const { return koff0 ^ (kk << 5); }
  __device__ __forceinline__ uint32_t voff(int db) const { return voff0 ^ (uint32_t)(db << 6); }
};

// DMA offsets of the copy of a tile of ROWS rows (row stride `stride`
// elements in global memory) by NW waves, for either swizzle.
template <int D, int ROWS, int NW>
struct TileCopy {
  static constexpr int CPR = D / 8;
  static constexpr int LOADS = ROWS * CPR / (NW * 64);
  static_assert(LOADS >= 1 && ROWS * CPR % (NW * 64) == 0, "tile copy shape");
  uint32_t k[LOADS], v[LOADS];
  __device__ __forceinline__ TileCopy(int wave, int lane, int stride) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int pos = (wave * LOADS + i) * 64 + lane;
      const int row = pos / CPR, phys = pos % CPR;
      k[i] = (uint32_t)(row * stride * 2 + ((phys ^ swz_k<D>(row)) << 4));
      v[i] = (uint32_t)(row * stride * 2 + ((phys ^ swz_v<D>(row)) << 4));
    }
  }
};

// Eight transposed reads (ds_read_b64_tr_b16): the A operands of two 16-row
// chunks at each of the addresses a0 and a1 (r[2 c], r[2 c + 1] = chunk c of
// a0; r[4 + 2 c], r[5 + 2 c] = chunk c of a1, c = 0, 1).  Wait for them with
// lds_wait; pair j is complete once at most 6 - 2 j reads issued after it
// are outstanding.
template <int D>
__device__ __forceinline__ void tr_issue8(uint32_t a0, uint32_t a1, i16x4 (&r)[8]) {
  constexpr int R = 2 * D;
  r[0] = lds_tr16<0>(a0);
  r[1] = lds_tr16<4 * R>(a0);
  r[2] = lds_tr16<16 * R>(a0);
  r[3] = lds_tr16<20 * R>(a0);
  r[4] = lds_tr16<0>(a1);
  r[5] = lds_tr16<4 * R>(a1);
  r[6] = lds_tr16<16 * R>(a1);
  r[7] = lds_tr16<20 * R>(a1);
}

template <typename V>
__device__ __forceinline__ V tr_pair(const i16x4 (&r)[8], int j) {
  const i16x8 w = __builtin_shufflevector(r[2 * j], r[2 * j + 1], 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(V, w);
}

// ---------------------------------------------------------------- dK, dV
// VARLEN: p.B sequences packed along the token axis (cu_seqlens); workgroup
// = (KV head, sequence, key block), the statistics read directly from global
// memory (their per-sequence rows are not 16-byte aligned for the copy).
template <typename T, int D, bool CAUSAL, bool VARLEN>
__global__ void __launch_bounds__(256) bwd_dkdv_kernel(BwdParams p) {
  typedef typename Mma<T>::vec8 vec8;
  constexpr int BMQ = 32;                 // query rows per step
  constexpr int KT = D / 16;              // k-steps over the head dimension
  constexpr int DB = D / 32;              // 32-column blocks of dK^T, dV^T
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

  // key blocks in ascending order first: with causal masking the first ones
  // see the most queries (longest first)
  int b, hkv, nblk, q_len, k_len;
  long long q_tok0, k_tok0;               // token index of the sequence's first query / key
  if constexpr (VARLEN) {
    hkv = blockIdx.x % p.Hkv;
    int r = blockIdx.x / p.Hkv, sq = 0, start = 0, len = 0;
    for (; sq < p.B; ++sq) {
      start = p.cu_seqlens[sq];
      len = p.cu_seqlens[sq + 1] - start;
      const int nb = (len + kBwdBlockN - 1) / kBwdBlockN;
      if (r < nb) break;
      r -= nb;
    }
    if (sq >= p.B) return;                // beyond the last block (uniform over the workgroup)
    b = 0;
    nblk = r;
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

  // K and V of the lane's key as B operands (k = head dimension); rows past
  // the end read a valid row and are masked
  vec8 kf[KT], vf[KT];
  {
    const long long row = (k_tok0 + min(key, k_len - 1)) * p.Hkv + hkv;
    const T* kr = (const T*)p.k + row * D + 8 * h;
    const T* vr = (const T*)p.v + row * D + 8 * h;
#pragma unroll
    for (int kk = 0; kk < KT; ++kk) {
      kf[kk] = *(const vec8*)(kr + 16 * kk);
      vf[kk] = *(const vec8*)(vr + 16 * kk);
    }
  }
  f32x16 dv[DB], dk[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) {
    dv[i] = f32x16{};
    dk[i] = f32x16{};
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
  auto issue = [&](int s) {
    int hq, q0;
    step_coords(s, hq, q0);
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
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    if (s + 1 < nsteps) issue(s + 1);
    int hq, q0;
    step_coords(s, hq, q0);
    const char* st = smem + (s & 1) * STAGE;
    const uint32_t stl = lds0 + (s & 1) * STAGE;

    // S = Q K^T and dP = dO V^T: row m of the MFMA is query key_perm(m)
    f32x16 sacc = f32x16{}, pacc = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KT; ++kk) {
      const vec8 qa = *(const vec8*)(st + 0 * QT + rd.koff(kk));
      const vec8 ga = *(const vec8*)(st + 2 * QT + rd.koff(kk));
      sacc = Mma<T>::run(qa, kf[kk], sacc);
      pacc = Mma<T>::run(ga, vf[kk], pacc);
    }
    // register r = 4 g + i holds query 16 (g >> 1) + 8 h + 4 (g & 1) + i:
    // 4 consecutive queries per g, read as 2 x 16 bytes of (lse2, delta)
    // (varlen: from global memory, rows past the sequence clamped to its last
    // row -- their Q and dO are zero, so they contribute nothing)
    const float* sp = (const float*)(st + 4 * QT);
    const float2* sg = p.stats + (long long)hq * p.Sq + q_tok0;   // varlen layout [Hq, T]
    vec8 pv[2], dsv[2];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int qr = 16 * (g >> 1) + 8 * h + 4 * (g & 1);
      float l2[4], dl[4];
      if constexpr (VARLEN) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float2 v2 = sg[min(q0 + qr + i, q_len - 1)];
          l2[i] = v2.x;
          dl[i] = v2.y;
        }
      } else {
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
    // transposed reads of block db + 1 are in flight during block db's MFMAs
    __builtin_amdgcn_sched_barrier(0);
    i16x4 tr[2][8];
    tr_issue8<D>(stl + 3 * QT + rd.voff(0), stl + 1 * QT + rd.voff(0), tr[0]);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      i16x4 (&cur)[8] = tr[db & 1];
      if (db + 1 < DB) {
        tr_issue8<D>(stl + 3 * QT + rd.voff(db + 1), stl + 1 * QT + rd.voff(db + 1), tr[(db + 1) & 1]);
        lds_wait<14>(cur);
        dv[db] = Mma<T>::run(tr_pair<vec8>(cur, 0), pv[0], dv[db]);
        lds_wait<12>(cur);
        dv[db] = Mma<T>::run(tr_pair<vec8>(cur, 1), pv[1], dv[db]);
        lds_wait<10>(cur);
        dk[db] = Mma<T>::run(tr_pair<vec8>(cur, 2), dsv[0], dk[db]);
        lds_wait<8>(cur);
        dk[db] = Mma<T>::run(tr_pair<vec8>(cur, 3), dsv[1], dk[db]);
      } else {
        lds_wait<6>(cur);
        dv[db] = Mma<T>::run(tr_pair<vec8>(cur, 0), pv[0], dv[db]);
        lds_wait<4>(cur);
        dv[db] = Mma<T>::run(tr_pair<vec8>(cur, 1), pv[1], dv[db]);
        lds_wait<2>(cur);
        dk[db] = Mma<T>::run(tr_pair<vec8>(cur, 2), dsv[0], dk[db]);
        lds_wait<0>(cur);
        dk[db] = Mma<T>::run(tr_pair<vec8>(cur, 3), dsv[1], dk[db]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // dK^T, dV^T: lane holds key `key` and channels 32 db + 8 g + 4 h + 0..3
  if (key < k_len) {
    const long long row = (k_tok0 + key) * p.Hkv + hkv;
    T* dkr = (T*)p.dk + row * D;
    T* dvr = (T*)p.dv + row * D;
    typedef T T4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        T4 wk, wv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          wk[e] = (T)(dk[db][4 * g + e] * p.scale);
          wv[e] = (T)dv[db][4 * g + e];
        }
        *(T4*)(dkr + 32 * db + 8 * g + 4 * h) = wk;
        *(T4*)(dvr + 32 * db + 8 * g + 4 * h) = wv;
      }
  }
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
  constexpr int lds_kv = 2 * (4 * 32 * 2 * D + 1024);
  constexpr int lds_q = 3 * (3 * 64 * 2 * D);
  static const hipError_t a1 = hipFuncSetAttribute((const void*)bwd_dkdv_kernel<T, D, CAUSAL, VARLEN>,
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, lds_kv);
  static const hipError_t a2 = hipFuncSetAttribute((const void*)bwd_dq_kernel<T, D, CAUSAL, VARLEN>,
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, lds_q);
  if (a1 != hipSuccess) return a1;
  if (a2 != hipSuccess) return a2;
  hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, CAUSAL, VARLEN>), dim3(p.grid_dkdv), dim3(256), lds_kv, s, p);
  e = hipGetLastError();
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
