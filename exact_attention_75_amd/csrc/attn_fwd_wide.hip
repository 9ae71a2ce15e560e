// attn_fwd_wide.hip -- fused attention forward for gfx950, d = 128 dense,
// bf16/fp16, one wave per SIMD.
//
// Same computation as attn_fwd.hip (O = softmax(scale * Q K^T + mask) V and
// the natural-log LSE, "FlashAttention-3 Deep Dive", introduction formula;
// Hopper tag page contents 4.2 and 4.6 for the streaming softmax state), with
// a different split of the work over the CU:
//
//  * A workgroup is 4 waves and owns BM = 256 query rows; each wave owns 64
//    of them (two 32-row blocks) and has a SIMD to itself.  Every K or V
//    fragment a wave reads from LDS feeds two MFMAs (one per 32-row block),
//    which halves the LDS read traffic per FLOP of the 32-rows-per-wave
//    layout; at the MFMA peak that layout needs about as many LDS bytes per
//    clock as the LDS delivers.  Q stays in registers for the whole loop.
//  * With one wave per SIMD all overlap of matrix and vector work happens
//    inside the wave.  Iteration t runs
//        A: S_t = K_t Q^T (32 MFMA)        with exp2 of the second half of
//                                          S_{t-1}; then the check of tile t-1
//        B: O += P_{t-1} V_{t-1} (32 MFMA) with the mask of S_t and exp2 of
//                                          its first half
//    so the softmax of a tile runs under the matrix products of the two
//    stretches around it (the pages' overlap of the GEMMs with the softmax,
//    "flash-attention-3", "Why a schedule", within one instruction stream).
//  * K and V tiles stream global -> LDS through four-slot rings of
//    direct-to-LDS copies, two tiles ahead, with one workgroup barrier per
//    two key tiles.  Every round issues the same copies (a copy past the
//    last tile has an empty buffer range and writes zeros into a free slot),
//    so the loop has no branches around them.
//  * The running max is exact after the first key tile and then moves only
//    when a tile's probabilities, taken against the current max, sum to more
//    than PMAX in some lane: the sum bounds every probability of the tile, so
//    no per-tile row max is needed (P <= PMAX, far inside the fp32, bf16 and
//    fp16 ranges).  Then -- rarely -- the tile's row max is taken, O and l
//    are rescaled and the tile's probabilities recomputed.
//  * Head-packed launches with more tiles than compute units are
//    persistent: one workgroup per CU runs a balanced share of its XCD's
//    longest-first tile list.  Between two tiles the next tile's Q rows are
//    loaded during the last P V of the current one (its Q registers are
//    free by then), and the finished tile's epilogue (O / l, LSE, stores)
//    runs after the next tile's first iteration (its S and row max leave O
//    alone), with that tile's copies already in flight; its stores drain
//    during the following iterations.  A fresh workgroup per tile instead
//    waits for its Q and first K/V tiles and runs its epilogue alone, ~9 us
//    of fixed cost per tile (measured on full attention at 8K and 16K).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>

#include <type_traits>

#include "kernel_common.h"
#include "kernels.h"
#include "wide_regs.h"

namespace attn {

using namespace wide;

template <int N>
using ic = std::integral_constant<int, N>;

// H4 (grouped-query attention with a group of 4k heads): the workgroup owns
// 64 query rows of four query heads of one KV head, one head per wave, and
// p.tm runs over (batch, head quadruple, 64-row block).  All four waves then
// see the same keys, so a causal workgroup has no waves idling past their
// diagonal while the last one finishes.
// VCOL: V given column-major, [B, Hkv, D, Sk] (key index innermost; the
// V_colmajor input of the FP8 layout discussion, "FlashAttention-3 Deep
// Dive"): the V tile is D channel rows of 64 keys, and the second GEMM's
// operand is read with one plain 16-byte read per fragment instead of two
// transposing reads.
template <typename T, bool CAUSAL, bool H4, bool VCOL>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
fwd_wide_kernel(FwdParams p) {
  typedef typename Mma<T>::vec8 vec8;
  constexpr int NW = 4;                // waves per workgroup
  constexpr int QB = 2;                // 32-row query blocks per wave
  constexpr int BM = 32 * QB * NW;     // 256 query rows per workgroup
  constexpr int BN = 64;               // keys per tile
  constexpr int D = 128;
  constexpr int CPR = D / 8;           // 16-byte chunks per row
  constexpr int KT = D / 16;           // k-steps of the first GEMM
  constexpr int NB = BN / 32;          // 32-key blocks per tile
  constexpr int NC = BN / 16;          // 16-key chunks per tile (second GEMM)
  constexpr int DB = D / 32;           // 32-column blocks of O^T
  constexpr int ROW = D * 2;           // bytes per K/V row in LDS
  constexpr int TILE = BN * ROW;       // 16 KiB per K or V tile
  constexpr int LOADS = BN * CPR / (NW * 64);   // copies per wave per tensor per tile
#ifndef ATTN_WIDE_STAGES
#define ATTN_WIDE_STAGES 4
#endif
  constexpr int STAGES = ATTN_WIDE_STAGES;   // K and V ring depth
#ifndef ATTN_WIDE_NBX
#define ATTN_WIDE_NBX 4
#endif
  // The 64 exponentials per lane of a tile come in 8 groups of 8: group g is
  // chunk g / 2 of query block g % 2.  The first NBX groups of S_t run in
  // stretch B of iteration t, the other groups in stretch A of iteration t+1.
  constexpr int NBX = ATTN_WIDE_NBX;
  constexpr int EA = 8 - NBX;          // exponentials per k-step of A
  constexpr float PMAX = 16384.0f;       // bound on a lane's share of a tile's probability sum
  constexpr float NEG_INF = -__builtin_inff();
  static_assert(LOADS == 4 && QB == 2 && DB == 4 && NB == 2 && KT == 8, "tile shape");
  // [K ring | V ring]
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int l32 = lane & 31;

  const int q_len = p.Sq, kv_len = p.Sk;
  const int qs = p.q_tok_stride;
  const int ks = p.kv_tok_stride;
  constexpr int ROWS = H4 ? 64 : BM;                    // query rows per head of the workgroup

  // ---------------------------------------------------------------- tiles
  // A workgroup runs one tile, or (persistent launch: fewer workgroups than
  // tiles) the tiles j, 2 J - 1 - j, 2 J + j, ... of its XCD's longest-first
  // list, j its index among the XCD's J workgroups.
  const int ntl = p.tm.ntiles;
  const bool persist = H4 && (int)gridDim.x < ntl;
  const int xg = blockIdx.x % kNumXcd, jg = blockIdx.x / kNumXcd, JG = gridDim.x / kNumXcd;
  auto tile_of_round = [&](int rr) {
    if (!persist) return rr == 0 ? (int)blockIdx.x : ntl;
    const int sl = rr * JG + ((rr & 1) ? JG - 1 - jg : jg);
    return xg + kNumXcd * sl;
  };
  int b, hq, mblk, hkv, q0, qw, q_hi, kv_end, ntile, n_w, t_edge;
  const T *Qp, *Kp, *Vp;
  T* Op;
  long long lse_off;
  auto tile_setup = [&](int pt) {
    tile_decode(p.tm, pt, b, hq, mblk);
    if constexpr (H4) hq = 4 * hq + wave;
    hkv = hq / p.group;
    Qp = (const T*)p.q + (long long)b * p.q_batch_stride + hq * D;
    Kp = (const T*)p.k + (long long)b * p.kv_batch_stride + hkv * D;
    Vp = (const T*)p.v + (long long)b * p.kv_batch_stride + hkv * D;
    Op = (T*)p.o + (long long)b * p.q_batch_stride + hq * D;
    lse_off = ((long long)b * p.Hq + hq) * p.Sq;
    q0 = mblk * ROWS;
    qw = H4 ? q0 : q0 + 64 * wave;              // first query row of this wave
    q_hi = q0 + ROWS < q_len ? q0 + ROWS : q_len;
    kv_end = CAUSAL ? (kv_len < q_hi ? kv_len : q_hi) : kv_len;
    ntile = (kv_end + BN - 1) / BN;
    // key tiles this wave computes: up to its diagonal when causal, none when
    // all its rows are past the end of the sequence
    n_w = CAUSAL ? min(ntile, (qw + 63) / BN + 1) : ntile;
    if (qw >= q_len) n_w = 0;
    // Tile t needs the mask when it reaches past the last key (t BN + BN >
    // kv_len) or, causal, past the wave's first row (t BN + BN - 1 > qw); both
    // hold from some t on, so one comparison with the first such t decides.
    t_edge = CAUSAL ? min(kv_len / BN, (qw + 1) / BN) : kv_len / BN;
  };

  // ---------------------------------------------------------------- Q, O
  // B operand of S^T = K Q^T: lane holds query qw + 32 qb + l32, head-dim
  // 16 kk + 8 h .. +7 (rows past the end repeat the last row; never stored).
  // The loads land before the first round's barrier (vmcnt(0)).
  auto q_issue_at = [&](const T* qbase, int qwv) {
    auto qrow = [&](int qb) {
      const int r = qwv + 32 * qb + l32;
      return qbase + (long long)(r < q_len ? r : q_len - 1) * qs + 8 * h;
    };
    const T* q0p = qrow(0);
    const T* q1p = qrow(1);
    q_load<0, 0>(q0p + 0);   q_load<0, 1>(q0p + 16);  q_load<0, 2>(q0p + 32);  q_load<0, 3>(q0p + 48);
    q_load<0, 4>(q0p + 64);  q_load<0, 5>(q0p + 80);  q_load<0, 6>(q0p + 96);  q_load<0, 7>(q0p + 112);
    q_load<1, 0>(q1p + 0);   q_load<1, 1>(q1p + 16);  q_load<1, 2>(q1p + 32);  q_load<1, 3>(q1p + 48);
    q_load<1, 4>(q1p + 64);  q_load<1, 5>(q1p + 80);  q_load<1, 6>(q1p + 96);  q_load<1, 7>(q1p + 112);
  };
  // the Q rows of tile pt, without touching the current tile's state
  // (QLOADS load instructions per wave)
  constexpr int QLOADS = 2 * KT;
  auto q_issue_tile = [&](int ptv) {
    int bv, hv, mv;
    tile_decode(p.tm, ptv, bv, hv, mv);
    if constexpr (H4) hv = 4 * hv + wave;
    const int q0v = mv * ROWS;
    q_issue_at((const T*)p.q + (long long)bv * p.q_batch_stride + hv * D, H4 ? q0v : q0v + 64 * wave);
  };
  int next_pt = ntl;     // the workgroup's next tile (ntl: none)
  bool q_early = false;  // its Q loads went out during this tile's last iteration

  // ---------------------------------------------------------------- K/V copies
  // Lane L of copy i fetches the global 16-byte chunk that belongs at LDS
  // position (wave*LOADS + i)*64 + L of the tile under the row swizzle.  Tiles
  // past the last one get an empty range: the copy writes zeros.
  uint32_t kdma[LOADS], vdma[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int pos = (wave * LOADS + i) * 64 + lane;
    const int row = pos / CPR, phys = pos % CPR;
    kdma[i] = (uint32_t)(row * ks * 2 + ((phys ^ swz_k<D>(row)) << 4));
    if constexpr (VCOL) {
      // V^T tile: D channel rows of BN keys = 8 chunks of 16 bytes, chunk c
      // of row r stored at c ^ (r & 7); global rows are Sk keys apart
      const int vr = pos / 8, vc = pos % 8;
      vdma[i] = (uint32_t)(vr * p.Sk * 2 + ((vc ^ (vr & 7)) << 4));
    } else {
      vdma[i] = (uint32_t)(row * ks * 2 + ((phys ^ swz_v<D>(row)) << 4));
    }
  }
  static_assert(!VCOL || BN * 2 == 8 * 16, "V^T tile rows of 8 chunks");
  // column-major V: this (batch, KV head)'s [D, Sk] plane
  const T* Vt = nullptr;
  // the copies of one K or V tile: source, size and destination, all
  // wave-uniform
  struct Copy {
    const void* src;
    uint32_t bytes;
    char* dst;
  };
  // K tiles 0, 1, 2, ... and V tiles 0, 1, 2, ... go out in order, so each
  // tensor keeps a running copy state (a few scalar adds per tile instead of
  // a 64-bit address product and a branch): the address of its next tile,
  // the bytes from there to the end of its range, the keys from the tile's
  // first key to kv_end (none left: the copy gets an empty range and writes
  // zeros) and the ring slot.  The range of a row-major tensor ends at
  // kv_end: keys from there to the tile's end read zeros, and every row of
  // the workgroup masks them.  The column-major V plane's range ends at the
  // plane's end: keys past Sk read the next channel's (finite) values, or
  // zeros past the plane; their P is 0.
  struct Stream {
    uint64_t src;
    uint32_t bytes;
    uint32_t step;
    int keys;
    int slot;
  };
  Stream ks_k, ks_v;
  auto streams_setup = [&]() {
    if constexpr (VCOL) Vt = (const T*)p.v + ((long long)b * p.Hkv + hkv) * D * p.Sk;
    ks_k = Stream{(uint64_t)(uintptr_t)Kp, (uint32_t)kv_end * (uint32_t)ks * 2u, (uint32_t)(BN * ks * 2), kv_end, 0};
    ks_v = VCOL ? Stream{(uint64_t)(uintptr_t)Vt, (uint32_t)(D * p.Sk) * 2u, (uint32_t)(BN * 2), kv_end, 0}
                : Stream{(uint64_t)(uintptr_t)Vp, (uint32_t)kv_end * (uint32_t)ks * 2u, (uint32_t)(BN * ks * 2), kv_end, 0};
  };
  auto next_copy = [&](Stream& st, int ring) {
    const Copy cp{(const void*)(uintptr_t)st.src, st.keys > 0 ? st.bytes : 0u,
                  smem + (ring + st.slot) * TILE + wave * LOADS * 1024};
    st.src += st.step;
    st.bytes -= st.step;
    st.keys -= BN;
    st.slot = st.slot + 1 == STAGES ? 0 : st.slot + 1;
    return cp;
  };
  auto issue_copy = [&](const Copy& cp, const uint32_t(&off)[LOADS]) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) copy_row_to_lds(cp.src, cp.bytes, cp.dst + i * 1024, off[i]);
  };
  // ring slot of tile t (t >= -1)
  auto slot_of = [&](int t) { return (t + STAGES) % STAGES; };

  // ---------------------------------------------------------------- LDS reads
  const uint32_t lds0 = (uint32_t)(uintptr_t)(LDS_AS char*)smem;
  // K: lane reads key row key_perm(l32) (+32 for the second block, an
  // immediate), chunk 2 kk + h stored at chunk (2 kk + h) ^ swz_k(row); the
  // ring slot is added per iteration
  uint32_t kaddr[KT];
  {
    const int r = key_perm(l32);
    const uint32_t koff0 = r * ROW + ((h ^ swz_k<D>(r)) << 4);
#pragma unroll
    for (int kk = 0; kk < KT; ++kk) kaddr[kk] = lds0 + (koff0 ^ (uint32_t)(kk << 5));
  }
  // V (transposing reads): channel block db at (voff0 ^ (db << 6)); chunk
  // (16 rows) and the second read (4 rows) are immediates, the ring slot is
  // added per iteration
  uint32_t vaddr[DB];
  if constexpr (VCOL) {
    // column-major: lane reads channel row 32 db + l32 (db: an immediate),
    // keys 16 CC + 8 h .. + 7 = chunk 2 CC + h of the row, stored at
    // (2 CC + h) ^ (l32 & 7)
#pragma unroll
    for (int cc = 0; cc < NC; ++cc)
      vaddr[cc] = lds0 + STAGES * TILE + l32 * 128 + ((((2 * cc + h) ^ (l32 & 7))) << 4);
  } else {
    const int G = lane >> 4, i16 = lane & 15;
    const int r = 8 * h + (i16 >> 2);
    const int dd = 16 * (G & 1) + 4 * (i16 & 3);
    const uint32_t voff0 = r * ROW + ((((dd >> 3) ^ swz_v<D>(r))) << 4) + ((dd & 7) << 1);
#pragma unroll
    for (int db = 0; db < DB; ++db) vaddr[db] = lds0 + STAGES * TILE + (voff0 ^ (uint32_t)(db << 6));
  }
  static_assert(NC == DB, "one V address per chunk (column-major) or per channel block");
  // K fragments of k-step KK of the tile at byte offset kst into register
  // ring slot KK % 3
  auto read_k = [&](uint32_t kst, auto kk_tag) {
    constexpr int KK = decltype(kk_tag)::value;
    const uint32_t a = kaddr[KK] + kst;
    k_read<KK % 3, 0, 0>(a);
    k_read<KK % 3, 1, 32 * ROW>(a);
  };
  // V chunk CC of the tile at byte offset vst into fragment buffer CC & 1
  auto read_v = [&](uint32_t vst, auto cc_tag) {
    constexpr int CC = decltype(cc_tag)::value;
    if constexpr (VCOL) {
      vcol_read<CC & 1, 0, 0 * 32 * 128>(vaddr[CC] + vst);
      vcol_read<CC & 1, 1, 1 * 32 * 128>(vaddr[CC] + vst);
      vcol_read<CC & 1, 2, 2 * 32 * 128>(vaddr[CC] + vst);
      vcol_read<CC & 1, 3, 3 * 32 * 128>(vaddr[CC] + vst);
    } else {
      constexpr int OFF = CC * 16 * ROW;
      v_read<CC & 1, 0, OFF, 4 * ROW>(vaddr[0] + vst);
      v_read<CC & 1, 1, OFF, 4 * ROW>(vaddr[1] + vst);
      v_read<CC & 1, 2, OFF, 4 * ROW>(vaddr[2] + vst);
      v_read<CC & 1, 3, OFF, 4 * ROW>(vaddr[3] + vst);
    }
  };
  // LDS operations one V chunk's reads add to the counter
  constexpr int VREADS = VCOL ? DB : 2 * DB;

  // ---------------------------------------------------------------- softmax state
  const float c = p.scale_log2;
  // per query block: running max (scale*log2e units), this lane half's share
  // of the running sum over the fp32 probabilities, and the exponent offset
  // of the current tile
  float m_run[QB], l_run[QB], msub[QB];
  auto softmax_init = [&]() {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      m_run[qb] = NEG_INF;
      l_run[qb] = 0.f;
      msub[qb] = 0.f;
    }
  };

  // mask: element i of s[qb][bb] is key j0 + 32 bb + 16 (i/8) + 8 h + i%8 for
  // query qw + 32 qb + l32
  auto mask = [&](int t, f32x16(&sn)[QB][NB]) {
    const int j0 = t * BN;
    if (t >= t_edge) {
      // (an opaque statement keeps this rare block a branch instead of
      // selects executed on every tile)
      asm volatile("" ::: "memory");
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int qi = qw + 32 * qb + l32;
#pragma unroll
        for (int bb = 0; bb < NB; ++bb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = j0 + 32 * bb + 16 * (i >> 3) + 8 * h + (i & 7);
            const bool dead = (key >= kv_len) || (CAUSAL && key > qi);
            sn[qb][bb][i] = dead ? NEG_INF : sn[qb][bb][i];
          }
      }
    }
  };
  // first tile: row max of block qb in four parts of 8 elements, then across
  // the lane halves, and the running max set from it
  float mxp[QB];
  auto max_part = [&](f32x16(&sn)[QB][NB], int qb, int part) {
    if (part == 0) mxp[qb] = NEG_INF;
#pragma unroll
    for (int k = 0; k < 8; ++k) mxp[qb] = fmaxf(mxp[qb], sn[qb][part >> 1][8 * (part & 1) + k]);
    keep(mxp[qb]);
  };
  auto finish_max = [&](int qb) {
    const float mx = fmaxf(mxp[qb], wave_half_swap(mxp[qb]));
    m_run[qb] = mx * c;
    msub[qb] = (m_run[qb] == NEG_INF) ? 0.f : m_run[qb];
    keep(msub[qb]);
  };
  // exp2(c s - m) of element e of chunk (qb, cc), added to the row sum and
  // written into the P fragment (qb, cc) one step later (reading a
  // transcendental result in the next instruction costs a wait state)
  struct Pend {
    float x;
    int qb, cc, e;
    bool valid;
  };
  auto commit = [&](Pend& pd, float(&rs)[QB], vec8(&pc)[QB][NC]) {
    if (pd.valid) {
      rs[pd.qb] += pd.x;
      pc[pd.qb][pd.cc][pd.e] = (T)pd.x;
      keep(rs[pd.qb]);
      if (pd.e == 7) keep_vec(pc[pd.qb][pd.cc]);
      pd.valid = false;
    }
  };
  auto ex1 = [&](Pend& pd, f32x16(&sc)[QB][NB], int qb, int cc, int e, float(&rs)[QB], vec8(&pc)[QB][NC]) {
    const float x = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[qb][cc >> 1][8 * (cc & 1) + e], c, -msub[qb]));
    keep(x);
    commit(pd, rs, pc);
    pd = Pend{x, qb, cc, e, true};
  };

  // Round r precedes iteration r, which reads K_r and V_{r-1}; the round's
  // copies go out one per k-step of the iteration's first stretch.  Without
  // BAR2: every round waits for the copies of round r-STAGES+1 and older
  // (every round issues the same 2 LOADS copies, so STAGES-2 rounds stay in
  // flight) and barriers, then copies K_{r+STAGES-1} into the slot of
  // K_{r-1} and V_{r+STAGES-2} into the slot of V_{r-2}.
#ifndef ATTN_WIDE_BAR2
#define ATTN_WIDE_BAR2 1
#endif
  // BAR2: one barrier per two iterations.  Iteration r copies K_{r+2} and
  // V_{r+1}; the barrier of an even iteration r waits for all of the wave's
  // copies (K_r, K_{r+1}, V_{r-1}, V_r), and every slot written until the
  // next barrier (those of K_{r-2}, K_{r-1}, V_{r-3}, V_{r-2}) was last read
  // before this one.
  constexpr bool BAR2 = ATTN_WIDE_BAR2;
  constexpr int KLA = BAR2 ? 2 : STAGES - 1;   // K tile copied by round r: r + KLA
  constexpr int VLA = BAR2 ? 1 : STAGES - 2;   // V tile copied by round r: r + VLA
  auto top_wait = [&]() {
    if constexpr (BAR2) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * LOADS * (STAGES - 2)) : "memory");
  };
  auto round_copy = [&](const Copy& kc, const Copy& vc, int i) {
    if (i < LOADS) copy_row_to_lds(kc.src, kc.bytes, kc.dst + i * 1024, kdma[i]);
    else copy_row_to_lds(vc.src, vc.bytes, vc.dst + (i - LOADS) * 1024, vdma[i - LOADS]);
  };
  auto top = [&](int r) {
    if (!BAR2 || (r & 1) == 0) top_wait();
    issue_copy(next_copy(ks_k, 0), kdma);
    issue_copy(next_copy(ks_v, STAGES), vdma);
  };

  // One iteration.  HS: S_t is computed (t < n_w); HP: tile
  // t-1 is finished and P_{t-1} V_{t-1} added (t >= 1).  s_cur / p_cur
  // receive tile t, s_prev / p_prev hold tile t-1.
  float rs_a[QB] = {0.f, 0.f};     // sums of P_{t-1} computed in A
  float rs_pend[QB] = {0.f, 0.f};  // sums of the tile's first NBX groups, computed in the previous B
  // Tile t-1 is complete (all its probabilities taken against msub): l takes
  // its sum, unless some lane's share exceeds PMAX (or is not finite).  Then
  // the running max moves to the tile's row max, O and l are rescaled, and
  // the tile's probabilities and sum are recomputed.
  auto check = [&](f32x16(&sp)[QB][NB], vec8(&pp)[QB][NC]) {
    float part[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) part[qb] = rs_pend[qb] + rs_a[qb];
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(!(part[0] <= PMAX) || !(part[1] <= PMAX)) != 0, 0)) {
      asm volatile("" ::: "memory");
      float a[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float mx = NEG_INF;
#pragma unroll
        for (int bb = 0; bb < NB; ++bb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sp[qb][bb][i]);
        mx = fmaxf(mx, wave_half_swap(mx));
        const float m_new = fmaxf(m_run[qb], mx * c);
        a[qb] = (m_new == m_run[qb]) ? 1.f : __builtin_amdgcn_exp2f(m_run[qb] - m_new);
        l_run[qb] *= a[qb];
        m_run[qb] = m_new;
        msub[qb] = (m_new == NEG_INF) ? 0.f : m_new;
        float sum = 0.f;
#pragma unroll
        for (int cc = 0; cc < NC; ++cc)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float x = __builtin_amdgcn_exp2f(__builtin_fmaf(sp[qb][cc >> 1][8 * (cc & 1) + e], c, -msub[qb]));
            pp[qb][cc][e] = (T)x;
            sum += x;
          }
        part[qb] = sum;
      }
      acc_scale<0, 0>(a[0]);
      acc_scale<0, 1>(a[0]);
      acc_scale<0, 2>(a[0]);
      acc_scale<0, 3>(a[0]);
      acc_scale<1, 0>(a[1]);
      acc_scale<1, 1>(a[1]);
      acc_scale<1, 2>(a[1]);
      acc_scale<1, 3>(a[1]);
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) l_run[qb] += part[qb];
  };
  auto iter = [&](int t, auto hs_tag, auto hp_tag, f32x16(&s_cur)[QB][NB],
                  f32x16(&s_prev)[QB][NB], vec8(&p_cur)[QB][NC], vec8(&p_prev)[QB][NC]) {
    constexpr bool HS = decltype(hs_tag)::value;
    constexpr bool HP = decltype(hp_tag)::value;
    // with S_t to compute, the round's copies go one per k-step of A
    Copy kc{}, vc{};
    if constexpr (HS) {
      if (!BAR2 || (t & 1) == 0) top_wait();
      kc = next_copy(ks_k, 0);         // K_{t+KLA}
      vc = next_copy(ks_v, STAGES);    // V_{t+VLA}
    } else {
      top(t);
      // this tile's last S is done: the Q registers can take the next tile's
      // rows, which then arrive behind this last P V and the epilogue
      if constexpr (H4) {
        if (next_pt < ntl) {
          q_issue_tile(next_pt);
          q_early = true;
        }
      }
    }
    const uint32_t kst = (uint32_t)(slot_of(t) * TILE);       // K_t
    const uint32_t vst = (uint32_t)(slot_of(t - 1) * TILE);   // V_{t-1}
    rs_a[0] = rs_a[1] = 0.f;
    float rs_b[QB] = {0.f, 0.f};

    // exponentials of S_{t-1} done in A: groups NBX .. 7
    Pend pa{0.f, 0, 0, 0, false}, pb{0.f, 0, 0, 0, false};
    auto ex_a = [&](int i) {
      const int g = NBX + (i >> 3);
      ex1(pa, s_prev, g & 1, g >> 1, i & 7, rs_a, p_prev);
    };
    // exponentials of S_t done in B: groups 0 .. NBX-1
    auto ex_b = [&](int i) {
      const int g = i >> 3;
      ex1(pb, s_cur, g & 1, g >> 1, i & 7, rs_b, p_cur);
    };
    // A's exponentials after MFMA j of k-step KK
    auto ex_a_after = [&](int kk, int j) {
#pragma unroll
      for (int i = EA * kk + (EA * j) / 4; i < EA * kk + (EA * (j + 1)) / 4; ++i) ex_a(i);
    };

    // ---- A: S_t = K_t Q^T, EA exponentials of S_{t-1} per k-step
    if constexpr (HS) {
      read_k(kst, ic<0>{});
      read_k(kst, ic<1>{});
      auto kstep = [&](auto kk_tag) {
        constexpr int KK = decltype(kk_tag)::value;
        constexpr int R = KK % 3;
        constexpr bool F = KK == 0;
        round_copy(kc, vc, KK);
        if constexpr (KK + 2 < KT) read_k(kst, ic<KK + 2>{});
        if constexpr (HP && KK == KT - 2) read_v(vst, ic<0>{});
        // LDS reads issued after k-step KK: up to two k-steps, and V chunk 0
        constexpr int LEFT = 2 * ((KK + 2 < KT ? KK + 2 : KT - 1) - KK) + ((HP && KK >= KT - 2) ? VREADS : 0);
        lgkm_wait<LEFT>();
        // MFMA (bb, qb), each with its share of the exponentials after it
        // (the scheduling barriers keep each group behind its MFMA)
        mfma_s<T, F, R, 0, 0, KK>(s_cur[0][0]);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (HP) ex_a_after(KK, 0);
        __builtin_amdgcn_sched_barrier(0);
        mfma_s<T, F, R, 0, 1, KK>(s_cur[1][0]);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (HP) ex_a_after(KK, 1);
        __builtin_amdgcn_sched_barrier(0);
        mfma_s<T, F, R, 1, 0, KK>(s_cur[0][1]);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (HP) ex_a_after(KK, 2);
        __builtin_amdgcn_sched_barrier(0);
        mfma_s<T, F, R, 1, 1, KK>(s_cur[1][1]);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (HP) ex_a_after(KK, 3);
        if constexpr (HP && KK == KT - 1) commit(pa, rs_a, p_prev);
        __builtin_amdgcn_sched_barrier(0);
      };
      kstep(ic<0>{});
      kstep(ic<1>{});
      kstep(ic<2>{});
      kstep(ic<3>{});
      kstep(ic<4>{});
      kstep(ic<5>{});
      kstep(ic<6>{});
      kstep(ic<7>{});
    } else if constexpr (HP) {
      read_v(vst, ic<0>{});
#pragma unroll
      for (int i = 0; i < 8 * EA; ++i) ex_a(i);
      commit(pa, rs_a, p_prev);
    }

    if constexpr (HP) check(s_prev, p_prev);

    // ---- B: P_{t-1} V_{t-1}; mask and exp2 of chunk 0 of S_t
    // vector work of slot j of chunk CC (after the chunk's j-th MFMA)
    auto slot = [&](auto cc_tag, auto j_tag) {
      constexpr int CC = decltype(cc_tag)::value;
      constexpr int J = decltype(j_tag)::value;
      if constexpr (HS) {
        if constexpr (CC == 1 && !HP) {
          if constexpr (J == 0) { max_part(s_cur, 0, 0); max_part(s_cur, 0, 1); }
          if constexpr (J == 1) { max_part(s_cur, 0, 2); max_part(s_cur, 0, 3); }
          if constexpr (J == 2) finish_max(0);
          if constexpr (J == 3) { max_part(s_cur, 1, 0); max_part(s_cur, 1, 1); }
          if constexpr (J == 4) { max_part(s_cur, 1, 2); max_part(s_cur, 1, 3); }
          if constexpr (J == 5) finish_max(1);
        }
        if constexpr (HP && CC >= 1) {
          // slot k = 8 (CC - 1) + J of 24 takes B's exponentials [lo, hi)
          constexpr int K = 8 * (CC - 1) + J;
#pragma unroll
          for (int i = (8 * NBX * K) / 24; i < (8 * NBX * (K + 1)) / 24; ++i) ex_b(i);
        }
        if constexpr (CC == 3 && J == 7) commit(pb, rs_b, p_cur);
      }
    };
    if constexpr (HP) {
      auto chunk = [&](auto cc_tag) {
        constexpr int CC = decltype(cc_tag)::value;
        constexpr int C = CC & 1;
        if constexpr (CC + 1 < NC) {
          read_v(vst, ic<CC + 1>{});
          lgkm_wait<VREADS>();
        } else {
          lgkm_wait<0>();
        }
        auto after = [&](auto j_tag) {
          __builtin_amdgcn_sched_barrier(0);
          slot(cc_tag, j_tag);
          __builtin_amdgcn_sched_barrier(0);
        };
        mfma_o<T, 0, 0, C>(p_prev[0][CC]);
        after(ic<0>{});
        mfma_o<T, 1, 0, C>(p_prev[1][CC]);
        after(ic<1>{});
        mfma_o<T, 0, 1, C>(p_prev[0][CC]);
        after(ic<2>{});
        mfma_o<T, 1, 1, C>(p_prev[1][CC]);
        after(ic<3>{});
        mfma_o<T, 0, 2, C>(p_prev[0][CC]);
        after(ic<4>{});
        mfma_o<T, 1, 2, C>(p_prev[1][CC]);
        after(ic<5>{});
        mfma_o<T, 0, 3, C>(p_prev[0][CC]);
        after(ic<6>{});
        mfma_o<T, 1, 3, C>(p_prev[1][CC]);
        after(ic<7>{});
        // S_t may be read after these eight MFMA issues; mask it (rare)
        if constexpr (HS && CC == 0) {
          tie_s(s_cur);
          mask(t, s_cur);
        }
      };
      chunk(ic<0>{});
      chunk(ic<1>{});
      chunk(ic<2>{});
      chunk(ic<3>{});
    } else if constexpr (HS) {
      pad_s(s_cur);
      mask(t, s_cur);
      slot(ic<1>{}, ic<0>{});
      slot(ic<1>{}, ic<1>{});
      slot(ic<1>{}, ic<2>{});
      slot(ic<1>{}, ic<3>{});
      slot(ic<1>{}, ic<4>{});
      slot(ic<1>{}, ic<5>{});
#pragma unroll
      for (int i = 0; i < 8 * NBX; ++i) ex_b(i);
      commit(pb, rs_b, p_cur);
    }
    rs_pend[0] = rs_b[0];
    rs_pend[1] = rs_b[1];
  };

  // ---------------------------------------------------------------- key loop
  // Iterations 0 .. n_w: S_t (t < n_w) and P_{t-1} V_{t-1} (t >= 1).  Even
  // iterations keep tile t in s0 / p0, odd ones in s1 / p1.
  // prologue rounds -KLA .. -1: K_0 .. K_{KLA-1} and V_{VLA-KLA} .. V_{VLA-1}
  // (a V tile before the first is an empty copy, so that every round issues
  // the same number of copies)
  auto prologue = [&]() {
#pragma unroll
    for (int r = -KLA; r < 0; ++r) {
      issue_copy(next_copy(ks_k, 0), kdma);
      if (r + VLA >= 0) issue_copy(next_copy(ks_v, STAGES), vdma);
      else issue_copy(Copy{Kp, 0u, smem + (STAGES + slot_of(r + VLA)) * TILE + wave * LOADS * 1024}, vdma);
    }
  };

  // ---------------------------------------------------------------- epilogue
  // O / l and the LSE of a finished tile.  With several tiles per workgroup
  // it runs after the next tile's first iteration (which leaves O alone),
  // once that tile's loads are in flight; what it needs of the finished tile
  // is kept in the e_ values.
  float e_inv[QB], e_lse[QB];
  int e_qw = 0;
  T* e_op = nullptr;
  long long e_lse_off = 0;
  auto epi_save = [&]() {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float l_tot = l_run[qb] + wave_half_swap(l_run[qb]);
      e_inv[qb] = l_tot > 0.f ? 1.f / l_tot : 0.f;
      e_lse[qb] = l_tot > 0.f ? (m_run[qb] + log2f(l_tot)) * 0.69314718055994530942f : NEG_INF;
    }
    e_qw = qw;
    e_op = Op;
    e_lse_off = lse_off;
  };
  auto store = [&](auto qb_tag, const f32x16 (&ob)[DB]) {
    constexpr int QBI = decltype(qb_tag)::value;
    const int qi = e_qw + 32 * QBI + l32;
    if (qi < q_len) {
      T* orow = e_op + (long long)qi * qs;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          typedef T T4 __attribute__((ext_vector_type(4)));
          T4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = (T)(ob[db][4 * g + e] * e_inv[QBI]);
          *(T4*)(orow + 32 * db + 8 * g + 4 * h) = w;
        }
      if (p.lse != nullptr && h == 0) p.lse[e_lse_off + qi] = e_lse[QBI];
    }
  };
  auto epi_store = [&]() {
    acc_read_pad();
    {
      const f32x16 ob[DB] = {acc_read<0, 0>(), acc_read<0, 1>(), acc_read<0, 2>(), acc_read<0, 3>()};
      store(ic<0>{}, ob);
    }
    {
      const f32x16 ob[DB] = {acc_read<1, 0>(), acc_read<1, 1>(), acc_read<1, 2>(), acc_read<1, 3>()};
      store(ic<1>{}, ob);
    }
  };

  // ---------------------------------------------------------------- tiles
  f32x16 s0[QB][NB], s1[QB][NB];
  vec8 p0[QB][NC], p1[QB][NC];
  typedef std::true_type Y;
  typedef std::false_type N;
  int rr = 0;
  int pt = tile_of_round(0);
  if (pt >= ntl) return;
  tile_setup(pt);
  streams_setup();
  o_zero();
  q_issue_at(Qp, qw);
  prologue();
  bool pending = false;   // a finished tile's O still waits in the accumulators
  for (;;) {
    softmax_init();
    next_pt = tile_of_round(rr + 1);
    int t = 0;
    if (n_w > 0) {
      iter(0, Y{}, N{}, s0, s1, p0, p1);
      if (pending) {
        epi_store();
        o_zero();
        pending = false;
      }
      t = 1;
      for (; t + 2 <= n_w; t += 2) {
        iter(t, Y{}, Y{}, s1, s0, p1, p0);
        iter(t + 1, Y{}, Y{}, s0, s1, p0, p1);
      }
      // t is odd, t >= n_w - 1
      if (t < n_w) {
        iter(t, Y{}, Y{}, s1, s0, p1, p0);
        iter(t + 1, N{}, Y{}, s0, s1, p0, p1);
        t += 2;
      } else {
        iter(t, N{}, Y{}, s1, s0, p1, p0);
        t += 1;
      }
    }
    if (pending) {
      epi_store();
      o_zero();
      pending = false;
    }
    // idle rounds keep the barrier count equal across the waves
    const bool idle = t <= ntile;
    for (; t <= ntile; ++t) top(t);
    // no copy may still be writing LDS past this point; the next tile's Q
    // loads, issued after the last copies, may stay in flight
    if (q_early && !idle) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(QLOADS) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    epi_save();
    pending = true;
    pt = tile_of_round(++rr);
    if (pt >= ntl) break;
    // every wave is past its last LDS read of this tile before the next
    // tile's copies go out; the Q registers are free (its last S is done)
    asm volatile("s_barrier" ::: "memory");
    tile_setup(pt);
    streams_setup();
    if (!q_early) q_issue_at(Qp, qw);
    q_early = false;
    prologue();
  }
  epi_store();
}

// Compute units of the current device (read once per device).
static int device_cus() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = -1;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n > 0 ? n : 0;
}

template <typename T, bool CAUSAL, bool H4, bool VCOL>
static hipError_t launch_wide_one(const FwdParams& p, hipStream_t s) {
  constexpr int lds = 2 * ATTN_WIDE_STAGES * 64 * 128 * 2;   // K and V rings of 16 KiB tiles
  static const hipError_t attr = hipFuncSetAttribute((const void*)fwd_wide_kernel<T, CAUSAL, H4, VCOL>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((fwd_wide_kernel<T, CAUSAL, H4, VCOL>), dim3(p.grid), dim3(256), lds, s, p);
  return hipGetLastError();
}

#ifndef ATTN_WIDE_HEADS4
#define ATTN_WIDE_HEADS4 1
#endif

template <typename T, bool VCOL>
static hipError_t launch_wide_t(const FwdParams& p, int causal, hipStream_t s) {
  if (ATTN_WIDE_HEADS4 && p.group % 4 == 0) {
    // four query heads of one KV head per workgroup, 64 rows each
    FwdParams q = p;
    q.tm = make_tile_map(p.B, p.Hq / 4, p.Hkv, p.Sq, 64, causal);
    // persistent when there are more tiles than CUs: one workgroup per CU,
    // the same number on every XCD
    const int cus = device_cus() / kNumXcd * kNumXcd;
    q.grid = (cus > 0 && q.tm.ntiles > cus) ? cus : q.tm.ntiles;
    return causal ? launch_wide_one<T, true, true, VCOL>(q, s) : launch_wide_one<T, false, true, VCOL>(q, s);
  }
  return causal ? launch_wide_one<T, true, false, VCOL>(p, s) : launch_wide_one<T, false, false, VCOL>(p, s);
}

// p.feat: 0, or kFeatVCol (column-major V); the tile map is the dense one of
// 256-row blocks (or the head-packed one, chosen here)
hipError_t launch_fwd_wide(const FwdParams& p, int dtype, int causal, hipStream_t s) {
  const bool vcol = (p.feat & kFeatVCol) != 0;
  if (dtype == 0) return vcol ? launch_wide_t<__bf16, true>(p, causal, s) : launch_wide_t<__bf16, false>(p, causal, s);
  return vcol ? launch_wide_t<_Float16, true>(p, causal, s) : launch_wide_t<_Float16, false>(p, causal, s);
}

}  // namespace attn
