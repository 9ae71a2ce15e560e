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
//    FMA, and a lazy running max without a per-tile row max: the first tile
//    takes the exact max, later probabilities are taken against it and their
//    sum is checked against a bound before they enter the second GEMM; only
//    when a sum exceeds it does the max move (and O, l get rescaled).  Exact
//    arithmetic: any reference point cancels in O = sum P V / sum P.
//  * Causal: a wave skips key tiles entirely above its diagonal; only tiles
//    that cross the diagonal or the sequence end are masked (the pages' split
//    loop, Hopper tag page contents 4.7).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include <utility>

#include "kernel_common.h"
#include "kernels.h"

namespace attn {

// NW waves per workgroup, each owning 32 query rows.  NW == 4: two
// workgroups share a CU and their waves interleave freely.  NW == 8: one
// workgroup per CU, two waves per SIMD (wave w and w + 4), run as two groups
// offset by half a tile (ping-pong, below).
// SPLIT: the key axis is cut into p.splits ranges of p.split_keys keys and
// workgroup split * ntiles + tile writes the fp32 partial result of its range
// to p.o_part / p.lse_part (flash-decoding; merged by combine_kernel).  The
// split index is the slow one, so the tile order within a split -- and its
// placement of K/V groups on XCDs -- is the plain forward's.
// PACK (PackGQA, dense only): a tile holds the query rows of all p.group
// query heads that share one KV head, row r = position * group + head in the
// group, so that few query positions (decoding) still fill the tile and K/V
// are fetched once for the group.  The tile map then runs over KV heads.
// FEAT (dense, not split or packed; bit flags):
//   kFeatSoftcap  scores capped as cap tanh(scale s / cap) before the mask
//                 (attention softcapping, "FlashAttention-3 Deep Dive" API
//                 surface); applied where each score tile is masked;
//   kFeatVCol     V given column-major, [B, Hkv, D, Sk] (key index
//                 innermost: the V_colmajor input, same page, FP8 layout
//                 discussion): the PV operand is then a plain 16-byte read
//                 of a V^T tile instead of a transposing read.
// Waves per SIMD the register budget is set for: two, except for the causal
// varlen d = 64 instance with 4 waves, whose 167 registers fit three (three
// 4-wave workgroups per CU, 96 KiB of LDS): more waves resident over ragged
// batches whose blocks vary in length.  The other d = 64 instances spill at
// that budget.
constexpr int fwd_waves_per_simd(int D, int NW, bool CAUSAL, bool VARLEN) {
  return (NW == 4 && D == 64 && CAUSAL && VARLEN) ? 3 : 2;
}

template <typename T, int D, int BN, int NW, bool CAUSAL, bool VARLEN, bool SPLIT, bool PACK, int FEAT>
__global__ void __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(fwd_waves_per_simd(D, NW, CAUSAL, VARLEN), fwd_waves_per_simd(D, NW, CAUSAL, VARLEN))))
fwd_kernel(FwdParams p) {
  typedef typename Mma<T>::vec8 vec8;
  constexpr int NTHREADS = 64 * NW;
  constexpr int BM = 32 * NW;
  constexpr int CPR = D / 8;           // 16-byte chunks per row
  constexpr int KT = D / 16;           // k-steps of the first GEMM
  constexpr int NB = BN / 32;          // 32-key blocks per tile
  constexpr int NC = BN / 16;          // 16-key chunks per tile (second GEMM)
  constexpr int DB = D / 32;           // 32-column blocks of O^T
  constexpr int ROW = D * 2;           // bytes per K/V row in LDS
  constexpr int TILE = BN * ROW;       // bytes per K or V tile
  // K/V buffers per tensor: three when one 8-wave workgroup has the CU's LDS
  // to itself (copies run two tiles ahead), two otherwise
  constexpr int STAGES = (NW == 8) ? 3 : 2;
  constexpr int LOADS = BN * CPR / (NW * 64);   // DMA instructions per wave per tile
  constexpr float NEG_INF = -__builtin_inff();
  static_assert(BN == 64 && (BN * CPR) % (NW * 64) == 0, "tile shape");
  static_assert(!(PACK && VARLEN), "PackGQA is for dense inputs");
  constexpr bool SOFTCAP = (FEAT & kFeatSoftcap) != 0;
  constexpr bool VCOL = (FEAT & kFeatVCol) != 0;
  static_assert(!VCOL || (!VARLEN && !SPLIT && !PACK), "column-major V: dense, plain tiles");

  // With d = 128 the Q block lives in LDS (its 32 registers per lane are
  // needed by the pipeline); with d = 64 it stays in registers.
  constexpr bool QLDS = (D == 128);
  // d = 128 with 4 waves: one K buffer instead of two (80 KiB of LDS in all,
  // so two workgroups share a CU): the next K tile is copied once every wave
  // has finished stretch A of the current one, behind a second barrier.
  constexpr bool KSINGLE = QLDS && NW == 4;
  constexpr int KST = KSINGLE ? 1 : STAGES;   // K buffers
  // [K buffers | V stages | Q block (QLDS)]
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* const qsm = smem + (KST + STAGES) * TILE;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
  const int h = lane >> 5;
  const int l32 = lane & 31;
  // Query row (within the wave's 32) of this lane's MFMA column.  Columns may
  // be assigned to queries in any fixed order; using the same permutation as
  // the key rows lets Q and K share their LDS read offsets.
  const int qlane = key_perm(l32);

  // ---------------------------------------------------------------- tile decode
  int b, hq, mblk, q_len, kv_len;
  long long q_off, kv_off;   // element offsets of token 0 of this (batch | sequence)
  long long lse_off;         // index of this head's token 0 in lse
  if (VARLEN) {
    const int pid = blockIdx.x;
    hq = pid % p.Hq;
    int r = pid / p.Hq;        // rank of the workgroup's (sequence, block) entry
    int s = -1, start = 0, len = 0;
    // longest blocks first over the whole batch (the grid's tail then holds
    // the short ones); the level is the query block's index
    VarlenEntry ve;
    const bool ranked = varlen_rank<BM, CAUSAL>(p.cu_seqlens, p.B, r, ve);
    if (ranked && ve.seq >= 0) {
      s = ve.seq;
      mblk = ve.level;
      start = ve.start;
      len = ve.len;
    }
    if (!ranked) {
      // many sequences, or one of more than 64 blocks: the batch's order,
      // longest block of each sequence first
      int nb = 0;
      for (s = 0; s < p.B; ++s) {
        start = p.cu_seqlens[s];
        len = p.cu_seqlens[s + 1] - start;
        nb = (len + BM - 1) / BM;
        if (r < nb) break;
        r -= nb;
      }
      if (s >= p.B) s = -1;
      mblk = nb - 1 - r;
    }
    if (s < 0) return;         // beyond the last block (uniform over the workgroup)
    b = 0;
    q_len = len;
    kv_len = len;
    q_off = (long long)start * p.q_tok_stride;
    kv_off = (long long)start * p.kv_tok_stride;
    lse_off = (long long)hq * p.Sq + start;
  } else {
    // with PACK the map runs over KV heads: hq is the KV head here
    tile_decode(p.tm, SPLIT ? (int)(blockIdx.x % p.tm.ntiles) : (int)blockIdx.x, b, hq, mblk);
    if (PACK) hq *= p.group;   // first query head of the group
    q_len = p.Sq;
    kv_len = p.Sk;
    q_off = (long long)b * p.q_batch_stride;
    kv_off = (long long)b * p.kv_batch_stride;
    lse_off = ((long long)b * p.Hq + hq) * p.Sq;
  }
  // key range of a split: keys [key0, key0 + kv_len) of the sequence; K/V
  // are addressed from key0, causal comparisons stay in sequence positions
  const int split = SPLIT ? (int)(blockIdx.x / p.tm.ntiles) : 0;
  const int key0 = split * (SPLIT ? p.split_keys : 0);
  if constexpr (SPLIT) {
    kv_len = min(kv_len - key0, p.split_keys);
    if (kv_len < 0) kv_len = 0;
    kv_off += (long long)key0 * p.kv_tok_stride;
  }
  const int hkv = hq / p.group;
  // Query rows of the tile: row r is query position row_pos(r) of head
  // hq + (r % grp); row_off(r) its element offset from Qp / Op.
  const int grp = PACK ? p.group : 1;
  const int rows_len = q_len * grp;
  auto row_pos = [&](int r) { return PACK ? r / grp : r; };
  auto row_off = [&](int r) -> long long {
    return PACK ? (long long)(r / grp) * p.q_tok_stride + (r % grp) * D : (long long)r * p.q_tok_stride;
  };
  auto lse_idx = [&](int r) -> long long { return PACK ? lse_off + (long long)(r % grp) * p.Sq + r / grp : lse_off + r; };
  const T* Qp = (const T*)p.q + q_off + hq * D;
  const T* Kp = (const T*)p.k + kv_off + hkv * D;
  const T* Vp = (const T*)p.v + kv_off + hkv * D;
  T* Op = (T*)p.o + q_off + hq * D;
  const int qs = p.q_tok_stride;
  const int ks = p.kv_tok_stride;

  const int q0 = mblk * BM;
  const int qw = q0 + wave * 32;                       // first query row of this wave
  const int cw = row_pos(qw) - key0;                   // its causal position relative to the first key
  const int cw_hi = row_pos(qw + 31) - key0;           // and that of its last row
  const int q_hi = min(q_len, row_pos(q0 + BM - 1) + 1);   // one past the block's last position
  const int kv_end = CAUSAL ? max(0, min(kv_len, q_hi - key0)) : kv_len;
  const int ntile = (kv_end + BN - 1) / BN;

  // ---------------------------------------------------------------- Q fragment
  // B operand of S^T = K Q^T: lane holds query qlane, head-dim 16*kk + 8*h
  // .. +7.  In registers for d = 64; for d = 128 read from LDS per k-step.
  constexpr int KTR = QLDS ? 1 : KT;
  vec8 qf[KTR];
  if constexpr (!QLDS) {
    const int qrow = (qw + qlane < rows_len) ? qw + qlane : rows_len - 1;
    const T* qr = Qp + row_off(qrow) + 8 * h;
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
    if constexpr (VCOL) {
      // V^T tile: D rows (channels) of BN keys = 8 chunks of 16 bytes, chunk c
      // of row r stored at c ^ (r & 7); global rows are Sk keys apart
      const int vr = pos / 8, vc = pos % 8;
      vdma[i] = (uint32_t)(vr * p.Sk * 2 + ((vc ^ (vr & 7)) << 4));
    } else {
      vdma[i] = (uint32_t)(row * ks * 2 + ((phys ^ swz_v<D>(row)) << 4));
    }
  }
  static_assert(!VCOL || BN * 2 == 8 * 16, "V^T tile rows of 8 chunks");
  // column-major V: this (batch, KV head)'s [D, Sk] plane
  const T* Vt = VCOL ? (const T*)p.v + ((long long)b * p.Hkv + hkv) * D * p.Sk : nullptr;
  auto issue = [&](const T* src, int t, char* dst, bool is_v) {
    const int j0 = t * BN;
    if (VCOL && is_v) {
      // range to the end of the plane: keys past Sk read the next channel's
      // (finite) values, or zeros past the plane; their P is 0
      const uint32_t bytes = (uint32_t)(D * p.Sk - j0) * 2u;
      copy_rows_to_lds<LOADS>((const void*)(Vt + j0), bytes, dst + wave_u * LOADS * 1024, vdma);
      return;
    }
    const uint32_t bytes = (uint32_t)(kv_len - j0) * (uint32_t)ks * 2u;
    copy_rows_to_lds<LOADS>((const void*)(src + (long long)j0 * ks), bytes, dst + wave_u * LOADS * 1024,
                            is_v ? vdma : kdma);
  };

  if constexpr (QLDS) {
    // the workgroup's BM query rows into LDS, K-style swizzle; rows past the
    // end of the sequence read as zeros (buffer range check)
    constexpr int QLOADS = BM * CPR / (NW * 64);
    uint32_t qdma[QLOADS];
#pragma unroll
    for (int i = 0; i < QLOADS; ++i) {
      const int pos = (wave * QLOADS + i) * 64 + lane;
      const int row = pos / CPR, phys = pos % CPR;
      // (q0 is a multiple of grp, so block row `row` is row_off(row) past row q0)
      qdma[i] = (uint32_t)(row_off(row) * 2 + ((phys ^ swz_k<D>(row)) << 4));
    }
    // bytes from row q0 to the end of the last valid row
    const uint32_t bytes = PACK ? (uint32_t)((q_len - q0 / grp - 1) * qs + grp * D) * 2u
                                : (uint32_t)(q_len - q0) * (uint32_t)qs * 2u;
    copy_rows_to_lds<QLOADS>((const void*)(Qp + row_off(q0)), bytes, qsm + wave * QLOADS * 1024, qdma);
  }

  // per-lane LDS byte offsets, invariant over tiles
  const uint32_t lds0 = (uint32_t)(uintptr_t)(LDS_AS char*)smem;
  // K (and Q) rows: lane reads row qlane, 16-byte chunk 2 kk + h, stored at
  // chunk (2 kk + h) ^ swz_k(row).  The k-step bits (bit 5 up of the byte
  // offset) and the rest are disjoint fields, so offset(kk) = koff0 ^ (kk << 5);
  // block bb adds 32 rows, an immediate.
  const int koff0 = qlane * ROW + (((h) ^ swz_k<D>(qlane)) << 4);
  auto koff = [&](int kk) { return koff0 ^ (kk << 5); };
  // V rows for the transposing reads: likewise offset(db) = voff0 ^ (db << 6)
  // (the 32-channel block index sits above the in-block bits of the offset);
  // chunk cc adds 16 rows and the second read 4 rows, immediates.
  uint32_t voff0;
  {
    const int G = lane >> 4, i16 = lane & 15;
    const int r = 8 * h + (i16 >> 2);
    const int dd = 16 * (G & 1) + 4 * (i16 & 3);
    voff0 = r * ROW + ((((dd >> 3) ^ swz_v<D>(r))) << 4) + ((dd & 7) << 1);
  }
  auto voff = [&](int db) { return (voff0 ^ (uint32_t)(db << 6)) + lds0 + KST * TILE; };

  f32x16 o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) o[i] = f32x16{};
  {
    // both V stages start as zeros, so that the rows past the end of a ragged
    // tile hold zeros or earlier V data, never arbitrary bit patterns
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    i32x4* z = (i32x4*)(smem + KST * TILE);
#pragma unroll
    for (int i = tid; i < STAGES * TILE / 16; i += NTHREADS) z[i] = i32x4{};
    // every wave's zeros must land before any wave's first V copy (issued
    // ahead of the first round's barrier with three stages)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
  float m_run = NEG_INF;   // running max of scale*log2(e)*s for the lane's query (same in both halves)
  float msub = 0.f;        // m_run, or 0 while it is -inf: the exponent offset of the probabilities
  // This lane half's share of the running sum of P, taken over the fp32
  // probabilities: bf16 keeps 8 significant bits, so summing the rounded
  // values could be off by 2^-9 relative, a 2e-3 error in LSE.
  float l_run = 0.f;
  const float c = p.scale_log2;
  const int qi = qw + qlane;
  const int qpos = row_pos(qi);   // causal position of the lane's query
  const char* const qwave = qsm + wave * 32 * ROW;   // this wave's Q rows (QLDS)

  // column-major V: lane reads channel row 32 db + l32, keys 16 CC + 8 h .. + 7
  // = logical chunk 2 CC + h of the row, at (2 CC + h) ^ (l32 & 7)
  uint32_t vcol[VCOL ? 4 : 1];
  if constexpr (VCOL) {
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
      vcol[cc] = lds0 + KST * TILE + l32 * 128 + ((((2 * cc + h) ^ (l32 & 7))) << 4);
  }
  auto read_v = [&](i16x4 (&vr)[2 * DB], uint32_t vstage, auto cc_tag) {
    constexpr int CC = decltype(cc_tag)::value;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      if constexpr (VCOL) {
        vr[2 * db] = lds_rd64<0>(vcol[CC] + vstage + db * 32 * 128);
        vr[2 * db + 1] = lds_rd64<8>(vcol[CC] + vstage + db * 32 * 128);
      } else {
        const uint32_t a = voff(db) + vstage;
        vr[2 * db] = lds_tr16<CC * 16 * ROW>(a);
        vr[2 * db + 1] = lds_tr16<CC * 16 * ROW + 4 * ROW>(a);
      }
    }
  };

  // Per-wave software pipeline.  MFMA and VALU work overlap well when one
  // wave interleaves them, poorly when they come from different waves, so
  // every stretch of MFMAs below carries its share of the softmax:
  //   A: S_{t+1} = K_{t+1} Q^T (16 MFMA)   with  exp2 of S_t, chunks 0-1
  //   B: P_t V_t, chunks 0-1 (8 MFMA)      with  exp2 of S_t, chunks 2-3
  //   C: P_t V_t, chunks 2-3 (8 MFMA)
  // with the mask of S_{t+1} between A and B and the sum check of each chunk
  // pair before its MFMAs.  The probabilities go straight into the packed
  // operand P; S_t keeps the raw scores.

  // P = exp2(c s - m) for elements [e0, e0+n) of 16-key chunk cc, into the
  // second GEMM's operand pc and the sum rs; S keeps the raw scores (the
  // rare rescale below needs them)
  auto exps = [&](const f32x16 (&sc)[NB], int cc, int e0, int n, float& rs, vec8 (&pc)[NC]) {
#pragma unroll
    for (int e = e0; e < e0 + n; ++e) {
      const float x = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[cc >> 1][8 * (cc & 1) + e], c, -msub));
      keep(x);
      rs += x;
      pc[cc][e] = (T)x;
    }
    if (e0 + n == 8) keep_vec(pc[cc]);
  };
  // mask: element i of block bb is key j0 + 32*bb + 16*(i/8) + 8*h + i%8
  auto mask = [&](int t, f32x16 (&sn)[NB]) {
    if constexpr (SOFTCAP) {
      // s <- (cap / scale) tanh(s scale / cap), so that c s is log2(e) times
      // the capped score; tanh x = 1 - 2 / (e^{2x} + 1) (saturates to +-1)
#pragma unroll
      for (int bb = 0; bb < NB; ++bb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float e2 = __builtin_amdgcn_exp2f(sn[bb][i] * p.softcap_b2);
          sn[bb][i] = p.softcap_a * (1.f - 2.f * __builtin_amdgcn_rcpf(e2 + 1.f));
        }
    }
    const int j0 = t * BN;
    const bool edge = (j0 + BN > kv_len) || (CAUSAL && j0 + BN - 1 > cw);
    if (edge) {
#pragma unroll
      for (int bb = 0; bb < NB; ++bb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = j0 + 32 * bb + 16 * (i >> 3) + 8 * h + (i & 7);
          const bool dead = (key >= kv_len) || (CAUSAL && key > qpos - key0);
          sn[bb][i] = dead ? NEG_INF : sn[bb][i];
        }
    }
  };
  // Running max without a per-tile row max.  The first tile sets m to its
  // exact row max.  After that each tile's probabilities are taken against
  // the current m, and before a pair of 16-key chunks enters the second GEMM
  // each lane's share of the pair's sum is compared with PMAX: the sum bounds
  // every probability of the pair, so in the common case P <= PMAX (far
  // inside the fp32, bf16 and fp16 ranges) and nothing else is needed.  When
  // some lane exceeds it (or a sum is not finite) the wave takes a rare
  // branch: m moves to the tile's row max (its raw scores are still in
  // registers), O and l are rescaled by 2^(m_old - m_new) and the pair's
  // probabilities are recomputed.  Any reference point cancels in
  // O = sum P V / sum P, so the result is the same exact arithmetic.
  constexpr float PMAX = 16384.0f;
  auto max16 = [&](const f32x16& x, float mx) {
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, x[i]);   // chains into v_max3
    return mx;
  };
  auto first_max = [&](const f32x16 (&sc)[NB]) {
    float mx = NEG_INF;
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) mx = max16(sc[bb], mx);
    mx = fmaxf(mx, wave_half_swap(mx));
    m_run = mx * c;
    msub = (m_run == NEG_INF) ? 0.f : m_run;
  };
  // rare: move m to the row max of tile sc; returns the factor applied to O
  // and l (the caller rescales its own partial sums)
  auto move_max = [&](const f32x16 (&sc)[NB]) {
    float mx = NEG_INF;
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) mx = max16(sc[bb], mx);
    mx = fmaxf(mx, wave_half_swap(mx));
    const float m_new = fmaxf(m_run, mx * c);
    const float a = (m_new == m_run) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] *= a;
    l_run *= a;
    m_run = m_new;
    msub = (m_new == NEG_INF) ? 0.f : m_new;
    return a;
  };

  // Operand reads for k-step kk: K of both 32-key blocks, and Q when it lives
  // in LDS (same lane offsets: same row permutation and swizzle)
  auto read_k = [&](const char* Ks, int kk, vec8 (&kr)[NB], vec8& qv) {
    const int ko = koff(kk);
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) kr[bb] = *(const vec8*)(Ks + ko + bb * 32 * ROW);
    if constexpr (QLDS) qv = *(const vec8*)(qwave + ko);
    else qv = qf[kk];
  };

  // S_t = K_t Q^T with no VALU work to interleave (first tile only)
  auto s_alone = [&](int t, f32x16 (&sn)[NB]) {
    const char* Ks = smem + (t % KST) * TILE;
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) sn[bb] = f32x16{};
    vec8 kr[3][NB], qv[3];
    read_k(Ks, 0, kr[0], qv[0]);
    read_k(Ks, 1, kr[1], qv[1]);
#pragma unroll
    for (int kk = 0; kk < KT; ++kk) {
      if (kk + 2 < KT) read_k(Ks, kk + 2, kr[(kk + 2) % 3], qv[(kk + 2) % 3]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) sn[bb] = Mma<T>::run(kr[kk % 3][bb], qv[kk % 3], sn[bb]);
    }
  };

  // KSINGLE: the second barrier of round r, once every wave is past stretch
  // A (its K reads complete), then this wave's share of the copy of K_{r+1}
  // into the single K buffer.  Every wave runs it once per round, idle
  // rounds included, so the barrier counts stay equal.
  auto mid = [&](int r) {
    if constexpr (KSINGLE) {
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (r + 1 < ntile) issue(Kp, r + 1, smem, false);
    }
  };

  // One tile: P_t V_t into O, S_{t+1} (when has_next) with its max.  The
  // transposing V reads run one 16-key chunk ahead of their MFMAs (chunk 0 is
  // issued near the end of stretch A, when the K prefetch registers free up).
  auto tile = [&](int t, bool has_next, f32x16 (&sc)[NB], f32x16 (&sn)[NB]) {
    float rs01 = 0.f, rs23 = 0.f;   // lane shares of the sums of chunks 0-1 and 2-3
    vec8 pc[NC];
    const uint32_t vst = (t % STAGES) * TILE;
    i16x4 vr0[2 * DB], vr1[2 * DB], vr2[2 * DB], vr3[2 * DB];
    auto mma_chunk = [&](i16x4 (&vr)[2 * DB], int db, const vec8& p) {
      const i16x8 w = __builtin_shufflevector(vr[2 * db], vr[2 * db + 1], 0, 1, 2, 3, 4, 5, 6, 7);
      o[db] = Mma<T>::run(__builtin_bit_cast(vec8, w), p, o[db]);
    };

    // ---- A: S_{t+1} with the exp2 of chunks 0-1 of S_t
    if (has_next) {
      const char* Ks = smem + ((t + 1) % KST) * TILE;
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) sn[bb] = f32x16{};
      // K (and Q) operands two k-steps ahead of their MFMAs
      vec8 kr[3][NB], qv[3];
      read_k(Ks, 0, kr[0], qv[0]);
      read_k(Ks, 1, kr[1], qv[1]);
#pragma unroll
      for (int kk = 0; kk < KT; ++kk) {
        if (kk + 2 < KT) read_k(Ks, kk + 2, kr[(kk + 2) % 3], qv[(kk + 2) % 3]);
        if (kk == KT - 2) read_v(vr0, vst, std::integral_constant<int, 0>{});
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) sn[bb] = Mma<T>::run(kr[kk % 3][bb], qv[kk % 3], sn[bb]);
        // 16 exponentials spread over the KT k-steps
        constexpr int PER = 16 / KT;
        exps(sc, (kk * PER) / 8, (kk * PER) % 8, PER, rs01, pc);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      read_v(vr0, vst, std::integral_constant<int, 0>{});
      exps(sc, 0, 0, 8, rs01, pc);
      exps(sc, 1, 0, 8, rs01, pc);
    }
    mid(t + 1);
    // chunks 0-1 enter the second GEMM next: their sum check
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(!(rs01 <= PMAX)) != 0, 0)) {
      asm volatile("" ::: "memory");
      move_max(sc);
      rs01 = 0.f;
      exps(sc, 0, 0, 8, rs01, pc);
      exps(sc, 1, 0, 8, rs01, pc);
    }

    // S_{t+1} is complete: mask it now (rare branch, outside the stretches)
    if (has_next) mask(t + 1, sn);

    // ---- B: chunks 0-1 of P V, exp2 of chunks 2-3
    read_v(vr1, vst, std::integral_constant<int, 1>{});
    exps(sc, 2, 0, 4, rs23, pc);
    lds_wait<2 * DB>(vr0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      mma_chunk(vr0, db, pc[0]);
      exps(sc, 2, 4 + db * (4 / DB), 4 / DB, rs23, pc);
      __builtin_amdgcn_sched_barrier(0);
    }
    read_v(vr2, vst, std::integral_constant<int, 2>{});
    exps(sc, 3, 0, 4, rs23, pc);
    lds_wait<2 * DB>(vr1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      mma_chunk(vr1, db, pc[1]);
      exps(sc, 3, 4 + db * (4 / DB), 4 / DB, rs23, pc);
      __builtin_amdgcn_sched_barrier(0);
    }
    // chunks 2-3: their sum check (O already holds chunks 0-1, taken against
    // the old m: the rescale of O covers them, and of rs01 their sum)
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(!(rs23 <= PMAX)) != 0, 0)) {
      asm volatile("" ::: "memory");
      rs01 *= move_max(sc);
      rs23 = 0.f;
      exps(sc, 2, 0, 8, rs23, pc);
      exps(sc, 3, 0, 8, rs23, pc);
    }
    l_run += rs01 + rs23;

    // ---- C: chunks 2-3 of P V
    read_v(vr3, vst, std::integral_constant<int, 3>{});
    lds_wait<2 * DB>(vr2);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int db = 0; db < DB; ++db) mma_chunk(vr2, db, pc[2]);
    __builtin_amdgcn_sched_barrier(0);
    lds_wait<0>(vr3);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int db = 0; db < DB; ++db) mma_chunk(vr3, db, pc[3]);
    __builtin_amdgcn_sched_barrier(0);
  };

  // tiles this wave computes (a causal wave stops at its diagonal; a wave
  // whose rows see no key still runs one fully masked tile)
  const int n_w = CAUSAL ? min(ntile, max(cw_hi, 0) / BN + 1) : ntile;

  // Round r (r = 0 .. ntile) precedes tile r-1's work (and the first tile's
  // S).  Two stages: wait for all copies, barrier, start K_{r+1} and V_r into
  // the buffers tile r-1 used.  Three stages: wait only for the copies of
  // round r-2 and older (vmcnt counts in order; round r-1's stay in flight),
  // barrier, start K_{r+2} and V_{r+1} into the buffers tile r-2 used.
  auto kbuf = [&](int t) { return smem + (t % KST) * TILE; };
  auto vbuf = [&](int t) { return smem + (KST + t % STAGES) * TILE; };
  // Two K buffers and two V stages: round 0's copies (K_1, V_0) go out
  // together with K_0, before the first wait, so the block starts after one
  // memory round trip instead of two.
  constexpr bool PRE2 = STAGES == 2 && !KSINGLE;
  auto top = [&](int r) {
    if constexpr (STAGES == 2) {
      // (KSINGLE: K_{r+1} goes out at this round's second barrier instead)
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (!PRE2 || r > 0) {
        if (!KSINGLE && r + 1 < ntile) issue(Kp, r + 1, kbuf(r + 1), false);
        if (r < ntile) issue(Vp, r, vbuf(r), true);
      }
    } else {
      const int prev = r >= 1 ? (int)(r + 1 < ntile) + (int)(r < ntile) : 0;  // copies of round r-1
      if (prev == 2)
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * LOADS) : "memory");
      else if (prev == 1)
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(LOADS) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (r + 2 < ntile) issue(Kp, r + 2, kbuf(r + 2), false);
      if (r + 1 < ntile) issue(Vp, r + 1, vbuf(r + 1), true);
    }
  };

  issue(Kp, 0, kbuf(0), false);
  if constexpr (STAGES == 3) {
    if (1 < ntile) issue(Kp, 1, kbuf(1), false);
    issue(Vp, 0, vbuf(0), true);
  }
  if constexpr (PRE2) {
    if (1 < ntile) issue(Kp, 1, kbuf(1), false);
    if (0 < ntile) issue(Vp, 0, vbuf(0), true);
  }
  top(0);
  f32x16 sA[NB], sB[NB];
  s_alone(0, sA);
  mask(0, sA);
  first_max(sA);
  mid(0);
  int t = 0;
  for (; t + 2 < n_w; t += 2) {          // unrolled by two: the S sets swap roles
    top(t + 1);
    tile(t, true, sA, sB);
    top(t + 2);
    tile(t + 1, true, sB, sA);
  }
  if (t + 1 < n_w) {
    top(t + 1);
    tile(t, true, sA, sB);
    top(t + 2);
    tile(t + 1, false, sB, sA);
    t += 2;
  } else {
    top(t + 1);
    tile(t, false, sA, sB);
    t += 1;
  }
  for (int r = t + 1; r <= ntile; ++r) {
    top(r);
    mid(r);
  }

  // ---------------------------------------------------------------- epilogue
  const float l_tot = l_run + wave_half_swap(l_run);
  if (SPLIT && qi < rows_len) {
    // fp32 partial of this key range: O_p = sum P V / l_p, LSE_p
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const long long plane = (long long)split * p.B * p.Sq * p.Hq;
    float* orow = p.o_part + (plane * D + q_off + hq * D + row_off(qi));
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float4 w;
        w.x = o[db][4 * g] * inv;
        w.y = o[db][4 * g + 1] * inv;
        w.z = o[db][4 * g + 2] * inv;
        w.w = o[db][4 * g + 3] * inv;
        *(float4*)(orow + 32 * db + 8 * g + 4 * h) = w;
      }
    if (h == 0) {
      const float lse = l_tot > 0.f ? (m_run + log2f(l_tot)) * 0.69314718055994530942f : NEG_INF;
      p.lse_part[plane + lse_idx(qi)] = lse;
    }
  } else if (qi < rows_len) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    T* orow = Op + row_off(qi);
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
      p.lse[lse_idx(qi)] = lse;
    }
  }
}

// Dynamic LDS bytes of a forward kernel instance: K buffers (one for d = 128
// with 4 waves, else as many as V's), V stages (three with 8 waves, else two),
// plus the Q block for d = 128.
template <int D, int BN, int NW>
constexpr int fwd_lds_bytes() {
  constexpr int vst = NW == 8 ? 3 : 2;
  constexpr int kst = (D == 128 && NW == 4) ? 1 : vst;
  return (kst + vst) * BN * D * 2 + (D == 128 ? 32 * NW * D * 2 : 0);
}

template <typename T, int D, int BN, int NW, bool CAUSAL, bool VARLEN, bool SPLIT = false, bool PACK = false,
          int FEAT = 0>
static hipError_t launch_one(const FwdParams& p, hipStream_t s) {
  constexpr int lds = fwd_lds_bytes<D, BN, NW>();
  auto* kern = fwd_kernel<T, D, BN, NW, CAUSAL, VARLEN, SPLIT, PACK, FEAT>;
  static const hipError_t attr = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(kern, dim3(p.grid), dim3(64 * NW), lds, s, p);
  return hipGetLastError();
}

// Dense 4-wave (128-row) blocks, optionally split-KV and / or PackGQA
template <typename T, int D, bool SPLIT>
static hipError_t launch_dense4(const FwdParams& p, int causal, hipStream_t s) {
  if (p.pack)
    return causal ? launch_one<T, D, 64, 4, true, false, SPLIT, true>(p, s)
                  : launch_one<T, D, 64, 4, false, false, SPLIT, true>(p, s);
  return causal ? launch_one<T, D, 64, 4, true, false, SPLIT, false>(p, s)
                : launch_one<T, D, 64, 4, false, false, SPLIT, false>(p, s);
}

template <bool SPLIT>
static hipError_t launch_dense4_any(const FwdParams& p, int dtype, int d, int causal, hipStream_t s) {
  if (dtype == 0)
    return d == 128 ? launch_dense4<__bf16, 128, SPLIT>(p, causal, s) : launch_dense4<__bf16, 64, SPLIT>(p, causal, s);
  return d == 128 ? launch_dense4<_Float16, 128, SPLIT>(p, causal, s) : launch_dense4<_Float16, 64, SPLIT>(p, causal, s);
}

hipError_t launch_fwd_split(const FwdParams& p, int dtype, int d, int causal, hipStream_t s) {
  return launch_dense4_any<true>(p, dtype, d, causal, s);
}

template <typename T, int D, int BN, int NW>
static hipError_t launch_t(const FwdParams& p, int causal, int varlen, hipStream_t s) {
  if (varlen) {
    return causal ? launch_one<T, D, BN, NW, true, true>(p, s) : launch_one<T, D, BN, NW, false, true>(p, s);
  }
  return causal ? launch_one<T, D, BN, NW, true, false>(p, s) : launch_one<T, D, BN, NW, false, false>(p, s);
}

// Query rows per workgroup: 256 (8 waves, one workgroup per CU, each K/V tile
// shared by 256 queries) for dense problems, 128 (4 waves, two workgroups per
// CU) for ragged batches, where a smaller block wastes less on short
// sequences.  ATTN_BLOCK_M=128|256 overrides the choice for tuning sweeps.
int fwd_block_m(int dtype, int d, int varlen) {
  (void)dtype;
  (void)d;
  static const int forced = [] {
    const char* e = getenv("ATTN_BLOCK_M");
    const int v = e ? atoi(e) : 0;
    return (v == 128 || v == 256) ? v : 0;
  }();
  if (forced) return forced;
  return varlen ? 128 : 256;
}

// Dense d = 128 problems with 256-row blocks run the one-wave-per-SIMD
// kernel (attn_fwd_wide.hip); ATTN_KERNEL=narrow selects this file's 8-wave
// kernel instead, for comparisons.
static bool use_wide() {
  static const bool wide = [] {
    const char* e = getenv("ATTN_KERNEL");
    return !(e && e[0] == 'n');
  }();
  return wide;
}

// Softcap (with or without column-major V), and column-major V at d = 64:
// dense 4-wave (128-row) blocks
template <typename T, int D, int FEAT>
static hipError_t launch_feat_t(const FwdParams& p, int causal, hipStream_t s) {
  return causal ? launch_one<T, D, 64, 4, true, false, false, false, FEAT>(p, s)
                : launch_one<T, D, 64, 4, false, false, false, false, FEAT>(p, s);
}
template <typename T, int D>
static hipError_t launch_feat_d(const FwdParams& p, int causal, hipStream_t s) {
  switch (p.feat) {
    case kFeatSoftcap: return launch_feat_t<T, D, kFeatSoftcap>(p, causal, s);
    case kFeatVCol: return launch_feat_t<T, D, kFeatVCol>(p, causal, s);
    default: return launch_feat_t<T, D, kFeatSoftcap | kFeatVCol>(p, causal, s);
  }
}

hipError_t launch_fwd(const FwdParams& p, int dtype, int d, int causal, int varlen, hipStream_t s) {
  if (p.feat == kFeatVCol && d == 128 && !varlen && use_wide()) {
    // column-major V alone: the one-wave-per-SIMD kernel, on its 256-row tiles
    FwdParams q = p;
    q.tm = make_tile_map(p.B, p.Hq, p.Hkv, p.Sq, 256, causal);
    q.grid = q.tm.ntiles;
    return launch_fwd_wide(q, dtype, causal, s);
  }
  if (p.feat != 0) {
    if (dtype == 0) return d == 128 ? launch_feat_d<__bf16, 128>(p, causal, s) : launch_feat_d<__bf16, 64>(p, causal, s);
    return d == 128 ? launch_feat_d<_Float16, 128>(p, causal, s) : launch_feat_d<_Float16, 64>(p, causal, s);
  }
  if (p.pack && !varlen) return launch_dense4_any<false>(p, dtype, d, causal, s);
  const int bm = fwd_block_m(dtype, d, varlen);
  if (bm == 256 && d == 128 && !varlen && use_wide()) return launch_fwd_wide(p, dtype, causal, s);
  if (bm == 256) {
    if (dtype == 0)
      return d == 128 ? launch_t<__bf16, 128, 64, 8>(p, causal, varlen, s)
                      : launch_t<__bf16, 64, 64, 8>(p, causal, varlen, s);
    return d == 128 ? launch_t<_Float16, 128, 64, 8>(p, causal, varlen, s)
                    : launch_t<_Float16, 64, 64, 8>(p, causal, varlen, s);
  }
  if (dtype == 0)
    return d == 128 ? launch_t<__bf16, 128, 64, 4>(p, causal, varlen, s)
                    : launch_t<__bf16, 64, 64, 4>(p, causal, varlen, s);
  return d == 128 ? launch_t<_Float16, 128, 64, 4>(p, causal, varlen, s)
                  : launch_t<_Float16, 64, 64, 4>(p, causal, varlen, s);
}

}  // namespace attn
