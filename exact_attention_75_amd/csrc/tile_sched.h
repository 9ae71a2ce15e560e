// tile_sched.h -- placement of (batch, query head, query block) tiles on
// workgroups for the attention forward kernels.  Host and device share this
// arithmetic: the kernel decodes its tile from blockIdx.x with it, and the
// host exports it (attn_tile_of) for inspection and tests.
//
// The unit of work is one query block of one (batch, head): the query block
// is an independent workgroup task as in FlashAttention-2 (Hopper tag page,
// l1-ca0.github.io, contents entries 3.4.2 and 4.1).  Two orderings are
// layered on it:
//
//  * Longest first for causal masks.  Query block m of a causal head attends
//    to (m + 1) key blocks, so late blocks carry the most work.  Dispatching
//    them first is the longest-processing-time list schedule that the
//    "flash-attention-3" article (ai.thesatyajit.com, "Five schedulers")
//    describes for the causal backward pass; the forward has the same
//    triangular imbalance.
//  * XCD affinity.  MI355X dispatches consecutive workgroup ids round-robin
//    over its 8 XCDs, each with a private L2.  When the number of KV groups
//    (batch x KV head) divides by 8, each XCD is given whole KV groups, so all
//    query heads that share a KV head, and all query blocks of that head,
//    stream their K/V through one L2.  Within an XCD the dispatch order is
//    query block (longest first), then KV group, then query head of the group.
//    Full attention (tiles of equal work) instead runs group-major: every
//    tile of one KV group before the next group's, so the XCD's workgroups
//    read one group's K/V at a time instead of all of its groups' (c5: 2
//    groups of 4 MiB per XCD against a 4 MB L2; HBM reads 5.4x -> 2.7x the
//    algorithmic bytes, 1.3 % faster).  Causal launches keep the query-block
//    order: there the longest-first balance is worth more than the L2
//    (group-major measured 0.3-0.6 % slower on the 8K causal shapes).
#pragma once

#ifdef __HIPCC__
#define ATTN_HD __host__ __device__
#else
#define ATTN_HD
#endif

namespace attn {

constexpr int kNumXcd = 8;

struct TileMap {
  int B, Hq, Hkv, group;  // group = Hq / Hkv
  int nM;                 // query blocks per (batch, head)
  int causal;
  int ntiles;             // B * Hq * nM
  int xcd;                // 1 when KV groups split evenly over the XCDs
  int gpx;                // KV groups per XCD when xcd == 1
  int gmaj;               // 1: group-major order within an XCD (needs xcd)
};

ATTN_HD inline TileMap make_tile_map(int B, int Hq, int Hkv, int Sq, int block_m, int causal) {
  TileMap t;
  t.B = B;
  t.Hq = Hq;
  t.Hkv = Hkv;
  t.group = Hq / Hkv;
  t.nM = (Sq + block_m - 1) / block_m;
  t.causal = causal ? 1 : 0;
  t.ntiles = B * Hq * t.nM;
  const int G = B * Hkv;
  t.xcd = (G % kNumXcd == 0) ? 1 : 0;
  t.gpx = t.xcd ? G / kNumXcd : 0;
  t.gmaj = (t.xcd && !causal) ? 1 : 0;
  return t;
}

// Workgroup index p in [0, ntiles) -> (batch b, query head hq, query block m).
// A bijection for every TileMap.
ATTN_HD inline void tile_decode(const TileMap& t, int p, int& b, int& hq, int& m) {
  int m_rev, g, hg;
  if (t.xcd && t.gmaj) {
    const int x = p % kNumXcd, slot = p / kNumXcd;
    const int per_g = t.nM * t.group;     // tiles of one KV group
    const int gl = slot / per_g;
    const int r = slot - gl * per_g;
    g = x * t.gpx + gl;
    m_rev = r / t.group;
    hg = r % t.group;
  } else if (t.xcd) {
    const int x = p % kNumXcd, slot = p / kNumXcd;
    const int per_row = t.gpx * t.group;  // tiles of one query-block row in one XCD
    m_rev = slot / per_row;
    const int r = slot - m_rev * per_row;
    g = x * t.gpx + r / t.group;
    hg = r % t.group;
  } else {
    const int per_row = t.B * t.Hq;
    m_rev = p / per_row;
    const int r = p - m_rev * per_row;
    g = r / t.group;
    hg = r % t.group;
  }
  m = t.causal ? t.nM - 1 - m_rev : m_rev;
  b = g / t.Hkv;
  hq = (g % t.Hkv) * t.group + hg;
}

}  // namespace attn
