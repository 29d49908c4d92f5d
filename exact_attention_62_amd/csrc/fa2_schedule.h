// Work schedules of the gfx950 kernels as plain integer functions, compiled
// both into the kernels (device) and into the library's host-side schedule
// queries, so that a CPU test checks exactly the code the kernels run.
//
// Forward pass (the pages' grid of one thread block per (query block, batch,
// head): page "FlashAttention学习笔记(2)", section "V2中的thread blocks排布";
// page "Flash Attention V2原理解读", the thread-block grid section).  The work
// items are the (query block, batch*head[, key/value split]) triples.  The
// kernel runs a persistent grid: workgroup ids reach the 8 XCDs round-robin
// (id % 8), XCD x owns a contiguous range of logical items (the query blocks of
// the same few heads, which read the same K/V and so share that XCD's L2), and
// the workgroups of an XCD walk that range in rounds, in a snake order (round
// k: slot s takes position s, or P-1-s when k is odd), so that heavy and light
// causal blocks pair up.  Within a head, logical items run from the heaviest
// causal query block to the lightest.
//
// Backward pass: one workgroup per block of keys (dK/dV) or queries (dQ); the
// logical block of workgroup id gives XCD x a contiguous range of blocks (whole
// heads).
#pragma once

// (__host__ / __device__ come from the HIP API header: attributes under the HIP
// compiler, nothing under a plain host compiler.)
#include <hip/hip_runtime_api.h>

namespace fa2 {
namespace sched {

// The walk of workgroup `wg` of a persistent grid of `grid` workgroups over
// `items` logical items (fewer than 8 workgroups split the items that many ways).
struct Walk {
  int P;        // workgroups on this workgroup's XCD
  int lslot;    // this workgroup's slot among them
  int x_base;   // first logical item of the XCD's range
  int x_items;  // items in the XCD's range
};
__host__ __device__ constexpr Walk walk_of(int items, int grid, int wg) {
  const int nx = grid < 8 ? grid : 8;
  const int xcd = wg % nx;
  const int per = items / nx, rem = items % nx;
  return Walk{(grid - xcd + nx - 1) / nx, wg / nx, xcd * per + (xcd < rem ? xcd : rem),
              per + (xcd < rem ? 1 : 0)};
}
// The k-th item of the walk (k = 0, 1, ...), or -1 once the walk has ended.
__host__ __device__ constexpr int item_of(const Walk& w, int k) {
  const int pos = k * w.P + ((k & 1) ? w.P - 1 - w.lslot : w.lslot);
  return pos < w.x_items ? w.x_base + pos : -1;
}

// Logical item -> (batch*head, query block, split): splits fastest, then the
// query blocks of a head (heaviest causal block first), then the heads.
struct Item {
  int bh;
  int m;
  int split;
};
__host__ __device__ constexpr Item decode(int logical, int num_m_block, int num_splits,
                                          bool causal, bool split) {
  int mi = logical, s = 0;
  if (split) {
    mi = logical / num_splits;
    s = logical - mi * num_splits;
  }
  const int bh = mi / num_m_block;
  mi -= bh * num_m_block;
  return Item{bh, causal ? num_m_block - 1 - mi : mi, s};
}

// K/V blocks of BN keys that query block m (rows m*kBM ..) visits: up to the
// last key its last row sees with the causal mask (aligned bottom-right,
// off = Nk - Nq), all nkb blocks without.  A query block whose last row sees no
// key has none with splits, and one block (computed fully masked) without.
__host__ __device__ constexpr int blocks_of(int m, int Nq, int off, int nkb, int kBM, int BN,
                                            bool causal, bool split) {
  if (!causal) return nkb;
  const int last_row = ((m + 1) * kBM < Nq ? (m + 1) * kBM : Nq) - 1;
  const int last_key = last_row + off;
  if (last_key < 0) return split ? 0 : 1;
  return last_key / BN + 1 < nkb ? last_key / BN + 1 : nkb;
}
// Blocks [beg, end) of split s of a query block with jt blocks: ceil(jt /
// num_splits) blocks per split, so split 0 is empty only when the query block
// sees no key at all; later splits can be empty.
struct Range {
  int beg;
  int end;
};
__host__ __device__ constexpr Range range_of(int jt, int s, int num_splits, bool split) {
  if (!split) return Range{0, jt};
  const int per = (jt + num_splits - 1) / num_splits;
  const int beg = s * per < jt ? s * per : jt;
  return Range{beg, beg + per < jt ? beg + per : jt};
}

// Backward pass: the logical block of workgroup `id` among G.  XCD x = id % 8
// takes logical blocks [x*(q+1), ...) for the first r = G % 8 XCDs and
// [r*(q+1) + (x-r)*q, ...) for the others (q = G / 8): a bijection on [0, G).
__host__ __device__ constexpr int xcd_block(int id, int G) {
  const int x = id & 7, i = id >> 3, q = G >> 3, r = G & 7;
  return x < r ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

}  // namespace sched
}  // namespace fa2
