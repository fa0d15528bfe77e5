// Tile scheduling shared by the block-sparse (routed) and dense attention kernels.
#pragma once
#include "sp_common.hpp"

namespace sp {

// Argument block of the attention kernels.  A "virtual row" v of KV head kv is the pair
// (position p = v / g, query head j = v % g); group a owns virtual rows
// [qoff[a] g, qoff[a+1] g), so all query heads of a KV head share one key stream.
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  int64_t q_skv, q_sp, q_sj;   // element strides of Q rows
  int64_t kv_skv;              // element stride between KV heads of K (n * d)
  int64_t v_skv;               // element stride between KV heads of transposed V (d * n_pad)
  int v_np;                    // n_pad: row length of transposed V
  const int32_t* qoff;         // [Hkv][Gq + 1]; NULL: one group holding every token
  const int32_t* koff;         // [Hkv][Gk + 1]
  const int32_t* row_ptr;      // [Hkv][Gq + 1]; NULL: every key
  const int32_t* cols;         // [Hkv][Gq * Gk]
  void* o;
  int64_t o_skv, o_sp, o_sj;
  float* lse;                  // [Hkv][n][g] or NULL
  int n, g, gq, gk;
  float scale;
  int tiles_per_head;          // tiles scheduled per KV head
  int n_heads_kv;
  const int32_t* order;        // NULL, or [Hkv][tiles_per_head][2]: (query group, tile of the group)
  const int32_t* order_count;  // [Hkv] tiles of each head in order
  // With an order: the grid's blocks go to the XCDs in turn, XCD x owning logical tiles
  // [x per_xcd, (x + 1) per_xcd).  Its first tail_start blocks take their tiles in place;
  // its later blocks (and a few spare ones) claim the rest of its range through claim[x],
  // then the rest of the other XCDs' ranges, so that a faster XCD takes over tiles that a
  // slower one has not started.  claim: NULL (every block in place) or [8] counters, each
  // set to tail_start before the launch.
  int* claim;
  int per_xcd, tail_start;
  // fused write-back (one query head per KV head): o_hat = o + c0 + (o A) B written to
  // out_tok[h][qperm[p]] in the input dtype
  const float* fitA;           // [Hq][d][rank] or NULL (no fused write-back)
  const float* fitB;           // [Hq][rank][d]
  const float* fitc0;          // [Hq][d]
  const int32_t* r_eff;        // [Hq]
  int rank;
  const int32_t* qperm;        // [Hkv][n]
  void* out_tok;               // [Hq][n][d]
};

struct TileInfo {
  int a;          // query group
  int v0, v1;     // virtual row range of this tile
  int kbeg, kend; // CSR range in cols (routed) or -1 (dense)
};

// Tile t of query group a of KV head kv (false past the group's last tile).
__device__ __forceinline__ bool group_tile(const AttnArgs& A, int kv, int a, int t, int BM, TileInfo& ti) {
  const int32_t* qo = A.qoff + (int64_t)kv * (A.gq + 1);
  const int r0 = qo[a] * A.g, r1 = qo[a + 1] * A.g;
  ti.a = a;
  ti.v0 = r0 + t * BM;
  if (ti.v0 >= r1) return false;
  ti.v1 = min(r1, ti.v0 + BM);
  const int32_t* rp = A.row_ptr + (int64_t)kv * (A.gq + 1);
  ti.kbeg = rp[a];
  ti.kend = rp[a + 1];
  return true;
}

// Number of tiles of a head is bounded by ceil(n g / BM) + Gq; blocks beyond the head's
// real tile count return early.
__device__ __forceinline__ bool find_tile(const AttnArgs& A, int kv, int t, int BM, TileInfo& ti) {
  if (A.qoff == nullptr) {
    const int rows = A.n * A.g;
    if (t * BM >= rows) return false;
    ti.a = 0;
    ti.v0 = t * BM;
    ti.v1 = min(rows, ti.v0 + BM);
    ti.kbeg = ti.kend = -1;
    return true;
  }
  const int32_t* qo = A.qoff + (int64_t)kv * (A.gq + 1);
  int acc = 0;
  for (int a = 0; a < A.gq; ++a) {
    const int r0 = qo[a] * A.g, r1 = qo[a + 1] * A.g;
    const int nt = (r1 - r0 + BM - 1) / BM;
    if (t < acc + nt) {
      ti.a = a;
      ti.v0 = r0 + (t - acc) * BM;
      ti.v1 = min(r1, ti.v0 + BM);
      const int32_t* rp = A.row_ptr + (int64_t)kv * (A.gq + 1);
      ti.kbeg = rp[a];
      ti.kend = rp[a + 1];
      return true;
    }
    acc += nt;
  }
  return false;
}

// Next contiguous key run [k0, k1) of the tile: consecutive kept key groups are adjacent
// in group-major order and merge into one run.  `ci` walks the CSR columns and must start
// at ti.kbeg (0 for the dense schedule).
__device__ __forceinline__ bool next_run(const AttnArgs& A, int kv, const TileInfo& ti, int& ci, int& k0,
                                         int& k1) {
  if (ti.kbeg < 0) {
    if (ci != 0) return false;
    ci = 1;
    k0 = 0;
    k1 = A.n;
    return true;
  }
  const int32_t* cl = A.cols + (int64_t)kv * A.gq * A.gk;
  const int32_t* ko = A.koff + (int64_t)kv * (A.gk + 1);
  while (ci < ti.kend) {
    int b = cl[ci++];
    int e = b;
    while (ci < ti.kend && cl[ci] == e + 1) { ++e; ++ci; }
    k0 = ko[b];
    k1 = ko[e + 1];
    if (k1 > k0) return true;
  }
  return false;
}

}  // namespace sp
