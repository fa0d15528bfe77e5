// Routing of (query group x key group) cells to a target execution density (summary page
// of "Partition the Support, Reconstruct the Residual", execution paragraph: rho_exec =
// rho_route + M / N, the router subtracts the probe cost first, cells are indivisible so
// the realised density deviates slightly from the target).
//
// Cell masses are exact fixed-point integers: every query row's mass on key group b is
// the size-weighted softmax of its responses to the key centroids, with logits rounded
// to 1/64 units and exponentiated through a 1024-entry table, floor-divided to 2^20
// units and summed with 64-bit integer atomics (order-free, hence deterministic).
// Selection is one block per KV head: a mandatory heaviest cell per non-empty query
// group, a bitonic sort of the other cells by mass per unit cost (exact 128-bit
// cross-multiplication, ties to the smaller cell index), a prefix scan of their costs
// and the longest prefix that fits the budget.  Variants: a cell may cost its tile-padded
// pairs, and one budget may be shared by all KV heads (each optional cell then finds its
// place in the shared order by binary searches over the other heads' sorted cells).
#include <climits>
#include <cmath>
#include <mutex>

#include "sp_common.hpp"
#include "sp_launch.hpp"

namespace sp {

// E[k] = rint(2^20 exp(-k / 64)), k < 1024, formed by every block that needs it in double
// precision: each 2^20 exp(-k / 64) lies at least 2.3e-4 from a rounding boundary (the
// closest is k = 657, 36.50023...), far above the few-ulp (2^-32 at 2^20) error of the
// double exponential, so the rounded entries are exact and nothing is uploaded or cached.
__device__ __forceinline__ void fill_exp_table(uint32_t* etab, int tid, int nthreads) {
  for (int i = tid; i < kExpTable; i += nthreads) etab[i] = (uint32_t)rint(1048576.0 * exp(-(double)i / 64.0));
}

// One wave per query row (lanes over key groups): coalesced loads of the row's
// responses, wave max / sum, per-lane fixed-point division, LDS accumulation per block,
// then 64-bit integer atomics.  Each wave walks kRouteRows rows, with the responses and
// labels of the next kRoutePrefetch rows in flight and the exponential table staged in
// LDS, so a row costs no dependent global load.  grid (ceil(n / (4 kRouteRows)), Hq),
// block 256.  mass [Hkv][Gq][Gk] must be zero on entry.
constexpr int kRouteRows = 64;
static_assert(4 * kRouteRows <= 4096, "a block's cell sums must stay below 2^32");
constexpr int kRoutePrefetch = 8;

__global__ __launch_bounds__(256) void route_mass_kernel(const float* __restrict__ U,
                                                         const int32_t* __restrict__ qlabels,
                                                         const int32_t* __restrict__ koff, int n,
                                                         int g, int Gq, int Gk,
                                                         unsigned long long* __restrict__ mass) {
  // a block's rows (at most 4 kRouteRows = 256, each adding at most 2^20 to a cell) keep a
  // cell's partial sum below 2^28: 32-bit LDS accumulators (16 KB), 64-bit global atomics
  __shared__ uint32_t acc[kMaxGroups * kMaxGroups];
  __shared__ uint32_t etab[kExpTable];
  const int h = blockIdx.y, kv = h / g;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < Gq * Gk; i += 256) acc[i] = 0u;
  fill_exp_table(etab, threadIdx.x, 256);
  const int nb = lane < Gk ? koff[(int64_t)kv * (Gk + 1) + lane + 1] - koff[(int64_t)kv * (Gk + 1) + lane] : 0;
  __syncthreads();
  const int r0 = (blockIdx.x * 4 + w) * kRouteRows;
  const int r1 = min(n, r0 + kRouteRows);
  const float* Uh = U + (int64_t)h * n * Gk;
  const int32_t* lab = qlabels + (int64_t)kv * n;
  for (int i0 = r0; i0 < r1; i0 += kRoutePrefetch) {
    float u[kRoutePrefetch];
    int la[kRoutePrefetch];
#pragma unroll
    for (int j = 0; j < kRoutePrefetch; ++j) {
      const int i = min(i0 + j, r1 - 1);
      u[j] = lane < Gk ? Uh[(int64_t)i * Gk + lane] : 0.f;
      la[j] = lab[i];
    }
#pragma unroll
    for (int j = 0; j < kRoutePrefetch; ++j) {
      if (i0 + j >= r1) break;
      int z = INT_MIN;
      if (lane < Gk) z = (int)fminf(fmaxf(rintf(64.f * u[j]), -1073741824.f), 1073741824.f);
      const int mu = wave_max_i32((nb > 0) ? z : INT_MIN);
      uint64_t e = 0;
      if (nb > 0) {
        const int64_t dz = (int64_t)mu - (int64_t)z;
        const int k = dz > kExpTable - 1 ? kExpTable - 1 : (int)dz;
        e = (uint64_t)nb * (uint64_t)etab[k];
      }
      // e <= 2^22 * 2^20 per lane, so every partial sum of the 64 lanes stays below 2^48
      // and the float64 sum is exact
      const uint64_t tot = (uint64_t)wave_sum_f64((double)e);
      if (e) atomicAdd(&acc[la[j] * Gk + lane], (uint32_t)udiv_exact(e << 20, tot));
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < Gq * Gk; idx += 256) {
    const unsigned long long v = acc[idx];
    if (v) atomicAdd(&mass[(int64_t)kv * Gq * Gk + idx], v);
  }
}

struct CellKey {
  uint64_t m;
  uint64_t c;
};

// a precedes b: valid first, then larger m/c, then smaller index
__device__ __forceinline__ bool cell_before(const uint64_t* m, const uint64_t* cost, const uint8_t* valid,
                                            int x, int y) {
  if (valid[x] != valid[y]) return valid[x] > valid[y];
  if (!valid[x]) return x < y;
  unsigned __int128 l = (unsigned __int128)m[x] * cost[y];
  unsigned __int128 r = (unsigned __int128)m[y] * cost[x];
  if (l != r) return l > r;
  return x < y;
}

// Cost of a cell: n_a n_b pairs, or the pairs of the tile x tile blocks it occupies.
__device__ __forceinline__ uint64_t cell_cost(int na, int nb, int tile) {
  if (na <= 0 || nb <= 0) return 0;
  if (tile > 0) {
    na = (na + tile - 1) / tile * tile;
    nb = (nb + tile - 1) / tile * tile;
  }
  return (uint64_t)na * (uint64_t)nb;
}

// CSR (columns ascending), kept masks and routed (unpadded) pairs of one KV head from its
// kept flags (LDS or global).  Called by the whole block: thread a < G_Q counts, then
// writes, row a; one thread forms the row offsets and the pair total.
__device__ void emit_route(const uint8_t* kept, const int* na, const int* nbk, int kv, int Gq, int Gk,
                           int* rcount, int32_t* __restrict__ row_ptr, int32_t* __restrict__ cols,
                           uint64_t* __restrict__ kept_mask, int64_t* __restrict__ pairs) {
  __shared__ int rstart[kMaxGroups];
  __shared__ int64_t rpairs[kMaxGroups];
  const int tid = threadIdx.x, ncell = Gq * Gk;
  if (tid < Gq) {
    int cnt = 0;
    uint64_t msk = 0;
    for (int b = 0; b < Gk; ++b)
      if (kept[tid * Gk + b]) { ++cnt; msk |= 1ull << b; }
    rcount[tid] = cnt;
    kept_mask[(int64_t)kv * Gq + tid] = msk;
  }
  __syncthreads();
  if (tid == 0) {
    int s = 0;
    for (int a = 0; a < Gq; ++a) {
      rstart[a] = s;
      row_ptr[(int64_t)kv * (Gq + 1) + a] = s;
      s += rcount[a];
    }
    row_ptr[(int64_t)kv * (Gq + 1) + Gq] = s;
  }
  __syncthreads();
  if (tid < Gq) {
    int w = rstart[tid];
    int64_t pr = 0;
    for (int b = 0; b < Gk; ++b)
      if (kept[tid * Gk + b]) { cols[(int64_t)kv * ncell + w++] = b; pr += (int64_t)na[tid] * nbk[b]; }
    rpairs[tid] = pr;
  }
  __syncthreads();
  if (tid == 0) {
    int64_t pr = 0;
    for (int a = 0; a < Gq; ++a) pr += rpairs[a];
    pairs[kv] = pr;
  }
}

// Per-head selection products for the global budget (workspace): the head's optional
// cells in its sorted order, each cell's position there (-1: mandatory or empty), the
// inclusive prefix cost along that order, every cell's cost, the kept flags (mandatory
// cells only so far) and per head {mandatory cost, number of optional cells}.
struct GlobalRoute {
  int32_t* order;
  int32_t* pos;
  int64_t* prefix;
  uint64_t* cost;
  uint8_t* kept;
  int64_t* head;
};

// One block (1024 threads) per KV head.  Per-head budget: the whole selection and the
// route outputs.  Global budget (g.order != nullptr): only the per-head products above.
__global__ __launch_bounds__(1024) void route_select_kernel(const unsigned long long* __restrict__ mass,
                                                            const int32_t* __restrict__ qoff,
                                                            const int32_t* __restrict__ koff, int Gq,
                                                            int Gk, int64_t budget, int tile,
                                                            int32_t* __restrict__ row_ptr,
                                                            int32_t* __restrict__ cols,
                                                            uint64_t* __restrict__ kept_mask,
                                                            int64_t* __restrict__ pairs, GlobalRoute g) {
  constexpr int CELLS = kMaxGroups * kMaxGroups;
  __shared__ uint64_t sm[CELLS];
  __shared__ uint64_t sc[CELLS];
  __shared__ uint8_t valid[CELLS];
  __shared__ uint8_t kept[CELLS];
  __shared__ uint16_t order[CELLS];
  __shared__ int64_t part[1024];
  __shared__ int na[kMaxGroups], nbk[kMaxGroups], mand[kMaxGroups], rcount[kMaxGroups];
  __shared__ int64_t left_s, mcost_s;
  const bool global = g.order != nullptr;
  const int kv = blockIdx.x, tid = threadIdx.x;
  const int ncell = Gq * Gk;
  int P = 1;
  while (P < ncell) P <<= 1;
  if (tid < Gq) na[tid] = qoff[(int64_t)kv * (Gq + 1) + tid + 1] - qoff[(int64_t)kv * (Gq + 1) + tid];
  if (tid < Gk) nbk[tid] = koff[(int64_t)kv * (Gk + 1) + tid + 1] - koff[(int64_t)kv * (Gk + 1) + tid];
  __syncthreads();
  for (int c = tid; c < P; c += 1024) {
    if (c < ncell) {
      int a = c / Gk, b = c % Gk;
      sm[c] = mass[(int64_t)kv * ncell + c];
      sc[c] = cell_cost(na[a], nbk[b], tile);
    } else {
      sm[c] = 0; sc[c] = 0;
    }
    kept[c] = 0;
    order[c] = (uint16_t)c;
  }
  __syncthreads();
  // mandatory heaviest non-empty key group of every non-empty query group (ties: smaller b)
  if (tid < Gq) {
    int best = -1;
    if (na[tid] > 0) {
      for (int b = 0; b < Gk; ++b) {
        if (nbk[b] == 0) continue;
        if (best < 0 || sm[tid * Gk + b] > sm[tid * Gk + best]) best = b;
      }
    }
    mand[tid] = best;
    if (best >= 0) kept[tid * Gk + best] = 1;
  }
  __syncthreads();
  if (tid == 0) {
    int64_t mc = 0;
    for (int a = 0; a < Gq; ++a)
      if (mand[a] >= 0) mc += (int64_t)sc[a * Gk + mand[a]];
    mcost_s = mc;
    left_s = budget - mc;
  }
  for (int c = tid; c < P; c += 1024) valid[c] = (c < ncell && sc[c] > 0 && !kept[c]) ? 1 : 0;
  __syncthreads();
  // bitonic sort of cell indices
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = tid; t < P / 2; t += 1024) {
        int lo = 2 * t - (t & (stride - 1));
        int hi = lo + stride;
        bool up = ((lo & size) == 0);
        int x = order[lo], y = order[hi];
        bool swap = up ? cell_before(sm, sc, valid, y, x) : cell_before(sm, sc, valid, x, y);
        if (swap) { order[lo] = (uint16_t)y; order[hi] = (uint16_t)x; }
      }
      __syncthreads();
    }
  }
  // inclusive prefix sum of costs in sorted order (valid cells come first)
  const int per = (P + 1023) / 1024;
  int64_t local = 0;
  for (int i = 0; i < per; ++i) {
    int pos = tid * per + i;
    if (pos < P) { int c = order[pos]; if (valid[c]) local += (int64_t)sc[c]; }
  }
  part[tid] = local;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    int64_t v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int64_t run = tid > 0 ? part[tid - 1] : 0;
  const int64_t left = left_s;
  if (global) {
    const int64_t base = (int64_t)kv * ncell;
    for (int c = tid; c < ncell; c += 1024) {
      g.pos[base + c] = -1;
      g.cost[base + c] = sc[c];
      g.kept[base + c] = kept[c];
    }
    __syncthreads();
    for (int i = 0; i < per; ++i) {
      int pos = tid * per + i;
      if (pos < P) {
        int c = order[pos];
        if (valid[c]) {
          run += (int64_t)sc[c];
          g.order[base + pos] = c;
          g.prefix[base + pos] = run;
          g.pos[base + c] = pos;
        }
      }
    }
    __syncthreads();
    if (tid == 0) {
      int cnt = 0;
      for (int c = 0; c < ncell; ++c) cnt += valid[c];
      g.head[2 * kv] = mcost_s;
      g.head[2 * kv + 1] = cnt;
    }
    return;
  }
  for (int i = 0; i < per; ++i) {
    int pos = tid * per + i;
    if (pos < P) {
      int c = order[pos];
      if (valid[c]) {
        run += (int64_t)sc[c];
        if (run <= left) kept[c] = 1;
      }
    }
  }
  __syncthreads();
  emit_route(kept, na, nbk, kv, Gq, Gk, rcount, row_ptr, cols, kept_mask, pairs);
}

// Global budget: every optional cell of every head decides on its own whether it lies in
// the shared prefix.  Its inclusive cumulative cost in the shared order (mass per unit cost
// descending, ties to the smaller head, then the smaller cell) is its own head's prefix
// cost plus, for every other head, the prefix cost of that head's cells that precede it
// (a binary search along that head's sorted order).  grid (ceil(Hkv G_Q G_K / 256)),
// block 256.
__global__ __launch_bounds__(256) void route_global_kernel(const unsigned long long* __restrict__ mass, int hkv,
                                                           int ncell, int64_t budget_total, GlobalRoute g) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)hkv * ncell) return;
  const int h = (int)(idx / ncell), c = (int)(idx % ncell);
  const int pos = g.pos[idx];
  if (pos < 0) return;
  int64_t left = budget_total;
  for (int k = 0; k < hkv; ++k) left -= g.head[2 * k];
  const uint64_t mp = mass[idx], cp = g.cost[idx];
  int64_t cum = g.prefix[idx - c + pos];
  for (int k = 0; k < hkv; ++k) {
    if (k == h) continue;
    const int64_t base = (int64_t)k * ncell;
    // number of head-k cells before (h, c): ratio above ours, or equal with k < h
    int lo = 0, hi = (int)g.head[2 * k + 1];
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      const int x = g.order[base + mid];
      const unsigned __int128 l = (unsigned __int128)mass[base + x] * cp;
      const unsigned __int128 r = (unsigned __int128)mp * g.cost[base + x];
      const bool before = l > r || (l == r && k < h);
      if (before) lo = mid + 1; else hi = mid;
    }
    if (lo > 0) cum += g.prefix[base + lo - 1];
  }
  if (cum <= left) g.kept[idx] = 1;
}

// Global budget: the route outputs of one KV head from the kept flags.  grid Hkv, block 64.
__global__ __launch_bounds__(64) void route_emit_kernel(const int32_t* __restrict__ qoff,
                                                        const int32_t* __restrict__ koff, int Gq, int Gk,
                                                        const uint8_t* __restrict__ kept_all,
                                                        int32_t* __restrict__ row_ptr, int32_t* __restrict__ cols,
                                                        uint64_t* __restrict__ kept_mask,
                                                        int64_t* __restrict__ pairs) {
  __shared__ int na[kMaxGroups], nbk[kMaxGroups], rcount[kMaxGroups];
  const int kv = blockIdx.x, tid = threadIdx.x;
  if (tid < Gq) na[tid] = qoff[(int64_t)kv * (Gq + 1) + tid + 1] - qoff[(int64_t)kv * (Gq + 1) + tid];
  if (tid < Gk) nbk[tid] = koff[(int64_t)kv * (Gk + 1) + tid + 1] - koff[(int64_t)kv * (Gk + 1) + tid];
  __syncthreads();
  emit_route(kept_all + (int64_t)kv * Gq * Gk, na, nbk, kv, Gq, Gk, rcount, row_ptr, cols, kept_mask, pairs);
}

void launch_route(const Dims& dm, int64_t budget, const sparsepr_partition_t& part, const sparsepr_route_t& out,
                  const Workspace& wp, char* ws, hipStream_t s) {
  fill_u32(reinterpret_cast<uint32_t*>(out.cell_mass), (size_t)dm.hkv * dm.gq * dm.gk * 2, 0, s);
  hipLaunchKernelGGL(route_mass_kernel, dim3((unsigned)ceil_div(dm.n, 4 * kRouteRows), dm.hq), dim3(256), 0, s,
                     part.responses_u, part.query_labels, part.key_offsets, dm.n, dm.g, dm.gq, dm.gk,
                     reinterpret_cast<unsigned long long*>(out.cell_mass));
  GlobalRoute g{};
  if (dm.global_budget) {
    g.order = reinterpret_cast<int32_t*>(ws + wp.rt_order);
    g.pos = reinterpret_cast<int32_t*>(ws + wp.rt_pos);
    g.prefix = reinterpret_cast<int64_t*>(ws + wp.rt_prefix);
    g.cost = reinterpret_cast<uint64_t*>(ws + wp.rt_cost);
    g.kept = reinterpret_cast<uint8_t*>(ws + wp.rt_kept);
    g.head = reinterpret_cast<int64_t*>(ws + wp.rt_head);
  }
  const auto* cm = reinterpret_cast<const unsigned long long*>(out.cell_mass);
  hipLaunchKernelGGL(route_select_kernel, dim3(dm.hkv), dim3(1024), 0, s, cm, part.query_offsets, part.key_offsets,
                     dm.gq, dm.gk, budget, dm.tile, out.row_ptr, out.cols, out.kept_mask, out.pairs, g);
  if (!dm.global_budget) return;
  const int ncell = dm.gq * dm.gk;
  hipLaunchKernelGGL(route_global_kernel, dim3((unsigned)ceil_div((int64_t)dm.hkv * ncell, 256)), dim3(256), 0, s,
                     cm, dm.hkv, ncell, budget * dm.hkv, g);
  hipLaunchKernelGGL(route_emit_kernel, dim3(dm.hkv), dim3(64), 0, s, part.query_offsets, part.key_offsets, dm.gq,
                     dm.gk, g.kept, out.row_ptr, out.cols, out.kept_mask, out.pairs);
}

}  // namespace sp
