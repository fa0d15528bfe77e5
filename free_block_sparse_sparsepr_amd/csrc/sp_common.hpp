// Shared device/host helpers of the SparsePR library (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/sparsepr.h"

namespace sp {

typedef uint16_t bf16_t;

constexpr int kWave = 64;
constexpr int kMaxGroups = 64;      // G_Q, G_K <= 64 (one 64-bit kept mask per query group)
constexpr int kMaxFeat = 64;        // r_k and G_K feature widths <= 64
constexpr int kMaxSemFeat = 128;    // feature width of the semantic partition (d)
constexpr int kMaxProbe = 64;
constexpr int kMaxRank = 32;
constexpr int kMaxCorrRank = 64;   // columns of A / rows of B: rank, or n_probe for the unprojected ridge
constexpr int kExpTable = 1024;     // route exponential table entries
constexpr int kProbeChunk = 1024;   // keys per probe-attention work item, at most

// Keys per probe-attention work item: an eighth of the keys rounded up to 64, between 64
// and kProbeChunk, so that short sequences still spread over several blocks.  It depends on
// n alone, so a head's probe rows (their per-chunk rounding) do not depend on how many heads
// a call holds.
inline int probe_chunk(int n) {
  const int c = ((n + 7) / 8 + 63) / 64 * 64;
  return c < 64 ? 64 : (c > kProbeChunk ? kProbeChunk : c);
}
constexpr int kGmChunk = 1024;      // tokens per chunk of the group-major counting sort

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Per-query-head float64 scratch of the probe fit (probe_merge_kernel and the three fit
// kernels), in doubles from the head's base: raw X = O_sparse and Y = O_dense - O_sparse
// rows, their weighted centred and scaled copies Xt, Yt, the dual matrix K (Cholesky factor
// in place) and the residual Gram matrix G, the ordered leading eigenvectors a and
// eigenvalues ev of G, the weighted means xbar and ybar, and r_eff.
struct FitBuf {
  static constexpr int MM = kMaxProbe;
  __host__ __device__ static int64_t x(int) { return 0; }
  __host__ __device__ static int64_t y(int d) { return (int64_t)MM * d; }
  __host__ __device__ static int64_t xt(int d) { return 2 * (int64_t)MM * d; }
  __host__ __device__ static int64_t yt(int d) { return 3 * (int64_t)MM * d; }
  __host__ __device__ static int64_t k(int d) { return 4 * (int64_t)MM * d; }
  __host__ __device__ static int64_t g(int d) { return k(d) + MM * MM; }
  __host__ __device__ static int64_t a(int d) { return g(d) + MM * MM; }
  __host__ __device__ static int64_t ev(int d) { return a(d) + MM * kMaxRank; }
  __host__ __device__ static int64_t xbar(int d) { return ev(d) + MM; }
  __host__ __device__ static int64_t ybar(int d) { return xbar(d) + d; }
  __host__ __device__ static int64_t reff(int d) { return ybar(d) + d; }
  __host__ __device__ static int64_t per_head(int d) { return reff(d) + 8; }
};

// Group-major V is stored transposed (d-major) as [Hkv][d][n_pad], n_pad = n rounded up to
// 16.  Within every 16-key group the keys are stored in the order 0-3, 8-11, 4-7, 12-15
// (bits 2 and 3 of the position swapped), which is the order in which the matrix cores'
// k-permuted P^T operand pairs them with V: a lane's 8 keys of one k-step are one
// contiguous 16-byte chunk.  Element (d, p) lives at d * n_pad + vt_pos(p).
__host__ __device__ inline int64_t vt_pad(int64_t n) { return (n + 15) & ~(int64_t)15; }
__host__ __device__ inline int vt_pos(int p) { return (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1); }
__host__ __device__ inline int round_up4(int x) { return (x + 3) & ~3; }

__device__ __forceinline__ float bf16_to_f32(bf16_t x) { return __uint_as_float(((uint32_t)x) << 16); }
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  __bf16 h = (__bf16)f;  // round to nearest even (v_cvt_pk_bf16_f32)
  return __builtin_bit_cast(bf16_t, h);
}

template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t x) { return bf16_to_f32(x); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return f32_to_bf16(x); }

// Largest integer e with m * 2^e <= limit (0 when m == 0).  Power-of-two scaling of a
// float is exact, so this decision is identical in float32 and float64.
// Non-finite or non-positive maxima give 0; the adjustment loops are bounded.
__device__ __forceinline__ int pow2_exponent(float m, float limit) {
  if (!(m > 0.f) || !(m < INFINITY)) return 0;
  int e;
  frexpf(limit / m, &e);
  e -= 1;
  for (int it = 0; it < 320 && ldexpf(m, e + 1) <= limit; ++it) ++e;
  for (int it = 0; it < 320 && ldexpf(m, e) > limit; ++it) --e;
  return e;
}

// Integer a / b (b > 0) rounded half away from zero.
__device__ __forceinline__ int div_rhaz(int a, int b) {
  int q = (2 * (a < 0 ? -a : a) + b) / (2 * b);
  return a < 0 ? -q : q;
}

// Exact floor(num / den) for 64-bit unsigned operands below 2^62.
__device__ __forceinline__ uint64_t udiv_exact(uint64_t num, uint64_t den) {
  if (den == 0) return 0;
  uint64_t q = (uint64_t)((double)num / (double)den);
  while (q > 0 && q * den > num) --q;
  while ((q + 1) * den <= num) ++q;
  return q;
}

// Butterfly reductions over the 64 lanes of a wave (every lane receives the result) with DPP
// row permutes (quad pairs, quads, half-row and row mirrors) and the gfx950 lane-swap
// instructions across 16- and 32-lane halves: no LDS traffic.  All lanes must be active.
template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ int wave_max_i32(int v) {
  v = max(v, dpp_i32<0xB1>(v));    // quad_perm [1,0,3,2]
  v = max(v, dpp_i32<0x4E>(v));    // quad_perm [2,3,0,1]
  v = max(v, dpp_i32<0x141>(v));   // row_half_mirror
  v = max(v, dpp_i32<0x140>(v));   // row_mirror
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = max((int)a[0], (int)a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max((int)b[0], (int)b[1]);
}
__device__ __forceinline__ int wave_sum_i32(int v) {
  v += dpp_i32<0xB1>(v);
  v += dpp_i32<0x4E>(v);
  v += dpp_i32<0x141>(v);
  v += dpp_i32<0x140>(v);
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = (int)a[0] + (int)a[1];
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return (int)b[0] + (int)b[1];
}
// A lane's value combined with that of lane l ^ 32 (both lanes get the same result).
__device__ __forceinline__ float max_xor32(float v) {
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  return fmaxf(__int_as_float((int)b[0]), __int_as_float((int)b[1]));
}
__device__ __forceinline__ float add_xor32(float v) {
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  return __int_as_float((int)b[0]) + __int_as_float((int)b[1]);
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const int lo = dpp_i32<CTRL>(__double2loint(x)), hi = dpp_i32<CTRL>(__double2hiint(x));
  return __hiloint2double(hi, lo);
}
__device__ __forceinline__ double swap16_f64(double x, double& other) {
  const auto lo = __builtin_amdgcn_permlane16_swap(__double2loint(x), __double2loint(x), false, false);
  const auto hi = __builtin_amdgcn_permlane16_swap(__double2hiint(x), __double2hiint(x), false, false);
  other = __hiloint2double((int)hi[1], (int)lo[1]);
  return __hiloint2double((int)hi[0], (int)lo[0]);
}
__device__ __forceinline__ double swap32_f64(double x, double& other) {
  const auto lo = __builtin_amdgcn_permlane32_swap(__double2loint(x), __double2loint(x), false, false);
  const auto hi = __builtin_amdgcn_permlane32_swap(__double2hiint(x), __double2hiint(x), false, false);
  other = __hiloint2double((int)hi[1], (int)lo[1]);
  return __hiloint2double((int)hi[0], (int)lo[0]);
}
// Sum over the wave in float64: exact whenever every partial sum is an integer below 2^53.
__device__ __forceinline__ double wave_sum_f64(double x) {
  x += dpp_f64<0xB1>(x);
  x += dpp_f64<0x4E>(x);
  x += dpp_f64<0x141>(x);
  x += dpp_f64<0x140>(x);
  double o;
  double s = swap16_f64(x, o);
  x = s + o;
  s = swap32_f64(x, o);
  return s + o;
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// A zero-fill kernel (used instead of hipMemsetAsync so the call can be captured).
__global__ void fill_u32_kernel(uint32_t* p, size_t n, uint32_t v);
void fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t s);

// Workspace layout shared by the entry points (regions may overlap across entry
// points because calls on one stream never run concurrently).
struct Workspace {
  size_t maxbits, xk, xq, centroids, sums, usum, gm_hist, total_partition;
  size_t partials, fitbuf, probe_alloc, total_probe;
  size_t dense_meta, dense_claim, total_dense;
  size_t fused_ogm, total_fused;
  size_t rt_order, rt_pos, rt_prefix, rt_cost, rt_kept, rt_head, total_route;   // global route budget
  size_t attn_order;   // attention tile order, past every other region (attend may run beside probe_fit)
  size_t total;
  int fpk, fpq, nchunks;
};
Workspace plan_workspace(const sparsepr_params& p);

struct Dims {
  int hq, hkv, g, n, d, gq, gk, rk, m, r, iters;
  int ablation, probe_mode;
  bool semantic;   // partition on raw activations (ablation)
  int fq;          // query feature width: G_K, or d for the semantic partition
  int rc;   // correction rank: columns of A / rows of B (rank, or m for the unprojected ridge)
  bool global_budget;   // one route budget shared by all KV heads
  int tile;             // cell cost padded to tile x tile blocks (0: unpadded pairs)
  float scale, lambda;
  bool bf16;
};
Dims dims_of(const sparsepr_params& p);

}  // namespace sp
