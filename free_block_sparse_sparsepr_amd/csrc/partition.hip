// Response-coupled Q/K partition (summary page of "Partition the Support, Reconstruct the
// Residual", response-coupled partition paragraph): sampled-query key responses, integer
// key features, online k-means over keys (values follow keys), key centroids in the
// original space, query responses to those centroids, integer response-direction
// features, online k-means over queries (one asymmetric pass), stable group-major
// permutations and the gathers of Q, K and V into group-major order (execution
// paragraph).
//
// Every integer decision is exact: features are integers in [-127, 127], distances and
// sums are exact 32-bit integer arithmetic, ties go to the smallest index and the
// partition is a stable counting sort, so the result is deterministic and independent
// of scheduling.
#include "sp_common.hpp"
#include "sp_launch.hpp"

namespace sp {

__global__ void fill_u32_kernel(uint32_t* p, size_t n, uint32_t v) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) p[i] = v;
}

void fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t s) {
  if (n == 0) return;
  int blocks = (int)std::min<size_t>(4096, (n + 255) / 256);
  hipLaunchKernelGGL(fill_u32_kernel, dim3(blocks), dim3(256), 0, s, p, n, v);
}

// ---------------------------------------------------------------------------------------
// S = Q_s K^T * scale for the r_k sampled query rows (token floor((2s+1) n / (2 r_k)),
// query head s mod g of the KV head).  One thread per key; fp32 accumulation in
// ascending d.  Also the per-head max |S| (float bits are monotone for |x|).
// grid (ceil(n / 256), Hkv), block 256.
// ---------------------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void resp_s_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                     int n, int g, int rk, float scale,
                                                     float* __restrict__ S, uint32_t* maxbits) {
  __shared__ float qs[kMaxFeat][D];
  __shared__ float red[4];
  const int kv = blockIdx.y;
  for (int idx = threadIdx.x; idx < rk * D; idx += 256) {
    int s = idx / D, c = idx % D;
    int64_t tok = ((int64_t)(2 * s + 1) * n) / (2 * rk);
    int h = kv * g + (s % g);
    qs[s][c] = to_f32(q[((int64_t)h * n + tok) * D + c]);
  }
  __syncthreads();
  const int j = blockIdx.x * 256 + threadIdx.x;
  float acc[kMaxFeat];
#pragma unroll
  for (int s = 0; s < kMaxFeat; ++s) acc[s] = 0.f;
  float mx = 0.f;
  if (j < n) {
    const T* kr = k + ((int64_t)kv * n + j) * D;
    for (int c0 = 0; c0 < D; c0 += 8) {
      float kf[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) kf[e] = to_f32(kr[c0 + e]);
#pragma unroll
      for (int s = 0; s < kMaxFeat; ++s) {
        if (s < rk) {
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[s] = fmaf(qs[s][c0 + e], kf[e], acc[s]);
        }
      }
    }
#pragma unroll
    for (int s = 0; s < kMaxFeat; ++s) {
      if (s < rk) {
        float v = acc[s] * scale;
        S[((int64_t)kv * rk + s) * n + j] = v;
        mx = fmaxf(mx, fabsf(v));
      }
    }
  }
  mx = wave_max(mx);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    atomicMax(&maxbits[kv], __float_as_uint(m));
  }
}

// X^K[j][s] = clamp(rint(S[s][j] * 2^e_S), -127, 127), e_S the largest e with
// max|S| 2^e <= 127.  Features stored point-major with a padded stride fp (zeros).
// A block converts 256 keys: coalesced reads of S rows, transpose through LDS, 16-byte
// stores of the contiguous [256][fp] byte tile.  grid (ceil(n / 256), Hkv), block 256.
__global__ __launch_bounds__(256) void key_features_kernel(const float* __restrict__ S,
                                                           const uint32_t* maxbits, int n, int rk,
                                                           int fp, int8_t* __restrict__ X,
                                                           int32_t* exps) {
  __shared__ __attribute__((aligned(16))) int8_t tile[256 * kMaxFeat];
  const int kv = blockIdx.y;
  const int j0 = blockIdx.x * 256;
  const int e = pow2_exponent(__uint_as_float(maxbits[kv]), 127.f);
  if (blockIdx.x == 0 && threadIdx.x == 0) exps[kv * 2 + 0] = e;
  const int j = j0 + threadIdx.x;
  for (int s = 0; s < fp; ++s) {
    float v = 0.f;
    if (s < rk && j < n) v = fminf(fmaxf(rintf(ldexpf(S[((int64_t)kv * rk + s) * n + j], e)), -127.f), 127.f);
    tile[threadIdx.x * fp + s] = (int8_t)(int)v;
  }
  __syncthreads();
  const int rows = min(256, n - j0);
  const int bytes = rows * fp;   // multiple of 4
  int8_t* dst = X + ((int64_t)kv * n + j0) * fp;
  for (int b = threadIdx.x * 4; b < bytes; b += 256 * 4)
    *reinterpret_cast<int32_t*>(dst + b) = *reinterpret_cast<const int32_t*>(tile + b);
}

// ---------------------------------------------------------------------------------------
// Online Lloyd k-means on integer features (exact).  Centroids C [H][G][fp] int32.
// ---------------------------------------------------------------------------------------
__global__ void kmeans_init_kernel(const int8_t* __restrict__ X, int n, int G, int fp,
                                   int32_t* __restrict__ C) {
  const int h = blockIdx.x;
  for (int idx = threadIdx.x; idx < G * fp; idx += blockDim.x) {
    int gi = idx / fp, f = idx % fp;
    int64_t tok = ((int64_t)(2 * gi + 1) * n) / (2 * G);
    C[((int64_t)h * kMaxGroups + gi) * fp + f] = X[((int64_t)h * n + tok) * fp + f];
  }
}

// Assignment argmin_g ||c_g||^2 - 2 <x, c_g> (ties: smallest g) with 4-way int8 dot
// products, plus exact per-group feature sums and counts: the block's points are
// bucketed by label (counting sort in LDS), each (group, feature) sum runs over its
// bucket, and non-zero sums go to global memory with integer atomics (order-free).
// sums: [H][G][fp + 1] (last column = count), zeroed by the caller.
// grid (ceil(n / 256), H), block 256.
template <int FP>
__global__ __launch_bounds__(256) void kmeans_assign_kernel(const int8_t* __restrict__ X, int n,
                                                            int G, const int32_t* __restrict__ C,
                                                            int32_t* __restrict__ labels,
                                                            int32_t* __restrict__ sums) {
  constexpr int W = FP / 4;
  __shared__ int32_t cw[kMaxGroups][W];
  __shared__ int32_t cn[kMaxGroups];
  __shared__ int32_t cnt[kMaxGroups], start[kMaxGroups];
  __shared__ int32_t xs[256 * W];
  __shared__ uint8_t order[256];
  const int h = blockIdx.y;
  for (int idx = threadIdx.x; idx < G * W; idx += 256) {
    int gi = idx / W, w = idx % W;
    const int32_t* c = C + ((int64_t)h * kMaxGroups + gi) * FP + 4 * w;
    uint32_t packed = (uint32_t)(uint8_t)(int8_t)c[0] | ((uint32_t)(uint8_t)(int8_t)c[1] << 8) |
                      ((uint32_t)(uint8_t)(int8_t)c[2] << 16) | ((uint32_t)(uint8_t)(int8_t)c[3] << 24);
    cw[gi][w] = (int32_t)packed;
  }
  for (int gi = threadIdx.x; gi < G; gi += 256) {
    int s = 0;
    const int32_t* c = C + ((int64_t)h * kMaxGroups + gi) * FP;
    for (int f = 0; f < FP; ++f) s += c[f] * c[f];
    cn[gi] = s;
  }
  for (int gi = threadIdx.x; gi < kMaxGroups; gi += 256) cnt[gi] = 0;
  __syncthreads();
  const int j = blockIdx.x * 256 + threadIdx.x;
  int lab = -1, slot = 0;
  if (j < n) {
    int32_t xw[W];
    const int32_t* xr = reinterpret_cast<const int32_t*>(X + ((int64_t)h * n + j) * FP);
#pragma unroll
    for (int w = 0; w < W; ++w) xw[w] = xr[w];
    int best = 0x7fffffff, bi = 0;
    for (int gi = 0; gi < G; ++gi) {
      int dot = 0;
#pragma unroll
      for (int w = 0; w < W; ++w) dot = __builtin_amdgcn_sdot4(xw[w], cw[gi][w], dot, false);
      int score = cn[gi] - 2 * dot;
      if (score < best) { best = score; bi = gi; }
    }
    labels[(int64_t)h * n + j] = bi;
    lab = bi;
#pragma unroll
    for (int w = 0; w < W; ++w) xs[threadIdx.x * W + w] = xw[w];
    slot = atomicAdd(&cnt[bi], 1);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int s = 0;
    for (int gi = 0; gi < G; ++gi) { start[gi] = s; s += cnt[gi]; }
  }
  __syncthreads();
  if (lab >= 0) order[start[lab] + slot] = (uint8_t)threadIdx.x;
  __syncthreads();
  // per (group, feature) sums over the group's members in this block (exact integers)
  const int8_t* xb = reinterpret_cast<const int8_t*>(xs);
  int32_t* sh = sums + (int64_t)h * kMaxGroups * (FP + 1);
  for (int idx = threadIdx.x; idx < G * FP; idx += 256) {
    const int gi = idx / FP, f = idx % FP;
    const int m0 = start[gi], m1 = m0 + cnt[gi];
    int acc = 0;
    for (int m = m0; m < m1; ++m) acc += xb[order[m] * FP + f];
    if (acc) atomicAdd(&sh[gi * (FP + 1) + f], acc);
  }
  for (int gi = threadIdx.x; gi < G; gi += 256)
    if (cnt[gi]) atomicAdd(&sh[gi * (FP + 1) + FP], cnt[gi]);
}

typedef int32_t ki32x4_t __attribute__((ext_vector_type(4)));
typedef int32_t ki32x16_t __attribute__((ext_vector_type(16)));

constexpr int kAssignChunk = 256;       // points per chunk: 64 per wave

// Matrix-core assignment with the same decisions and sums as kmeans_assign_kernel, on the
// int8 matrix cores (exact int32 accumulation).  Every MFMA pairs byte e of the A lane
// (i, l / 32) with byte e of the B lane (j, l / 32), so the two operands only have to agree
// on which feature (or point) each byte stands for.
//  * scores^T = C X^T: a lane owns one point and 16 of each 32-group block (its partner
//    lane l ^ 32 the other 16).  key = 64 (||c_g||^2 - 2 <x, c_g>) + g orders by score,
//    then by g; it is held negated, 128 <x, c_g> - (64 ||c_g||^2 + g) (one shift-add per
//    score, |key| < 2^28), and the maximum over the lane and its partner gives the label
//    (-key mod 64).  Groups beyond G carry a key below every real one.
//  * transpose: the same X operand times an identity slice puts the features on the lanes
//    and the points in the accumulator registers.
//  * sums: S^T += X^T onehot(labels), byte e of both operands standing for the point in
//    accumulator register e; the sums stay in registers across the block's chunks.
//  * counts: runs of equal labels among each 32 consecutive points (ballot of run starts),
//    one LDS add per run.
// At the end the waves' sums meet in LDS and go to global memory with one integer atomic
// per non-zero (group, feature).  FP must be a multiple of 16.
// The centroid update of the previous iteration runs in every block's prologue: with
// prev_sums, c_g = div_rhaz(sum_g, count_g) for features below F and groups with members,
// otherwise c_g keeps its value in Cprev; block 0 of a head stores the result in Cout.
// The blocks of a head also clear that head's slice of zero_sums (the buffer the next
// iteration accumulates into).  Without SUMS only the labels are produced.
// grid (blocks_per_head, H), block 256; block b of a head takes chunks [b chunks, (b+1) chunks).
template <int FP, bool SUMS>
__global__ __launch_bounds__(256, FP > 64 ? 1 : 2) void kmeans_assign_mfma_kernel(
    const int8_t* __restrict__ X, int n, int G, int F, const int32_t* __restrict__ Cprev,
    const int32_t* __restrict__ prev_sums, int32_t* __restrict__ Cout, int chunks, int32_t* __restrict__ labels,
    int32_t* __restrict__ sums, int32_t* __restrict__ zero_sums) {
  constexpr int KB = (FP + 31) / 32;   // 32-feature blocks
  constexpr int CROW = 32 * KB + 16;   // int8 row of C in LDS, padded
  constexpr int SROW = FP + 1;         // int32 row of the LDS sums (last column = count)
  __shared__ __attribute__((aligned(16))) int8_t cs[kMaxGroups * CROW];
  __shared__ int32_t cnk[kMaxGroups];
  __shared__ int32_t ssum[kMaxGroups * SROW];
  __shared__ __attribute__((aligned(16))) uint8_t lab_s[4][2][32];
  const int h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, hf = lane >> 5;
  const int32_t* ps = prev_sums ? prev_sums + (int64_t)h * kMaxGroups * SROW : nullptr;
  for (int idx = tid; idx < kMaxGroups * 32 * KB; idx += 256) {
    const int gi = idx / (32 * KB), f = idx % (32 * KB);
    int c = 0;
    if (gi < G && f < FP) {
      const int64_t ci = ((int64_t)h * kMaxGroups + gi) * FP + f;
      c = Cprev[ci];
      if (ps != nullptr) {
        const int cnt = ps[gi * SROW + FP];
        if (cnt > 0 && f < F) c = div_rhaz(ps[gi * SROW + f], cnt);
        if (Cout != nullptr && blockIdx.x == 0) Cout[ci] = c;
      }
    }
    cs[gi * CROW + f] = (int8_t)c;
  }
  if (zero_sums != nullptr) {
    int32_t* zh = zero_sums + (int64_t)h * kMaxGroups * SROW;
    for (int idx = blockIdx.x * 256 + tid; idx < kMaxGroups * SROW; idx += gridDim.x * 256) zh[idx] = 0;
  }
  for (int idx = tid; idx < kMaxGroups * SROW; idx += 256) ssum[idx] = 0;
  __syncthreads();
  {  // -(64 ||c_g||^2 + g), four lanes per group
    const int gi = tid >> 2, q = tid & 3;
    int s2 = 0;
#pragma unroll
    for (int t = 0; t < FP / 4; ++t) {
      const int c = cs[gi * CROW + q + 4 * t];
      s2 += c * c;
    }
    s2 += __shfl_xor(s2, 1);
    s2 += __shfl_xor(s2, 2);
    if (q == 0) cnk[gi] = -(gi < G ? 64 * s2 + gi : (1 << 30) + gi);
  }
  __syncthreads();
  // identity slice: byte e of lane (j, hf) is 1 where 16 hf + e == j
  ki32x4_t ident;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e0 = l32 - 16 * hf - 4 * q;
    ident[q] = (e0 >= 0 && e0 < 4) ? (1 << (8 * e0)) : 0;
  }
  ki32x16_t acc[KB][2];
#pragma unroll
  for (int fb = 0; fb < KB; ++fb)
#pragma unroll
    for (int gb = 0; gb < 2; ++gb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[fb][gb][r] = 0;

  const int8_t* xh = X + (int64_t)h * n * FP;
  const int pbeg = blockIdx.x * chunks * kAssignChunk;
  const int pend = min(n, pbeg + chunks * kAssignChunk);
  // operand bytes of 32 points: lane (p, hf) holds features 32 kb + 16 hf .. + 15 of point p;
  // the next 32 points' bytes are in flight while the current 32 are processed
  auto load32 = [&](int pt, ki32x4_t* raw) {
    const bool pv = pt < pend;
    const int8_t* xr = xh + (int64_t)(pv ? pt : 0) * FP + 16 * hf;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const bool in = pv && (32 * kb + 16 * hf < FP);
      raw[kb] = in ? *reinterpret_cast<const ki32x4_t*>(xr + 32 * kb) : ki32x4_t{0, 0, 0, 0};
    }
  };
  // both 32-point halves of a wave's 64 points go through each step together (two
  // independent instruction streams for the scheduler); the next 64 points are in flight
  ki32x4_t nraw[2][KB];
  load32(pbeg + w * 64 + l32, nraw[0]);
  load32(pbeg + w * 64 + 32 + l32, nraw[1]);
  for (int pbase = pbeg + w * 64; pbase < pend; pbase += kAssignChunk) {
    ki32x4_t xo[2][KB];
    int pt[2], lab[2];
    bool pv[2];
#pragma unroll
    for (int pb = 0; pb < 2; ++pb) {
      pt[pb] = pbase + pb * 32 + l32;
      pv[pb] = pt[pb] < pend;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) xo[pb][kb] = nraw[pb][kb];
      load32(pt[pb] + kAssignChunk, nraw[pb]);
    }
    // -- assignment
    int best[2] = {(int)0x80000000u, (int)0x80000000u};
#pragma unroll
    for (int gb = 0; gb < 2; ++gb) {
      const int8_t* crow = cs + (32 * gb + l32) * CROW + 16 * hf;
#pragma unroll
      for (int pb = 0; pb < 2; ++pb) {
        ki32x16_t sc;
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[r] = 0;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          sc = __builtin_amdgcn_mfma_i32_32x32x32_i8(*reinterpret_cast<const ki32x4_t*>(crow + 32 * kb), xo[pb][kb],
                                                     sc, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int gi = 32 * gb + 8 * (r >> 2) + 4 * hf + (r & 3);
          best[pb] = max(best[pb], (int)(((uint32_t)sc[r] << 7) + (uint32_t)cnk[gi]));   // one shift-add
        }
      }
    }
#pragma unroll
    for (int pb = 0; pb < 2; ++pb) {
      best[pb] = max(best[pb], __shfl_xor(best[pb], 32));
      const int bg = (-best[pb]) & 63;
      lab[pb] = pv[pb] ? bg : kMaxGroups;          // points past the end: no group
      if (pv[pb] && hf == 0) labels[(int64_t)h * n + pt[pb]] = bg;
    }
    if constexpr (!SUMS) continue;
    // -- counts: one add per run of equal labels among each half's 32 points
#pragma unroll
    for (int pb = 0; pb < 2; ++pb) {
      const int prev = __shfl(lab[pb], lane - (l32 > 0 ? 1 : 0));
      const int next = __shfl(lab[pb], lane + (l32 < 31 ? 1 : 0));
      const uint64_t startm = __ballot(l32 == 0 || prev != lab[pb]);
      if (hf == 0) {
        lab_s[w][pb][l32] = (uint8_t)lab[pb];
        if (lab[pb] < kMaxGroups && (l32 == 31 || next != lab[pb])) {
          const uint32_t m = (uint32_t)startm & (0xffffffffu >> (31 - l32));
          const int first = 31 - __builtin_clz(m);
          atomicAdd(&ssum[lab[pb] * SROW + FP], l32 - first + 1);
        }
      }
    }
    // -- onehot: byte e of lane (g, hf) is [label of point 8 (e / 4) + 4 hf + e % 4 == g]
    ki32x4_t oh[2][2];
#pragma unroll
    for (int pb = 0; pb < 2; ++pb) {
      const uint32_t* lw = reinterpret_cast<const uint32_t*>(lab_s[w][pb]);
      uint32_t lq[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) lq[q] = lw[2 * q + hf];
#pragma unroll
      for (int gb = 0; gb < 2; ++gb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          // label bytes are <= 64 and g < 64, so x + 0x7f per byte never carries
          const uint32_t x = lq[q] ^ ((uint32_t)(32 * gb + l32) * 0x01010101u);
          oh[pb][gb][q] = (int32_t)((~(x + 0x7f7f7f7fu) >> 7) & 0x01010101u);
        }
    }
    // -- transpose and sums: tx[r] = X[8 (r / 4) + 4 hf + r % 4][32 fb + l32]
#pragma unroll
    for (int fb = 0; fb < KB; ++fb) {
#pragma unroll
      for (int pb = 0; pb < 2; ++pb) {
        ki32x16_t tx;
#pragma unroll
        for (int r = 0; r < 16; ++r) tx[r] = 0;
        tx = __builtin_amdgcn_mfma_i32_32x32x32_i8(xo[pb][fb], ident, tx, 0, 0, 0);
        ki32x4_t xa;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t lo = __builtin_amdgcn_perm((uint32_t)tx[4 * q + 1], (uint32_t)tx[4 * q], 0x0c0c0400u);
          const uint32_t hi = __builtin_amdgcn_perm((uint32_t)tx[4 * q + 3], (uint32_t)tx[4 * q + 2], 0x04000c0cu);
          xa[q] = (int32_t)(lo | hi);
        }
#pragma unroll
        for (int gb = 0; gb < 2; ++gb)
          acc[fb][gb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(xa, oh[pb][gb], acc[fb][gb], 0, 0, 0);
      }
    }
  }
  if constexpr (!SUMS) return;
  // acc[fb][gb][r] = sum of feature 32 fb + 8 (r / 4) + 4 hf + r % 4 over group 32 gb + l32
#pragma unroll
  for (int fb = 0; fb < KB; ++fb)
#pragma unroll
    for (int gb = 0; gb < 2; ++gb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int f = 32 * fb + 8 * (r >> 2) + 4 * hf + (r & 3), gi = 32 * gb + l32;
        const int v = acc[fb][gb][r];
        if (f < FP && gi < G && v) atomicAdd(&ssum[gi * SROW + f], v);
      }
  __syncthreads();
  int32_t* sh = sums + (int64_t)h * kMaxGroups * SROW;
  for (int idx = tid; idx < G * SROW; idx += 256) {
    const int v = ssum[idx];
    if (v) atomicAdd(&sh[idx], v);
  }
}

// c_g = div_rhaz(sum_g, count_g); an empty group keeps its centroid.  Also clears the
// other sums buffer for the next assignment.  grid H, block 256.
__global__ void kmeans_update_kernel(const int32_t* __restrict__ sums, int G, int F, int fp,
                                     int32_t* __restrict__ C, int32_t* __restrict__ next_sums) {
  const int h = blockIdx.x;
  const int32_t* sh = sums + (int64_t)h * kMaxGroups * (fp + 1);
  for (int idx = threadIdx.x; idx < G * fp; idx += blockDim.x) {
    int gi = idx / fp, f = idx % fp;
    int cnt = sh[gi * (fp + 1) + fp];
    if (cnt > 0 && f < F) C[((int64_t)h * kMaxGroups + gi) * fp + f] = div_rhaz(sh[gi * (fp + 1) + f], cnt);
  }
  int32_t* nh = next_sums + (int64_t)h * kMaxGroups * (fp + 1);
  for (int idx = threadIdx.x; idx < kMaxGroups * (fp + 1); idx += blockDim.x) nh[idx] = 0;
}

__global__ void copy_centroids_kernel(const int32_t* __restrict__ C, int G, int F, int fp,
                                      int32_t* __restrict__ out) {
  const int h = blockIdx.x;
  for (int idx = threadIdx.x; idx < G * F; idx += blockDim.x) {
    int gi = idx / F, f = idx % F;
    out[((int64_t)h * G + gi) * F + f] = C[((int64_t)h * kMaxGroups + gi) * fp + f];
  }
}

// ---------------------------------------------------------------------------------------
// Stable counting sort of labels: offsets (exclusive scan of counts) and perm (token at
// each group-major position, tokens ascending within a group), over 1024-token chunks in
// three passes: per-chunk group counts, a scan over chunks (group offsets plus each
// chunk's base per group), and the scatter.  Within a chunk a token's rank among equal
// labels comes from wave ballots (one round per distinct label of the wave) plus the
// counts of earlier waves.
// ---------------------------------------------------------------------------------------
// Per-wave counts of the chunk's labels into wcnt[w][.] (zeroed by the caller) and the
// lane's rank among the equal labels of its wave.
__device__ __forceinline__ int gm_wave_ranks(int lab, bool valid, int lane, int w, int (*wcnt)[kMaxGroups]) {
  const uint64_t lt = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
  uint64_t active = __ballot(valid);
  int rank = 0;
  while (active) {
    const int leader = __ffsll((long long)active) - 1;
    const int L = __shfl(lab, leader);
    const uint64_t m = __ballot(lab == L) & active;
    if (valid && lab == L) rank = __popcll(m & lt);
    if (lane == leader) wcnt[w][L] = __popcll(m);
    active &= ~m;
  }
  return rank;
}

// grid (nchunks, H), block 1024: hist[h][c][b] = count of label b in chunk c
__global__ __launch_bounds__(1024) void gm_count_kernel(const int32_t* __restrict__ labels, int n, int G,
                                                        int32_t* __restrict__ hist) {
  __shared__ int wcnt[16][kMaxGroups];
  const int c = blockIdx.x, h = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  (&wcnt[0][0])[tid] = 0;
  __syncthreads();
  const int j = c * kGmChunk + tid;
  const bool valid = j < n;
  gm_wave_ranks(valid ? labels[(int64_t)h * n + j] : -1, valid, lane, w, wcnt);
  __syncthreads();
  if (tid < kMaxGroups) {
    int sum = 0;
#pragma unroll
    for (int ww = 0; ww < 16; ++ww) sum += wcnt[ww][tid];
    hist[((int64_t)h * gridDim.x + c) * kMaxGroups + tid] = sum;
  }
}

// grid (H), block 64 (lane = group): offsets and, in place, hist[h][c][b] = first
// group-major position of chunk c's tokens of group b
__global__ __launch_bounds__(64) void gm_scan_kernel(int32_t* __restrict__ hist, int nchunks, int G,
                                                     int32_t* __restrict__ offsets) {
  constexpr int U = 8;
  const int h = blockIdx.x, b = threadIdx.x;
  int32_t* hh = hist + (int64_t)h * nchunks * kMaxGroups + b;
  int total = 0;
  for (int c0 = 0; c0 < nchunks; c0 += U) {
    int v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = c0 + u < nchunks ? hh[(int64_t)(c0 + u) * kMaxGroups] : 0;
#pragma unroll
    for (int u = 0; u < U; ++u) total += v[u];
  }
  int incl = total;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int x = __shfl_up(incl, o);
    if (b >= o) incl += x;
  }
  int run = incl - total;
  if (b < G) offsets[(int64_t)h * (G + 1) + b] = run;
  if (b == G - 1) offsets[(int64_t)h * (G + 1) + G] = incl;
  for (int c0 = 0; c0 < nchunks; c0 += U) {
    int v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = c0 + u < nchunks ? hh[(int64_t)(c0 + u) * kMaxGroups] : 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (c0 + u < nchunks) hh[(int64_t)(c0 + u) * kMaxGroups] = run;
      run += v[u];
    }
  }
}

// grid (nchunks, H), block 1024
__global__ __launch_bounds__(1024) void gm_scatter_kernel(const int32_t* __restrict__ labels, int n,
                                                          const int32_t* __restrict__ base,
                                                          int32_t* __restrict__ perm) {
  __shared__ int wcnt[16][kMaxGroups];
  const int c = blockIdx.x, h = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  (&wcnt[0][0])[tid] = 0;
  __syncthreads();
  const int j = c * kGmChunk + tid;
  const bool valid = j < n;
  const int lab = valid ? labels[(int64_t)h * n + j] : -1;
  const int rank = gm_wave_ranks(lab, valid, lane, w, wcnt);
  __syncthreads();
  if (valid) {
    int pre = base[((int64_t)h * gridDim.x + c) * kMaxGroups + lab];
    for (int ww = 0; ww < w; ++ww) pre += wcnt[ww][lab];
    perm[(int64_t)h * n + pre + rank] = j;
  }
}

// ---------------------------------------------------------------------------------------
// Row gather into group-major order: dst row (kv, p, j) <- src head kv*g + j, token
// perm[kv][p].  16-byte vector copies; dst layout [Hkv][n][g][D].
// ---------------------------------------------------------------------------------------
template <int ROW_BYTES>
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint4* __restrict__ src,
                                                          const int32_t* __restrict__ perm, int n,
                                                          int g, int64_t rows, uint4* __restrict__ dst) {
  constexpr int VPR = ROW_BYTES / 16;
  int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  int64_t r = t / VPR;
  int c = (int)(t % VPR);
  if (r >= rows) return;
  int64_t kvp = r / g;
  int jh = (int)(r % g);
  int64_t kv = kvp / n;
  int64_t p = kvp % n;
  int64_t tok = perm[kv * n + p];
  int64_t srow = (kv * g + jh) * n + tok;
  dst[r * VPR + c] = src[srow * VPR + c];
}

// Transposing gather of V into group-major, d-major order: block = kVtBlock positions; rows
// perm[p] (or p when perm is NULL) are staged in LDS with 16-byte loads, then each thread
// assembles one 16-byte chunk (8 positions of one d row, in the layout's key order
// vt_pos, an involution within each 16-key group) and stores it whole.  Positions from n
// up to n_pad are zero.  grid (ceil(n_pad / kVtBlock), Hkv), block 256.  128 positions make
// each d row's store 256 contiguous bytes (bf16) at four blocks per CU.
constexpr int kVtBlock = 128;

static_assert(kVtBlock % 16 == 0, "vt_pos permutes within 16-key groups");

template <typename T, int D>
__global__ __launch_bounds__(256) void gather_vt_kernel(const T* __restrict__ v, const int32_t* __restrict__ perm,
                                                        int n, int np, T* __restrict__ vt) {
  constexpr int EPC = 16 / sizeof(T);       // elements per 16-byte chunk
  constexpr int CPR = D / EPC;              // chunks per row
  constexpr int ROW = D + 2;                // padded LDS row (elements)
  __shared__ T tile[kVtBlock * ROW];
  const int kv = blockIdx.y, p0 = blockIdx.x * kVtBlock;
  for (int idx = threadIdx.x; idx < kVtBlock * CPR; idx += 256) {
    const int r = idx / CPR, c = idx % CPR, p = p0 + r;
    uint4 x = make_uint4(0, 0, 0, 0);
    if (p < n) {
      const int64_t tok = perm ? perm[(int64_t)kv * n + p] : p;
      x = *reinterpret_cast<const uint4*>(v + ((int64_t)kv * n + tok) * D + c * EPC);
    }
    const T* xe = reinterpret_cast<const T*>(&x);
#pragma unroll
    for (int e = 0; e < EPC; ++e) tile[r * ROW + c * EPC + e] = xe[e];
  }
  __syncthreads();
  // output chunk: row d, positions p0 + EPC q .. + EPC - 1
  constexpr int QPR = kVtBlock / EPC;       // chunks per d row in this block
  for (int idx = threadIdx.x; idx < D * QPR; idx += 256) {
    const int d = idx / QPR, q = idx % QPR;
    if (p0 + EPC * q >= np) continue;
    uint4 y;
    T* ye = reinterpret_cast<T*>(&y);
#pragma unroll
    for (int e = 0; e < EPC; ++e) ye[e] = tile[vt_pos(EPC * q + e) * ROW + d];
    *reinterpret_cast<uint4*>(vt + ((int64_t)kv * D + d) * np + p0 + EPC * q) = y;
  }
}

// Row of K holding group-major position r: K itself is group-major when perm is NULL.
__device__ __forceinline__ int row_of(const int32_t* __restrict__ perm, int h, int n, int r) {
  return perm ? perm[(int64_t)h * n + r] : r;
}

// C^K_b = mean of the group-major key rows of group b in fixed order (fp32), read from K_gm,
// or from K through the key permutation (perm non-NULL) when K_gm is formed later.  Thread t
// sums 8 columns (8 * (t % (D / 8)) ..) over rows start + ph, ph + P, ... with P = 256 /
// (D / 8) row phases (16-byte loads), then the phases are combined in ascending order.
// grid (G, Hkv), block 256.
template <typename T>
__device__ __forceinline__ void load8f(const T* p, float* x);
template <>
__device__ __forceinline__ void load8f<bf16_t>(const bf16_t* p, float* x) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = __uint_as_float(w[e] << 16);
    x[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void load8f<float>(const float* p, float* x) {
  const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void segment_mean_kernel(const T* __restrict__ kgm, const int32_t* __restrict__ perm,
                                                           const int32_t* __restrict__ offsets, int n,
                                                           int G, float* __restrict__ C) {
  constexpr int CQ = D / 8;
  constexpr int P = 256 / CQ;
  __shared__ float red[P][D];
  const int b = blockIdx.x, h = blockIdx.y;
  const int cq = threadIdx.x % CQ, ph = threadIdx.x / CQ;
  const int start = offsets[(int64_t)h * (G + 1) + b], end = offsets[(int64_t)h * (G + 1) + b + 1];
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // eight rows' loads in flight per thread, added in row order (the sum order is unchanged)
  int r = start + ph;
  for (; r + 7 * P < end; r += 8 * P) {
    float x[8][8];
#pragma unroll
    for (int u = 0; u < 8; ++u) load8f<T>(kgm + ((int64_t)h * n + row_of(perm, h, n, r + u * P)) * D + 8 * cq, x[u]);
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += x[u][e];
  }
  for (; r < end; r += P) {
    float x[8];
    load8f<T>(kgm + ((int64_t)h * n + row_of(perm, h, n, r)) * D + 8 * cq, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += x[e];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[ph][8 * cq + e] = acc[e];
  __syncthreads();
  for (int col = threadIdx.x; col < D; col += 256) {
    float tot = 0.f;
    for (int i = 0; i < P; ++i) tot += red[i][col];
    const int cnt = end - start;
    C[((int64_t)h * G + b) * D + col] = cnt > 0 ? tot / (float)cnt : 0.f;
  }
}

// U^(h) = Q^(h) C^K^T * scale for the g query heads of a KV head over a 64-token tile;
// the head sum (fp32, ascending head order) is kept for the direction features, with
// its per-head max |.|.  Lanes run over key groups so U rows are written coalesced.
// grid (ceil(n / 64), Hkv), block 256.
template <typename T, int D>
__global__ __launch_bounds__(256) void resp_u_kernel(const T* __restrict__ q, const float* __restrict__ Ck,
                                                     int n, int g, int Gk, float scale,
                                                     float* __restrict__ U, float* __restrict__ Usum,
                                                     uint32_t* maxbits) {
  __shared__ float cs[kMaxGroups][D + 1];
  __shared__ float qs[64][D];
  __shared__ float red[4];
  const int kv = blockIdx.y;
  const int t0 = blockIdx.x * 64;
  for (int idx = threadIdx.x; idx < Gk * D; idx += 256) {
    int b = idx / D, c = idx % D;
    cs[b][c] = Ck[((int64_t)kv * Gk + b) * D + c];
  }
  const int b = threadIdx.x & 63;
  const int rg = threadIdx.x >> 6;
  float usum[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) usum[i] = 0.f;
  for (int jh = 0; jh < g; ++jh) {
    const int h = kv * g + jh;
    __syncthreads();
    for (int idx = threadIdx.x; idx < 64 * D; idx += 256) {
      int r = idx / D, c = idx % D;
      int t = t0 + r;
      qs[r][c] = t < n ? to_f32(q[((int64_t)h * n + t) * D + c]) : 0.f;
    }
    __syncthreads();
    if (b < Gk) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = rg + 4 * i;
        float acc = 0.f;
        for (int c = 0; c < D; ++c) acc = fmaf(qs[r][c], cs[b][c], acc);
        const float u = acc * scale;
        usum[i] = (jh == 0) ? u : usum[i] + u;
        const int t = t0 + r;
        if (t < n) U[((int64_t)h * n + t) * Gk + b] = u;
      }
    }
  }
  float mx = 0.f;
  if (b < Gk) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int t = t0 + rg + 4 * i;
      if (t < n) {
        mx = fmaxf(mx, fabsf(usum[i]));
        if (Usum) Usum[((int64_t)kv * n + t) * Gk + b] = usum[i];
      }
    }
  }
  mx = wave_max(mx);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    atomicMax(&maxbits[kv], __float_as_uint(m));
  }
}

// All-reduce over the 16 lanes of a DPP row (every lane of the row gets the result).
__device__ __forceinline__ int row16_sum_i32(int v) {
  v += dpp_i32<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp_i32<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp_i32<0x141>(v);   // row_half_mirror
  return v + dpp_i32<0x140>(v);   // row_mirror
}
__device__ __forceinline__ int row16_max_i32(int v) {
  v = max(v, dpp_i32<0xB1>(v));
  v = max(v, dpp_i32<0x4E>(v));
  v = max(v, dpp_i32<0x141>(v));
  return max(v, dpp_i32<0x140>(v));
}

// div_rhaz(127 c, m) for |c| <= m < 2^22: the quotient (254 |c| + m) / (2 m) is at most 127.5;
// its fp32 estimate (operand rounding, a 1-ulp reciprocal and the product: relative error
// below 2^-21) truncates to the floor or one off it, and the exact integer remainder
// corrects that step.
__device__ __forceinline__ int div127_rhaz(int c, int m) {
  const int a = 254 * (c < 0 ? -c : c) + m, b = 2 * m;
  int q = (int)((float)a * __builtin_amdgcn_rcpf((float)b));
  const int r = a - q * b;
  q += (r >= b) ? 1 : (r < 0 ? -1 : 0);
  return c < 0 ? -q : q;
}

// Response-direction features: u = rint(Usum 2^e_U) (e_U: largest e with
// max|Usum| 2^e <= 2^14), c_b = G_K u_b - sum u, x_b = div_rhaz(127 c_b, max|c|).
// Written to the caller's [Hkv][n][G_K] buffer and to a stride-fp copy for the k-means.
// One row per 16 lanes (a DPP row: sum and max without cross-row traffic), each lane
// holding key groups 4 l .. 4 l + 3 (G_K <= 64); every 16 lanes walk four rows, all four
// rows' loads issued before the first is used.  |u| <= 2^14 keeps |c| <= 2^21.
// grid (ceil(n / 64), Hkv), block 256.
__global__ __launch_bounds__(256) void query_features_kernel(const float* __restrict__ Usrc,
                                                             const uint32_t* maxbits, int n, int Gk,
                                                             int fp, int8_t* __restrict__ Xout,
                                                             int8_t* __restrict__ Xpad, int32_t* exps) {
  const int kv = blockIdx.y;
  const int l16 = threadIdx.x & 15, rw = threadIdx.x >> 4, f0 = 4 * l16;
  const int e = pow2_exponent(__uint_as_float(maxbits[kv]), 16384.f);
  if (blockIdx.x == 0 && threadIdx.x == 0) exps[kv * 2 + 1] = e;
  const bool vin = (Gk & 3) == 0 && ((uintptr_t)Usrc & 15) == 0;
  const bool vout = (Gk & 3) == 0 && ((uintptr_t)Xout & 3) == 0;
  float uv[4][4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int i = min(blockIdx.x * 64 + 16 * rr + rw, n - 1);
    const float* src = Usrc + ((int64_t)kv * n + i) * Gk;
    if (vin) {
      const float4 t = f0 < Gk ? *reinterpret_cast<const float4*>(src + f0) : make_float4(0.f, 0.f, 0.f, 0.f);
      uv[rr][0] = t.x; uv[rr][1] = t.y; uv[rr][2] = t.z; uv[rr][3] = t.w;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) uv[rr][j] = f0 + j < Gk ? src[f0 + j] : 0.f;
    }
  }
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int i = blockIdx.x * 64 + 16 * rr + rw;
    int u[4], s = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u[j] = f0 + j < Gk ? (int)rintf(ldexpf(uv[rr][j], e)) : 0;
      s += u[j];
    }
    s = row16_sum_i32(s);
    int c[4], m = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      c[j] = Gk * u[j] - s;
      if (f0 + j < Gk) m = max(m, c[j] < 0 ? -c[j] : c[j]);
    }
    m = row16_max_i32(m);
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int x = (f0 + j < Gk && m > 0) ? div127_rhaz(c[j], m) : 0;
      word |= (uint32_t)(uint8_t)(int8_t)x << (8 * j);
    }
    if (i >= n) continue;
    int8_t* xo = Xout + ((int64_t)kv * n + i) * Gk;
    if (vout) {
      if (f0 < Gk) *reinterpret_cast<uint32_t*>(xo + f0) = word;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (f0 + j < Gk) xo[f0 + j] = (int8_t)(word >> (8 * j));
    }
    // fp is a multiple of four: lanes past G_K store the zero padding
    if (f0 < fp) *reinterpret_cast<uint32_t*>(Xpad + ((int64_t)kv * n + i) * fp + f0) = word;
  }
}

// ---------------------------------------------------------------------------------------
// Semantic partition (ablation paragraph of the summary page of "Partition the Support,
// Reconstruct the Residual": clustering the activations instead of their responses).
// Row i of head kv is x = sum_j X[kv g + j][i] over the g heads of the group (fp32,
// ascending j; g = 1 for keys), quantised as rint(x 2^e) clamped to [-127, 127] with e the
// largest power of two such that max |x| 2^e <= 127 over the head.
// ---------------------------------------------------------------------------------------
template <typename T, int D>
__device__ __forceinline__ float sem_value(const T* __restrict__ x, int n, int g, int kv, int i, int c) {
  float acc = to_f32(x[((int64_t)(kv * g) * n + i) * D + c]);
  for (int j = 1; j < g; ++j) acc = acc + to_f32(x[((int64_t)(kv * g + j) * n + i) * D + c]);
  return acc;
}

// grid (ceil(n * D / 1024), Hkv), block 256: atomic max of |x| (float bits) per head
template <typename T, int D>
__global__ __launch_bounds__(256) void sem_maxabs_kernel(const T* __restrict__ x, int n, int g,
                                                         uint32_t* __restrict__ maxbits) {
  __shared__ float red[4];
  const int kv = blockIdx.y;
  float mx = 0.f;
  for (int u = 0; u < 4; ++u) {
    const int64_t idx = ((int64_t)blockIdx.x * 4 + u) * 256 + threadIdx.x;
    if (idx < (int64_t)n * D) mx = fmaxf(mx, fabsf(sem_value<T, D>(x, n, g, kv, (int)(idx / D), (int)(idx % D))));
  }
  mx = wave_max(mx);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  if (threadIdx.x == 0) atomicMax(&maxbits[kv], __float_as_uint(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]))));
}

// grid (ceil(n * D / 256), Hkv), block 256: int8 features into Xpad [Hkv][n][D] (and Xout
// when given), exponent into exps[kv * 2 + slot], the summed rows into xsum when given
template <typename T, int D>
__global__ __launch_bounds__(256) void sem_quant_kernel(const T* __restrict__ x, int n, int g,
                                                        const uint32_t* __restrict__ maxbits, int slot,
                                                        int8_t* __restrict__ Xout, int8_t* __restrict__ Xpad,
                                                        int32_t* __restrict__ exps, float* __restrict__ xsum) {
  const int kv = blockIdx.y;
  const int e = pow2_exponent(__uint_as_float(maxbits[kv]), 127.f);
  if (blockIdx.x == 0 && threadIdx.x == 0) exps[kv * 2 + slot] = e;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)n * D) return;
  const int i = (int)(idx / D), c = (int)(idx % D);
  const float xv = sem_value<T, D>(x, n, g, kv, i, c);
  if (xsum) xsum[((int64_t)kv * n + i) * D + c] = xv;
  const float v = fminf(fmaxf(rintf(ldexpf(xv, e)), -127.f), 127.f);
  const int8_t q = (int8_t)(int)v;
  Xpad[((int64_t)kv * n + i) * D + c] = q;
  if (Xout) Xout[((int64_t)kv * n + i) * D + c] = q;
}

template <typename T, int D>
static void launch_semantic_features(const T* x, int n, int hkv, int g, uint32_t* maxbits, int slot, int8_t* Xout,
                                     int8_t* Xpad, int32_t* exps, float* xsum, hipStream_t s) {
  const int64_t total = (int64_t)n * D;
  hipLaunchKernelGGL((sem_maxabs_kernel<T, D>), dim3((unsigned)ceil_div(total, 1024), hkv), dim3(256), 0, s, x, n, g,
                     maxbits);
  hipLaunchKernelGGL((sem_quant_kernel<T, D>), dim3((unsigned)ceil_div(total, 256), hkv), dim3(256), 0, s, x, n, g,
                     maxbits, slot, Xout, Xpad, exps, xsum);
}

// ---------------------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------------------
template <int FP>
static void launch_assign(const int8_t* X, int n, int H, int G, const int32_t* C, int32_t* labels,
                          int32_t* sums, hipStream_t s) {
  hipLaunchKernelGGL(kmeans_assign_kernel<FP>, dim3((unsigned)ceil_div(n, 256), H), dim3(256), 0, s,
                     X, n, G, C, labels, sums);
}

// One k-means iteration on the matrix cores (see kmeans_assign_mfma_kernel): the update
// from prev_sums (or none), the assignment, and the sums into `sums` (none: labels only).
struct AssignStep {
  const int32_t* cprev;
  const int32_t* prev_sums;
  int32_t* cout;
  int32_t* sums;
  int32_t* zero_sums;
};

template <int FP>
static void launch_assign_mfma(const int8_t* X, int n, int H, int G, int F, const AssignStep& st, int32_t* labels,
                               hipStream_t s) {
  // at most 512 blocks in all (two 4-wave blocks per CU at two waves per SIMD): one pass
  // over the chip, and few per-block atomic flushes of G * (FP + 1) sums
  const int nchunks = (int)ceil_div(n, kAssignChunk);
  const int per_head = std::max(1, std::min(nchunks, 512 / std::max(H, 1)));
  const int chunks = (int)ceil_div(nchunks, per_head);
  const dim3 grid((unsigned)ceil_div(nchunks, chunks), H);
  if (st.sums != nullptr)
    hipLaunchKernelGGL((kmeans_assign_mfma_kernel<FP, true>), grid, dim3(256), 0, s, X, n, G, F, st.cprev,
                       st.prev_sums, st.cout, chunks, labels, st.sums, st.zero_sums);
  else
    hipLaunchKernelGGL((kmeans_assign_mfma_kernel<FP, false>), grid, dim3(256), 0, s, X, n, G, F, st.cprev,
                       st.prev_sums, st.cout, chunks, labels, st.sums, st.zero_sums);
}

static bool assign_mfma_dispatch(int fp, const int8_t* X, int n, int H, int G, int F, const AssignStep& st,
                                 int32_t* labels, hipStream_t s) {
  switch (fp) {
    case 16: launch_assign_mfma<16>(X, n, H, G, F, st, labels, s); return true;
    case 32: launch_assign_mfma<32>(X, n, H, G, F, st, labels, s); return true;
    case 48: launch_assign_mfma<48>(X, n, H, G, F, st, labels, s); return true;
    case 64: launch_assign_mfma<64>(X, n, H, G, F, st, labels, s); return true;
    case 128: launch_assign_mfma<128>(X, n, H, G, F, st, labels, s); return true;
    default: return false;
  }
}

static bool has_assign_mfma(int fp) { return fp == 16 || fp == 32 || fp == 48 || fp == 64 || fp == 128; }

static void assign_dispatch(int fp, const int8_t* X, int n, int H, int G, const int32_t* C,
                            int32_t* labels, int32_t* sums, hipStream_t s) {
  switch (fp) {
#define SP_FP_CASE(V) case V: launch_assign<V>(X, n, H, G, C, labels, sums, s); break;
    SP_FP_CASE(4) SP_FP_CASE(8) SP_FP_CASE(12) SP_FP_CASE(16) SP_FP_CASE(20) SP_FP_CASE(24)
    SP_FP_CASE(28) SP_FP_CASE(32) SP_FP_CASE(36) SP_FP_CASE(40) SP_FP_CASE(44) SP_FP_CASE(48)
    SP_FP_CASE(52) SP_FP_CASE(56) SP_FP_CASE(60) SP_FP_CASE(64)
#undef SP_FP_CASE
    default: break;
  }
}

// C2: two centroid buffers [H][kMaxGroups][fp]; sums3: three sums buffers [H][kMaxGroups][fp + 1].
void run_kmeans(const int8_t* X, int n, int H, int G, int F, int fp, int iters, int32_t* C2,
                int32_t* sums3, int32_t* labels, int32_t* centroids_out, hipStream_t s) {
  const size_t sums_elems = (size_t)H * kMaxGroups * (fp + 1);
  const size_t c_elems = (size_t)H * kMaxGroups * fp;
  hipLaunchKernelGGL(kmeans_init_kernel, dim3(H), dim3(256), 0, s, X, n, G, fp, C2);
  fill_u32(reinterpret_cast<uint32_t*>(sums3), sums_elems, 0, s);
  if (has_assign_mfma(fp)) {
    // iteration t assigns with C_t (kept in buffer t % 2), forming C_t from the sums of
    // iteration t - 1 (buffer (t - 1) % 3); it accumulates into buffer t % 3 and clears
    // buffer (t + 1) % 3, which iteration t - 1 read and iteration t + 1 fills
    int32_t* Cb[2] = {C2, C2 + c_elems};
    int32_t* Sb[3] = {sums3, sums3 + sums_elems, sums3 + 2 * sums_elems};
    for (int t = 0; t <= iters; ++t) {
      AssignStep st;
      st.cprev = t > 0 ? Cb[(t - 1) & 1] : Cb[0];
      st.prev_sums = t > 0 ? Sb[(t - 1) % 3] : nullptr;
      st.cout = t > 0 ? Cb[t & 1] : nullptr;
      st.sums = t < iters ? Sb[t % 3] : nullptr;
      st.zero_sums = t + 1 < iters ? Sb[(t + 1) % 3] : nullptr;
      assign_mfma_dispatch(fp, X, n, H, G, F, st, labels, s);
    }
    hipLaunchKernelGGL(copy_centroids_kernel, dim3(H), dim3(256), 0, s, Cb[iters & 1], G, F, fp, centroids_out);
    return;
  }
  int32_t* C = C2;
  int32_t* sums[2] = {sums3, sums3 + sums_elems};
  for (int t = 0; t < iters; ++t) {
    assign_dispatch(fp, X, n, H, G, C, labels, sums[t & 1], s);
    hipLaunchKernelGGL(kmeans_update_kernel, dim3(H), dim3(256), 0, s, sums[t & 1], G, F, fp, C,
                       sums[(t + 1) & 1]);
  }
  assign_dispatch(fp, X, n, H, G, C, labels, sums[iters & 1], s);
  hipLaunchKernelGGL(copy_centroids_kernel, dim3(H), dim3(256), 0, s, C, G, F, fp, centroids_out);
}

void run_group_major(const int32_t* labels, int n, int H, int G, int32_t* perm, int32_t* offsets,
                     int32_t* hist, hipStream_t s) {
  const int nchunks = (int)ceil_div(n, kGmChunk);
  hipLaunchKernelGGL(gm_count_kernel, dim3(nchunks, H), dim3(1024), 0, s, labels, n, G, hist);
  hipLaunchKernelGGL(gm_scan_kernel, dim3(H), dim3(64), 0, s, hist, nchunks, G, offsets);
  hipLaunchKernelGGL(gm_scatter_kernel, dim3(nchunks, H), dim3(1024), 0, s, labels, n, hist, perm);
}

void run_gather(const void* src, const int32_t* perm, int n, int hkv, int g, int d, bool bf16,
                void* dst, hipStream_t s) {
  const int row_bytes = d * (bf16 ? 2 : 4);
  const int64_t rows = (int64_t)hkv * n * g;
  const int64_t threads = rows * (row_bytes / 16);
  const dim3 grid((unsigned)ceil_div(threads, 256));
  const uint4* sp = static_cast<const uint4*>(src);
  uint4* dp = static_cast<uint4*>(dst);
  switch (row_bytes) {
    case 128: hipLaunchKernelGGL(gather_rows_kernel<128>, grid, dim3(256), 0, s, sp, perm, n, g, rows, dp); break;
    case 256: hipLaunchKernelGGL(gather_rows_kernel<256>, grid, dim3(256), 0, s, sp, perm, n, g, rows, dp); break;
    case 512: hipLaunchKernelGGL(gather_rows_kernel<512>, grid, dim3(256), 0, s, sp, perm, n, g, rows, dp); break;
    default: break;
  }
}

template <typename T, int D>
static void gather_kv_typed(const Dims& dm, const T* k, const T* v, const sparsepr_partition_t& out, hipStream_t s) {
  run_gather(k, out.key_perm, dm.n, dm.hkv, 1, D, dm.bf16, out.k_gm, s);
  hipLaunchKernelGGL((gather_vt_kernel<T, D>), dim3((unsigned)ceil_div(vt_pad(dm.n), kVtBlock), dm.hkv), dim3(256), 0,
                     s, v, out.key_perm, dm.n, (int)vt_pad(dm.n), static_cast<T*>(out.v_gm));
}

template <typename T, int D>
static void partition_typed(const Dims& dm, const Workspace& wp, const T* q, const T* k, const T* v,
                            const sparsepr_partition_t& out, char* ws, bool defer_kv, hipStream_t s) {
  uint32_t* maxbits = reinterpret_cast<uint32_t*>(ws + wp.maxbits);
  int8_t* xk = reinterpret_cast<int8_t*>(ws + wp.xk);
  int8_t* xq = reinterpret_cast<int8_t*>(ws + wp.xq);
  int32_t* C = reinterpret_cast<int32_t*>(ws + wp.centroids);
  int32_t* sums = reinterpret_cast<int32_t*>(ws + wp.sums);
  // head-summed query responses (g > 1, response partition: the coordinate the query features
  // quantise): the caller's query_coord_sum when given, else scratch.  The semantic partition
  // sums the raw query rows instead (into query_coord_sum) and needs no response sum.
  float* usum = (dm.g > 1 && !dm.semantic)
                    ? (out.query_coord_sum ? out.query_coord_sum : reinterpret_cast<float*>(ws + wp.usum))
                    : nullptr;
  int32_t* gm_hist = reinterpret_cast<int32_t*>(ws + wp.gm_hist);
  const int n = dm.n, hkv = dm.hkv;
  fill_u32(maxbits, (size_t)hkv * 2, 0, s);
  // keys
  if (dm.semantic) {
    launch_semantic_features<T, D>(k, n, hkv, 1, maxbits, 0, nullptr, xk, out.exponents, nullptr, s);
    run_kmeans(xk, n, hkv, dm.gk, D, D, dm.iters, C, sums, out.key_labels, out.key_centroids_int, s);
  } else {
    if (dm.bf16)
      launch_resp_s_mfma(dm, q, k, out.responses_s, maxbits, s);
    else
      hipLaunchKernelGGL((resp_s_kernel<T, D>), dim3((unsigned)ceil_div(n, 256), hkv), dim3(256), 0, s, q, k,
                         n, dm.g, dm.rk, dm.scale, out.responses_s, maxbits);
    hipLaunchKernelGGL(key_features_kernel, dim3((unsigned)ceil_div(n, 256), hkv), dim3(256), 0, s,
                       out.responses_s, maxbits, n, dm.rk, wp.fpk, xk, out.exponents);
    run_kmeans(xk, n, hkv, dm.gk, dm.rk, wp.fpk, dm.iters, C, sums, out.key_labels, out.key_centroids_int, s);
  }
  run_group_major(out.key_labels, n, hkv, dm.gk, out.key_perm, out.key_offsets, gm_hist, s);
  if (defer_kv) {
    hipLaunchKernelGGL((segment_mean_kernel<T, D>), dim3(dm.gk, hkv), dim3(256), 0, s, k, out.key_perm,
                       out.key_offsets, n, dm.gk, out.key_centroids);
  } else {
    gather_kv_typed<T, D>(dm, k, v, out, s);
    hipLaunchKernelGGL((segment_mean_kernel<T, D>), dim3(dm.gk, hkv), dim3(256), 0, s,
                       static_cast<const T*>(out.k_gm), nullptr, out.key_offsets, n, dm.gk, out.key_centroids);
  }
  // queries (the semantic features are formed first: the response kernels below reuse the
  // second max slot)
  if (dm.semantic)
    launch_semantic_features<T, D>(q, n, hkv, dm.g, maxbits + hkv, 1, out.query_features, xq, out.exponents,
                                   dm.g > 1 ? out.query_coord_sum : nullptr, s);
  if (dm.bf16)
    launch_resp_u_mfma(dm, q, out.key_centroids, out.responses_u, usum, maxbits + hkv, s);
  else
    hipLaunchKernelGGL((resp_u_kernel<T, D>), dim3((unsigned)ceil_div(n, 64), hkv), dim3(256), 0, s, q,
                       out.key_centroids, n, dm.g, dm.gk, dm.scale, out.responses_u, usum, maxbits + hkv);
  if (!dm.semantic)
    hipLaunchKernelGGL(query_features_kernel, dim3((unsigned)ceil_div(n, 64), hkv), dim3(256), 0, s,
                       usum ? usum : out.responses_u, maxbits + hkv, n, dm.gk, wp.fpq, out.query_features,
                       xq, out.exponents);
  run_kmeans(xq, n, hkv, dm.gq, dm.fq, wp.fpq, dm.iters, C, sums, out.query_labels, out.query_centroids, s);
  run_group_major(out.query_labels, n, hkv, dm.gq, out.query_perm, out.query_offsets, gm_hist, s);
  run_gather(q, out.query_perm, n, hkv, dm.g, D, dm.bf16, out.q_gm, s);
}

void launch_transpose_v(const Dims& dm, const void* v, void* vt, hipStream_t s) {
  const dim3 grid((unsigned)ceil_div(vt_pad(dm.n), kVtBlock), dm.hkv);
  const int np = (int)vt_pad(dm.n);
  if (dm.bf16) {
    if (dm.d == 128) hipLaunchKernelGGL((gather_vt_kernel<bf16_t, 128>), grid, dim3(256), 0, s, (const bf16_t*)v, nullptr, dm.n, np, (bf16_t*)vt);
    else hipLaunchKernelGGL((gather_vt_kernel<bf16_t, 64>), grid, dim3(256), 0, s, (const bf16_t*)v, nullptr, dm.n, np, (bf16_t*)vt);
  } else {
    if (dm.d == 128) hipLaunchKernelGGL((gather_vt_kernel<float, 128>), grid, dim3(256), 0, s, (const float*)v, nullptr, dm.n, np, (float*)vt);
    else hipLaunchKernelGGL((gather_vt_kernel<float, 64>), grid, dim3(256), 0, s, (const float*)v, nullptr, dm.n, np, (float*)vt);
  }
}

void launch_partition(const Dims& dm, const Workspace& wp, const void* q, const void* k, const void* v,
                      const sparsepr_partition_t& out, char* ws, bool defer_kv, hipStream_t s) {
  if (dm.bf16) {
    if (dm.d == 128)
      partition_typed<bf16_t, 128>(dm, wp, (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, out, ws, defer_kv, s);
    else
      partition_typed<bf16_t, 64>(dm, wp, (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, out, ws, defer_kv, s);
  } else {
    if (dm.d == 128)
      partition_typed<float, 128>(dm, wp, (const float*)q, (const float*)k, (const float*)v, out, ws, defer_kv, s);
    else
      partition_typed<float, 64>(dm, wp, (const float*)q, (const float*)k, (const float*)v, out, ws, defer_kv, s);
  }
}

void launch_gather_kv(const Dims& dm, const void* k, const void* v, const sparsepr_partition_t& part,
                      hipStream_t s) {
  if (dm.bf16) {
    if (dm.d == 128) gather_kv_typed<bf16_t, 128>(dm, (const bf16_t*)k, (const bf16_t*)v, part, s);
    else gather_kv_typed<bf16_t, 64>(dm, (const bf16_t*)k, (const bf16_t*)v, part, s);
  } else {
    if (dm.d == 128) gather_kv_typed<float, 128>(dm, (const float*)k, (const float*)v, part, s);
    else gather_kv_typed<float, 64>(dm, (const float*)k, (const float*)v, part, s);
  }
}

}  // namespace sp
