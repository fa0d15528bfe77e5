// Support diagnostics (summary page of "Partition the Support, Reconstruct the
// Residual", support paragraph: how many keys one query row needs to keep 90 % of its
// attention mass, and how that grows when several queries share one route).
//
// For every (query head, set of s query tokens) one workgroup:
//  1. scores f = q . k for the s rows against all keys (fp32 from the stored values),
//     written to a per-workgroup slot of the workspace, and each row's maximum;
//  2. per row, the threshold key of its support by a four-pass radix select over the
//     order-preserving 32-bit key of f, from the largest down, with each key weighted
//     by its probability in 2^-40 fixed point relative to the row maximum, m =
//     floor(2^40 exp((f - max) scale)) formed in double precision, summed in 64-bit
//     integers (LDS atomics; lanes of a wave that share a bin are summed first).  The
//     target is min(ceil(mass * sum m), sum m), at least 1, with sum m as a double.
//     Keys above the threshold all belong to the support; of the keys equal to it, the
//     lowest indices are taken until the target is met;
//  3. the support count of each row and the size of the union over the set.
// Every decision is exact integer arithmetic on fixed fp32 scores, so the result does
// not depend on the launch.
#include <cmath>

#include "sp_common.hpp"
#include "sp_launch.hpp"

namespace sp {

constexpr int kSupThreads = 512;
constexpr int kSupWaves = kSupThreads / kWave;

// Larger float -> larger key; +0 and -0 are merged before the key is taken.
__device__ __forceinline__ uint32_t okey(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float from_okey(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}
// floor(2^40 exp((f - fmax) scale)) from the fp32 scores in double precision (the
// difference and the product are the double operations a float64 reference performs)
__device__ __forceinline__ uint64_t mass_fixed(float f, float fmax, double scale) {
  return (uint64_t)ldexp(exp(((double)f - (double)fmax) * scale), 40);
}

template <typename T>
__device__ __forceinline__ void load8(const T* p, float* out);
template <>
__device__ __forceinline__ void load8<bf16_t>(const bf16_t* p, float* out) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    out[2 * e] = __uint_as_float(w[e] << 16);
    out[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float* out) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Adds (m, 1) to bin b of one row's histogram for the participating lanes.  When at
// least 8 lanes share the first participant's bin, those lanes are summed across the
// wave and added once; the others add their own.
__device__ __forceinline__ void hist_add(bool part, int b, uint64_t m, unsigned long long* hm, uint32_t* hc) {
  const uint64_t act = __ballot(part);
  if (act == 0) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int leader = __ffsll((unsigned long long)act) - 1;
  const int lb = __shfl(b, leader);
  const uint64_t same = __ballot(part && b == lb);
  bool own = part;
  if (__popcll(same) >= 8) {
    const bool in = part && b == lb;
    const uint64_t tot = wave_sum_u64(in ? m : 0);
    if (lane == leader) {
      atomicAdd(&hm[lb], (unsigned long long)tot);
      atomicAdd(&hc[lb], (uint32_t)__popcll(same));
    }
    own = part && !in;
  }
  if (own) {
    atomicAdd(&hm[b], (unsigned long long)m);
    atomicAdd(&hc[b], 1u);
  }
}

// grid min(Hq * n_sets, slots), block 512.  q [Hq][n][D], k [Hkv][n][D]; sets
// [Hq][n_sets][S] token indices; scores: S * n floats per workgroup; row_out
// [Hq][n_sets][S]; union_out [Hq][n_sets].
template <typename T, int D>
__global__ __launch_bounds__(kSupThreads) void support_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                              const int32_t* __restrict__ sets, int n, int hq, int g,
                                                              int n_sets, int S, double c, double mass,
                                                              float* __restrict__ scratch, int32_t* __restrict__ row_out,
                                                              int32_t* __restrict__ union_out) {
  __shared__ __attribute__((aligned(16))) float qs[kSupportMaxSet][D];
  __shared__ unsigned long long hm[kSupportMaxSet][256];
  __shared__ uint32_t hc[kSupportMaxSet][256];
  __shared__ float wmax[kSupWaves][kSupportMaxSet];
  __shared__ float rmax[kSupportMaxSet];
  __shared__ int tok[kSupportMaxSet];
  __shared__ uint32_t prefix[kSupportMaxSet], above_c[kSupportMaxSet], tie_c[kSupportMaxSet];
  __shared__ int cut[kSupportMaxSet];
  __shared__ unsigned long long above_m[kSupportMaxSet], target[kSupportMaxSet];
  __shared__ uint32_t wcnt[kSupWaves];

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  float* sc = scratch + (size_t)blockIdx.x * (size_t)S * (size_t)n;
  const int64_t items = (int64_t)hq * n_sets;
  for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
    const int h = (int)(item / n_sets), kv = h / g;
    __syncthreads();
    if (tid < S) {
      const int t = sets[item * S + tid];
      tok[tid] = (t >= 0 && t < n) ? t : -1;
    }
    __syncthreads();
    for (int i = tid; i < S * D; i += kSupThreads) {
      const int r = i / D, e = i % D;
      qs[r][e] = tok[r] >= 0 ? to_f32(q[((int64_t)h * n + tok[r]) * D + e]) : 0.f;
    }
    __syncthreads();

    // 1. scores and row maxima
    float mx[kSupportMaxSet];
#pragma unroll
    for (int r = 0; r < kSupportMaxSet; ++r) mx[r] = -INFINITY;
    const T* kb = k + (int64_t)kv * n * D;
    for (int j = tid; j < n; j += kSupThreads) {
      float acc[kSupportMaxSet];
#pragma unroll
      for (int r = 0; r < kSupportMaxSet; ++r) acc[r] = 0.f;
      for (int e0 = 0; e0 < D; e0 += 8) {
        float kf[8];
        load8<T>(kb + (int64_t)j * D + e0, kf);
#pragma unroll
        for (int r = 0; r < kSupportMaxSet; ++r) {
          if (r < S) {
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[r] = fmaf(qs[r][e0 + e], kf[e], acc[r]);
          }
        }
      }
#pragma unroll
      for (int r = 0; r < kSupportMaxSet; ++r) {
        if (r < S) {
          const float f = acc[r] + 0.f;
          sc[(size_t)r * n + j] = f;
          mx[r] = fmaxf(mx[r], f);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < kSupportMaxSet; ++r) {
      const float v = wave_max(mx[r]);
      if (lane == 0 && r < S) wmax[wave][r] = v;
    }
    __syncthreads();
    if (tid < S) {
      float v = wmax[0][tid];
      for (int w = 1; w < kSupWaves; ++w) v = fmaxf(v, wmax[w][tid]);
      rmax[tid] = v;
      prefix[tid] = 0;
      above_m[tid] = 0;
      above_c[tid] = 0;
    }

    // 2. radix select, one byte of the key per pass from the top
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      for (int i = tid; i < S * 256; i += kSupThreads) {
        hm[i / 256][i % 256] = 0;
        hc[i / 256][i % 256] = 0;
      }
      __syncthreads();
      for (int r = 0; r < S; ++r) {
        if (tok[r] < 0) continue;
        const float fm = rmax[r];
        const uint32_t pre = prefix[r];
        for (int j0 = 0; j0 < n; j0 += kSupThreads) {
          const int j = j0 + tid;
          bool part = false;
          int b = 0;
          uint64_t m = 0;
          if (j < n) {
            const float f = sc[(size_t)r * n + j];
            const uint32_t u = okey(f);
            part = pass == 0 || (u >> (shift + 8)) == pre;
            b = (u >> shift) & 255;
            m = mass_fixed(f, fm, c);
          }
          hist_add(part, b, m, hm[r], hc[r]);
        }
      }
      __syncthreads();
      // one wave per row: lane l holds bins 255-4l .. 252-4l, scanned from the top
      for (int r = wave; r < S; r += kSupWaves) {
        if (tok[r] < 0) continue;
        uint64_t bm[4];
        uint32_t bc[4];
        uint64_t lm = 0;
        uint32_t lc = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bm[e] = hm[r][255 - 4 * lane - e];
          bc[e] = hc[r][255 - 4 * lane - e];
          lm += bm[e];
          lc += bc[e];
        }
        uint64_t tgt;
        if (pass == 0) {
          const uint64_t total = wave_sum_u64(lm);
          const double want = ceil((double)total * mass);
          tgt = want >= (double)total ? total : (uint64_t)want;
          if (tgt == 0) tgt = 1;
          if (lane == 0) target[r] = tgt;
        } else {
          tgt = target[r];
        }
        const uint64_t base_m = above_m[r];
        uint64_t incl = lm;
        uint32_t incl_c = lc;
        for (int o = 1; o < kWave; o <<= 1) {
          const uint64_t vm = __shfl_up(incl, o);
          const uint32_t vc = __shfl_up(incl_c, o);
          if (lane >= o) { incl += vm; incl_c += vc; }
        }
        const uint64_t hit = __ballot(base_m + incl >= tgt);
        const int first = hit ? __ffsll((unsigned long long)hit) - 1 : kWave - 1;
        if (lane == first) {
          uint64_t em = base_m + incl - lm;
          uint32_t ec = above_c[r] + incl_c - lc;
          int e = 0;
          for (; e < 3; ++e) {
            if (em + bm[e] >= tgt) break;
            em += bm[e];
            ec += bc[e];
          }
          above_m[r] = em;
          above_c[r] = ec;
          prefix[r] = (prefix[r] << 8) | (uint32_t)(255 - 4 * lane - e);
          tie_c[r] = bc[e];
        }
      }
      __syncthreads();
    }

    // ties at the threshold: the lowest indices are taken until the target is met
    for (int r = wave; r < S; r += kSupWaves) {
      if (tok[r] < 0) continue;
      const uint32_t us = prefix[r];
      const uint64_t ms = mass_fixed(from_okey(us), rmax[r], c);
      const uint64_t rest = target[r] - above_m[r];
      uint32_t need = ms ? (uint32_t)((rest + ms - 1) / ms) : tie_c[r];
      if (need > tie_c[r]) need = tie_c[r];
      if (need == 0) need = 1;
      int cj = n;
      if (need < tie_c[r]) {
        uint32_t seen = 0;
        for (int j0 = 0; j0 < n; j0 += kWave) {
          const int j = j0 + lane;
          const bool t = j < n && okey(sc[(size_t)r * n + j]) == us;
          uint64_t bal = __ballot(t);
          const uint32_t cnt = (uint32_t)__popcll(bal);
          if (seen + cnt >= need) {
            for (uint32_t skip = need - seen - 1; skip > 0; --skip) bal &= bal - 1;
            cj = j0 + __ffsll((unsigned long long)bal) - 1;
            break;
          }
          seen += cnt;
        }
      }
      if (lane == 0) {
        cut[r] = cj;
        above_c[r] += need;
      }
    }
    __syncthreads();

    // 3. union of the supports over the set
    uint32_t cnt = 0;
    for (int j = tid; j < n; j += kSupThreads) {
      bool in = false;
      for (int r = 0; r < S; ++r) {
        if (tok[r] < 0) continue;
        const uint32_t u = okey(sc[(size_t)r * n + j]);
        in |= u > prefix[r] || (u == prefix[r] && j <= cut[r]);
      }
      cnt += in;
    }
    for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o);
    if (lane == 0) wcnt[wave] = cnt;
    __syncthreads();
    if (tid == 0) {
      uint32_t u = 0;
      for (int w = 0; w < kSupWaves; ++w) u += wcnt[w];
      union_out[item] = (int32_t)u;
    }
    if (tid < S) row_out[item * S + tid] = tok[tid] >= 0 ? (int32_t)above_c[tid] : -1;
  }
}

size_t support_workspace_bytes(const Dims& dm, int n_sets, int set_size) {
  const int64_t items = (int64_t)dm.hq * n_sets;
  const int64_t slots = items < kSupportSlots ? items : kSupportSlots;
  return (size_t)slots * set_size * dm.n * sizeof(float);
}

void launch_support(const Dims& dm, const void* q, const void* k, const int32_t* sets, int n_sets, int set_size,
                    double mass, int32_t* row_out, int32_t* union_out, void* ws, hipStream_t s) {
  const int64_t items = (int64_t)dm.hq * n_sets;
  if (items == 0) return;
  const int grid = (int)(items < kSupportSlots ? items : kSupportSlots);
  const double c = (double)dm.scale;
  float* sc = static_cast<float*>(ws);
#define SUP_LAUNCH(T, DD)                                                                                      \
  hipLaunchKernelGGL((support_kernel<T, DD>), dim3(grid), dim3(kSupThreads), 0, s, static_cast<const T*>(q), \
                     static_cast<const T*>(k), sets, dm.n, dm.hq, dm.g, n_sets, set_size, c, mass, sc, row_out,  \
                     union_out)
  if (dm.bf16) {
    if (dm.d == 128) SUP_LAUNCH(bf16_t, 128); else SUP_LAUNCH(bf16_t, 64);
  } else {
    if (dm.d == 128) SUP_LAUNCH(float, 128); else SUP_LAUNCH(float, 64);
  }
#undef SUP_LAUNCH
}

}  // namespace sp
