// Matrix-core response GEMMs of the response-coupled partition (summary page of
// "Partition the Support, Reconstruct the Residual", response-coupled partition
// paragraph) for bf16 inputs:
//   S = Q_s K^T * scale   (r_k sampled query rows against every key; bf16 products are
//                          exact, fp32 accumulation)
//   U = Q C^T * scale     (every query row against the G_K key centroids; the fp32
//                          centroids are split as C = C_hi + C_lo in bf16 so U keeps
//                          close to fp32 accuracy), plus the fp32 head sum over the KV
//                          head's query heads (ascending order) and its max |.|.
// Layouts follow MFMA 32x32x16 bf16: A[i][k] in lane (i = l % 32, k = 8 (l / 32) + e),
// B[k][j] in lane (j = l % 32, same k), D[i][j] in lane (j = l % 32) register r with
// i = 8 (r / 4) + 4 (l / 32) + r % 4.
#include "sp_common.hpp"
#include "sp_launch.hpp"

namespace sp {

typedef __bf16 pbf16x8_t __attribute__((ext_vector_type(8)));
typedef float pf32x16_t __attribute__((ext_vector_type(16)));

// Row tiles of 128 per block of the two response kernels (the staged operand is shared by
// all of them).
constexpr int kRespTiles = 8;

// S: one wave = 32 keys; D[sample][key] so lanes run over consecutive keys.
// grid (ceil(n / (128 kRespTiles)), Hkv), block 256.
template <int D>
__global__ __launch_bounds__(256) void resp_s_mfma_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                          int n, int g, int rk, float scale, float* __restrict__ S,
                                                          uint32_t* maxbits) {
  constexpr int QROW = D + 8;
  __shared__ __attribute__((aligned(16))) bf16_t qs[kMaxFeat * QROW];
  __shared__ float red[4];
  const int kv = blockIdx.y;
  for (int idx = threadIdx.x; idx < kMaxFeat * (D / 8); idx += 256) {
    const int s = idx / (D / 8), c8 = idx % (D / 8);
    uint4 v = make_uint4(0, 0, 0, 0);
    if (s < rk) {
      const int64_t tok = ((int64_t)(2 * s + 1) * n) / (2 * rk);
      const int h = kv * g + (s % g);
      v = *reinterpret_cast<const uint4*>(q + ((int64_t)h * n + tok) * D + 8 * c8);
    }
    *reinterpret_cast<uint4*>(qs + s * QROW + 8 * c8) = v;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, l32 = lane & 31, hf = lane >> 5;
  float mx = 0.f;
  for (int t = 0; t < kRespTiles; ++t) {
    const int tile = blockIdx.x * kRespTiles + t;
    if (tile * 128 >= n) break;
    const int key = tile * 128 + 32 * w + l32;
    const bool kval = key < n;
    pbf16x8_t kreg[D / 16];
    const bf16_t* kr = k + ((int64_t)kv * n + (kval ? key : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      uint4 x = kval ? *reinterpret_cast<const uint4*>(kr + 16 * kk + 8 * hf) : make_uint4(0, 0, 0, 0);
      kreg[kk] = __builtin_bit_cast(pbf16x8_t, x);
    }
    const int nsb = (rk + 31) / 32;
    for (int sb = 0; sb < nsb; ++sb) {
      pf32x16_t acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
      const bf16_t* qrow = qs + (32 * sb + l32) * QROW + 8 * hf;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        pbf16x8_t a = *reinterpret_cast<const pbf16x8_t*>(qrow + 16 * kk);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kreg[kk], acc, 0, 0, 0);
      }
      if (kval) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int s = 32 * sb + 8 * (r >> 2) + 4 * hf + (r & 3);
          if (s < rk) {
            const float v = acc[r] * scale;
            S[((int64_t)kv * rk + s) * n + key] = v;
            mx = fmaxf(mx, fabsf(v));
          }
        }
      }
    }
  }
  mx = wave_max(mx);
  if (lane == 0) red[w] = mx;
  __syncthreads();
  if (threadIdx.x == 0) atomicMax(&maxbits[kv], __float_as_uint(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]))));
}

// U: one wave = 32 query rows (A = Q rows from global), B = C^T split in hi / lo bf16
// parts from LDS, groups padded to multiples of 32 with zero centroids.
// grid (ceil(n / (128 kRespTiles)), Hkv), block 256.
template <int D>
__global__ __launch_bounds__(256) void resp_u_mfma_kernel(const bf16_t* __restrict__ q, const float* __restrict__ Ck,
                                                          int n, int g, int Gk, float scale, float* __restrict__ U,
                                                          float* __restrict__ Usum, uint32_t* maxbits) {
  constexpr int CROW = D + 8;
  __shared__ __attribute__((aligned(16))) bf16_t chi[kMaxGroups * CROW];
  __shared__ __attribute__((aligned(16))) bf16_t clo[kMaxGroups * CROW];
  __shared__ float red[4];
  const int kv = blockIdx.y;
  const int ngb = (Gk + 31) / 32;
  for (int idx = threadIdx.x; idx < 32 * ngb * D; idx += 256) {
    const int b = idx / D, c = idx % D;
    const float x = b < Gk ? Ck[((int64_t)kv * Gk + b) * D + c] : 0.f;
    const bf16_t hi = f32_to_bf16(x);
    chi[b * CROW + c] = hi;
    clo[b * CROW + c] = f32_to_bf16(x - bf16_to_f32(hi));
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, l32 = lane & 31, hf = lane >> 5;
  float mx = 0.f;
  for (int t = 0; t < kRespTiles; ++t) {
    const int tile = blockIdx.x * kRespTiles + t;
    if (tile * 128 >= n) break;
    const int row0 = tile * 128 + 32 * w;
    pf32x16_t usum[2];
    for (int jh = 0; jh < g; ++jh) {
      const int h = kv * g + jh;
      const int qrow = row0 + l32;
      const bool qv = qrow < n;
      pbf16x8_t qa[D / 16];
      const bf16_t* qr = q + ((int64_t)h * n + (qv ? qrow : 0)) * D;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        uint4 x = qv ? *reinterpret_cast<const uint4*>(qr + 16 * kk + 8 * hf) : make_uint4(0, 0, 0, 0);
        qa[kk] = __builtin_bit_cast(pbf16x8_t, x);
      }
      // the 32-group blocks' accumulation chains run side by side (same order within each)
      pf32x16_t acc[2];
#pragma unroll
      for (int gb = 0; gb < 2; ++gb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[gb][r] = 0.f;
      if (ngb == 2) {
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
          for (int gb = 0; gb < 2; ++gb) {
            const bf16_t* ch = chi + (32 * gb + l32) * CROW + 8 * hf;
            const bf16_t* cl = clo + (32 * gb + l32) * CROW + 8 * hf;
            acc[gb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[kk], *reinterpret_cast<const pbf16x8_t*>(ch + 16 * kk),
                                                              acc[gb], 0, 0, 0);
            acc[gb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[kk], *reinterpret_cast<const pbf16x8_t*>(cl + 16 * kk),
                                                              acc[gb], 0, 0, 0);
          }
      } else {
        const bf16_t* ch = chi + l32 * CROW + 8 * hf;
        const bf16_t* cl = clo + l32 * CROW + 8 * hf;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
          acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[kk], *reinterpret_cast<const pbf16x8_t*>(ch + 16 * kk),
                                                           acc[0], 0, 0, 0);
          acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[kk], *reinterpret_cast<const pbf16x8_t*>(cl + 16 * kk),
                                                           acc[0], 0, 0, 0);
        }
      }
#pragma unroll
      for (int gb = 0; gb < 2; ++gb) {
        if (gb >= ngb) break;
        const int b = 32 * gb + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = row0 + 8 * (r >> 2) + 4 * hf + (r & 3);
          const float u = acc[gb][r] * scale;
          usum[gb][r] = (jh == 0) ? u : usum[gb][r] + u;
          if (row < n && b < Gk) U[((int64_t)h * n + row) * Gk + b] = u;
        }
        if (jh == g - 1) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = row0 + 8 * (r >> 2) + 4 * hf + (r & 3);
            if (row < n && b < Gk) {
              mx = fmaxf(mx, fabsf(usum[gb][r]));
              if (Usum) Usum[((int64_t)kv * n + row) * Gk + b] = usum[gb][r];
            }
          }
        }
      }
    }
  }
  mx = wave_max(mx);
  if (lane == 0) red[w] = mx;
  __syncthreads();
  if (threadIdx.x == 0) atomicMax(&maxbits[kv], __float_as_uint(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]))));
}

void launch_resp_s_mfma(const Dims& dm, const void* q, const void* k, float* S, uint32_t* maxbits, hipStream_t s) {
  const dim3 grid((unsigned)ceil_div(dm.n, 128 * kRespTiles), dm.hkv);
  if (dm.d == 128)
    hipLaunchKernelGGL(resp_s_mfma_kernel<128>, grid, dim3(256), 0, s, (const bf16_t*)q, (const bf16_t*)k, dm.n, dm.g,
                       dm.rk, dm.scale, S, maxbits);
  else
    hipLaunchKernelGGL(resp_s_mfma_kernel<64>, grid, dim3(256), 0, s, (const bf16_t*)q, (const bf16_t*)k, dm.n, dm.g,
                       dm.rk, dm.scale, S, maxbits);
}

void launch_resp_u_mfma(const Dims& dm, const void* q, const float* Ck, float* U, float* Usum, uint32_t* maxbits,
                        hipStream_t s) {
  const dim3 grid((unsigned)ceil_div(dm.n, 128 * kRespTiles), dm.hkv);
  if (dm.d == 128)
    hipLaunchKernelGGL(resp_u_mfma_kernel<128>, grid, dim3(256), 0, s, (const bf16_t*)q, Ck, dm.n, dm.g, dm.gk,
                       dm.scale, U, Usum, maxbits);
  else
    hipLaunchKernelGGL(resp_u_mfma_kernel<64>, grid, dim3(256), 0, s, (const bf16_t*)q, Ck, dm.n, dm.g, dm.gk,
                       dm.scale, U, Usum, maxbits);
}

}  // namespace sp
