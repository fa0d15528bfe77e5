// Residual diagnostics (summary page of "Partition the Support, Reconstruct the Residual",
// partition paragraph: the share of the hard-drop residual that is an affine function of
// the sparse output, and the energy orthogonal to it).  Over every row of each query
// head: R = O_dense - O_sparse and the ordinary least-squares fit R ~ c + O_sparse W.
//
//  1. dense attention (fp32, token order) and the block-sparse attention (fp32,
//     group-major) into the workspace, with the library's attention kernels;
//  2. diag_gram_kernel: M = X^T [X | R] with X = [O_sparse | 1] and T = ||R||_F^2, fp32
//     partial sums over row ranges (rows staged in LDS, 4 x 4 register tiles);
//  3. diag_solve_kernel: the partials summed in fp64, G = X^T X (with a 1e-9 relative
//     diagonal guard) Cholesky-factored in LDS, W = G^-1 X^T R column by column, then
//     ||R - X W||^2 = T - <W, X^T R>, ||R - mean R||^2 = T - ||sum R||^2 / n.
#include <cmath>

#include "sp_common.hpp"
#include "sp_launch.hpp"

namespace sp {

constexpr int kDiagBlocks = 16;   // row ranges per query head
constexpr int kDiagRows = 32;     // rows staged per LDS pass

template <int D>
struct DiagCfg {
  static constexpr int I = D + 1;             // columns of X (O_sparse and the constant)
  static constexpr int J = 2 * D + 1;         // columns of [X | R]
  static constexpr int JP = (J + 3) / 4 * 4;  // padded row of the LDS stage
  static constexpr int TI = (I + 3) / 4, TJ = JP / 4;
  static constexpr int TILES = TI * TJ;
  static constexpr int TPT = (TILES + 255) / 256;   // 4 x 4 tiles per thread
  static constexpr int PART = TI * 4 * JP + 1;      // floats per partial (M padded, then T)
};

// grid (kDiagBlocks, Hq), block 256.  o_d [Hq][n][D] token order; o_gm [Hkv][n][g][D]
// group-major; qperm [Hkv][n].  part [Hq][kDiagBlocks][PART].
template <int D>
__global__ __launch_bounds__(256) void diag_gram_kernel(const float* __restrict__ o_d, const float* __restrict__ o_gm,
                                                        const int32_t* __restrict__ qperm, int n, int g,
                                                        float* __restrict__ part) {
  using C = DiagCfg<D>;
  __shared__ __attribute__((aligned(16))) float zs[kDiagRows][C::JP];
  const int h = blockIdx.y, kv = h / g, j = h % g, tid = threadIdx.x;
  const int rows_per = (int)ceil_div(n, kDiagBlocks);
  const int p0 = blockIdx.x * rows_per, p1 = min(n, p0 + rows_per);
  float acc[C::TPT][16];
#pragma unroll
  for (int t = 0; t < C::TPT; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[t][e] = 0.f;
  float tacc = 0.f;
  for (int b0 = p0; b0 < p1; b0 += kDiagRows) {
    __syncthreads();
    for (int idx = tid; idx < kDiagRows * C::JP; idx += 256) {
      const int r = idx / C::JP, c = idx % C::JP, p = b0 + r;
      float z = 0.f;
      if (p < p1 && c < C::J) {
        const float xs = c < D ? o_gm[(((int64_t)kv * n + p) * g + j) * D + c] : 1.f;
        if (c <= D) {
          z = xs;
        } else {
          const int cc = c - D - 1;
          const int64_t tok = qperm[(int64_t)kv * n + p];
          z = o_d[((int64_t)h * n + tok) * D + cc] - o_gm[(((int64_t)kv * n + p) * g + j) * D + cc];
        }
      }
      zs[r][c] = z;
    }
    __syncthreads();
    const int rn = min(kDiagRows, p1 - b0);
    for (int r = 0; r < rn; ++r) {
#pragma unroll
      for (int t = 0; t < C::TPT; ++t) {
        const int tile = tid + 256 * t;
        if (tile < C::TILES) {
          const int ti = tile / C::TJ, tj = tile % C::TJ;
          const float4 a = *reinterpret_cast<const float4*>(&zs[r][4 * ti]);
          const float4 b = *reinterpret_cast<const float4*>(&zs[r][4 * tj]);
          const float av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int w = 0; w < 4; ++w) acc[t][4 * u + w] = fmaf(av[u], bv[w], acc[t][4 * u + w]);
        }
      }
      if (tid < D) {
        const float x = zs[r][D + 1 + tid];
        tacc = fmaf(x, x, tacc);
      }
    }
  }
  float* out = part + ((int64_t)h * kDiagBlocks + blockIdx.x) * C::PART;
#pragma unroll
  for (int t = 0; t < C::TPT; ++t) {
    const int tile = tid + 256 * t;
    if (tile < C::TILES) {
      const int ti = tile / C::TJ, tj = tile % C::TJ;
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int w = 0; w < 4; ++w) out[(4 * ti + u) * C::JP + 4 * tj + w] = acc[t][4 * u + w];
    }
  }
  // T: wave sums of the per-column squares, then one add per wave
  float tv = tid < D ? tacc : 0.f;
  for (int o = 32; o > 0; o >>= 1) tv += __shfl_xor(tv, o);
  __shared__ float tred[4];
  if ((tid & 63) == 0) tred[tid >> 6] = tv;
  __syncthreads();
  if (tid == 0) out[C::PART - 1] = tred[0] + tred[1] + tred[2] + tred[3];
}

// grid Hq, block 256.  scratch [Hq][I][D] doubles (X^T R, then W).  out [Hq][4] doubles.
template <int D>
__global__ __launch_bounds__(256) void diag_solve_kernel(const float* __restrict__ part, int n,
                                                         double* __restrict__ scratch, double* __restrict__ out) {
  using C = DiagCfg<D>;
  constexpr int I = C::I;
  __shared__ double L[I * (I + 1) / 2];   // packed lower triangle, row i at i (i + 1) / 2
  __shared__ double red[256];
  __shared__ double tsum;
  const int h = blockIdx.x, tid = threadIdx.x;
  const float* ph = part + (int64_t)h * kDiagBlocks * C::PART;
  double* XR = scratch + (int64_t)h * I * D;
  // 1. fp64 sums of the partials
  for (int idx = tid; idx < I * I; idx += 256) {
    const int r = idx / I, c = idx % I;
    if (c > r) continue;
    double s = 0.0;
    for (int b = 0; b < kDiagBlocks; ++b) s += (double)ph[(int64_t)b * C::PART + r * C::JP + c];
    L[r * (r + 1) / 2 + c] = s;
  }
  for (int idx = tid; idx < I * D; idx += 256) {
    const int r = idx / D, c = idx % D;
    double s = 0.0;
    for (int b = 0; b < kDiagBlocks; ++b) s += (double)ph[(int64_t)b * C::PART + r * C::JP + I + c];
    XR[idx] = s;
  }
  if (tid == 0) {
    double s = 0.0;
    for (int b = 0; b < kDiagBlocks; ++b) s += (double)ph[(int64_t)b * C::PART + C::PART - 1];
    tsum = s;
  }
  __syncthreads();
  // 2. guard the diagonal, then Cholesky G = L L^T in place
  if (tid == 0) {
    double tr = 0.0;
    for (int i = 0; i < I; ++i) tr += L[i * (i + 1) / 2 + i];
    red[0] = 1e-9 * tr / I;
  }
  __syncthreads();
  for (int i = tid; i < I; i += 256) L[i * (i + 1) / 2 + i] += red[0];
  __syncthreads();
  for (int k = 0; k < I; ++k) {
    if (tid == 0) L[k * (k + 1) / 2 + k] = sqrt(L[k * (k + 1) / 2 + k]);
    __syncthreads();
    for (int i = k + 1 + tid; i < I; i += 256) L[i * (i + 1) / 2 + k] /= L[k * (k + 1) / 2 + k];
    __syncthreads();
    const int rem = I - k - 1;
    for (int idx = tid; idx < rem * rem; idx += 256) {
      const int i = k + 1 + idx / rem, jj = k + 1 + idx % rem;
      if (jj <= i) L[i * (i + 1) / 2 + jj] -= L[i * (i + 1) / 2 + k] * L[jj * (jj + 1) / 2 + k];
    }
    __syncthreads();
  }
  // 3. W = G^-1 X^T R (one column per thread), <W, X^T R> and ||sum R||^2
  double wdot = 0.0, sdot = 0.0;
  for (int c = tid; c < D; c += 256) {
    double y[I];
    for (int i = 0; i < I; ++i) {
      double s = XR[i * D + c];
      for (int k = 0; k < i; ++k) s -= L[i * (i + 1) / 2 + k] * y[k];
      y[i] = s / L[i * (i + 1) / 2 + i];
    }
    for (int i = I - 1; i >= 0; --i) {
      double s = y[i];
      for (int k = i + 1; k < I; ++k) s -= L[k * (k + 1) / 2 + i] * y[k];
      y[i] = s / L[i * (i + 1) / 2 + i];
    }
    for (int i = 0; i < I; ++i) wdot += y[i] * XR[i * D + c];
    const double sr = XR[(I - 1) * D + c];   // the constant column: sum over rows of R
    sdot += sr * sr;
  }
  red[tid] = wdot;
  __syncthreads();
  for (int s2 = 128; s2 > 0; s2 >>= 1) { if (tid < s2) red[tid] += red[tid + s2]; __syncthreads(); }
  const double wsum = red[0];
  __syncthreads();
  red[tid] = sdot;
  __syncthreads();
  for (int s2 = 128; s2 > 0; s2 >>= 1) { if (tid < s2) red[tid] += red[tid + s2]; __syncthreads(); }
  if (tid == 0) {
    const double tot = tsum, cen = tsum - red[0] / (double)n, orth = fmax(tsum - wsum, 0.0);
    out[h * 4 + 0] = tot;
    out[h * 4 + 1] = cen;
    out[h * 4 + 2] = orth;
    out[h * 4 + 3] = cen > 0.0 ? 1.0 - orth / cen : 0.0;
  }
}

DiagWorkspace plan_diagnostics(const Dims& dm) {
  DiagWorkspace w{};
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t rows = (size_t)dm.hq * dm.n * dm.d;
  const int I = dm.d + 1, JP = (2 * dm.d + 1 + 3) / 4 * 4, TI = (I + 3) / 4;
  const size_t part = (size_t)TI * 4 * JP + 1;
  size_t o = 0;
  w.o_dense = o; o = up(o + rows * 4);
  w.o_gm = o; o = up(o + rows * 4);
  w.vt = o; o = up(o + (size_t)dm.hkv * dm.d * vt_pad(dm.n) * (dm.bf16 ? 2 : 4));
  w.part = o; o = up(o + (size_t)dm.hq * kDiagBlocks * part * 4);
  w.scratch = o; o = up(o + (size_t)dm.hq * I * dm.d * 8);
  w.total = o;
  return w;
}

void launch_diagnostics(const Dims& dm, const DiagWorkspace& w, AttnArgs dense, AttnArgs sparse,
                        const int32_t* qperm, double* out, char* ws, hipStream_t s) {
  float* od = reinterpret_cast<float*>(ws + w.o_dense);
  float* ogm = reinterpret_cast<float*>(ws + w.o_gm);
  float* part = reinterpret_cast<float*>(ws + w.part);
  double* scratch = reinterpret_cast<double*>(ws + w.scratch);
  dense.o = od;
  launch_attention(dm, dense, false, s);
  sparse.o = ogm;
  launch_attention(dm, sparse, false, s);
  if (dm.d == 128) {
    hipLaunchKernelGGL(diag_gram_kernel<128>, dim3(kDiagBlocks, dm.hq), dim3(256), 0, s, od, ogm, qperm, dm.n, dm.g,
                       part);
    hipLaunchKernelGGL(diag_solve_kernel<128>, dim3(dm.hq), dim3(256), 0, s, part, dm.n, scratch, out);
  } else {
    hipLaunchKernelGGL(diag_gram_kernel<64>, dim3(kDiagBlocks, dm.hq), dim3(256), 0, s, od, ogm, qperm, dm.n, dm.g,
                       part);
    hipLaunchKernelGGL(diag_solve_kernel<64>, dim3(dm.hq), dim3(256), 0, s, part, dm.n, scratch, out);
  }
}

}  // namespace sp
