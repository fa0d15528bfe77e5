// Write-back (summary page of "Partition the Support, Reconstruct the Residual", execution
// paragraph lists write-back among the timed steps; the correction is the
// probe-fit residual reconstruction paragraph's affine fit with its feature-dependent part
// projected on the rank-r subspace): o_hat = o + c0 + (o A) B for every group-major row,
// scattered to token order through the query permutation and cast; then the probe rows
// are overwritten with their exact dense output.
#include "sp_common.hpp"
#include "sp_launch.hpp"

namespace sp {

// grid (ceil(n / 64), Hq), block 256 (4 waves x 16 rows).
template <typename OutT, int D>
__global__ __launch_bounds__(256) void apply_kernel(const float* __restrict__ o_gm, const int32_t* __restrict__ qperm,
                                                    const float* __restrict__ A, const float* __restrict__ B,
                                                    const float* __restrict__ c0, const int32_t* __restrict__ r_eff,
                                                    int n, int g, int rank, OutT* __restrict__ out) {
  __shared__ float As[D][kMaxRank + 1];
  __shared__ float Bs[kMaxRank][D];
  __shared__ float cs[D];
  __shared__ float orow[4][D];
  __shared__ float tk[4][kMaxRank];
  const int h = blockIdx.y, kv = h / g, j = h % g;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int re = r_eff[h];
  for (int idx = tid; idx < D * kMaxRank; idx += 256) {
    const int c = idx / kMaxRank, k = idx % kMaxRank;
    As[c][k] = k < re ? A[((int64_t)h * D + c) * rank + k] : 0.f;
    Bs[k][c % D] = 0.f;
  }
  __syncthreads();
  for (int idx = tid; idx < re * D; idx += 256) Bs[idx / D][idx % D] = B[((int64_t)h * rank) * D + idx];
  for (int c = tid; c < D; c += 256) cs[c] = c0[(int64_t)h * D + c];
  __syncthreads();
  for (int rr = 0; rr < 16; ++rr) {
    const int p = blockIdx.x * 64 + w * 16 + rr;
    const bool valid = p < n;
    if (valid)
      for (int c = l; c < D; c += 64) orow[w][c] = o_gm[(((int64_t)kv * n + p) * g + j) * D + c];
    __syncthreads();
    if (valid) {
      const int k = l & 31, half = l >> 5;
      float t = 0.f;
      for (int c = half * (D / 2); c < (half + 1) * (D / 2); ++c) t = fmaf(orow[w][c], As[c][k], t);
      t += __shfl_xor(t, 32);
      if (half == 0) tk[w][k] = t;
    }
    __syncthreads();
    if (valid) {
      const int64_t tok = qperm[(int64_t)kv * n + p];
      OutT* orow_out = out + ((int64_t)h * n + tok) * D;
      for (int c = l; c < D; c += 64) {
        float v = orow[w][c] + cs[c];
        for (int k = 0; k < re; ++k) v = fmaf(tk[w][k], Bs[k][c], v);
        orow_out[c] = from_f32<OutT>(v);
      }
    }
  }
}

// Probe rows take their exact dense output.  grid Hq, block 256.
template <typename OutT>
__global__ void probe_writeback_kernel(const float* __restrict__ o_dense, const int32_t* __restrict__ ptok, int n,
                                       int g, int M, int D, OutT* __restrict__ out) {
  const int h = blockIdx.x, kv = h / g;
  for (int idx = threadIdx.x; idx < M * D; idx += blockDim.x) {
    const int r = idx / D, c = idx % D;
    out[((int64_t)h * n + ptok[kv * M + r]) * D + c] = from_f32<OutT>(o_dense[((int64_t)h * M + r) * D + c]);
  }
}

template <typename OutT, int D>
static void apply_typed(const Dims& dm, const float* o_gm, const sparsepr_partition_t& part, const sparsepr_fit_t& fit,
                        OutT* o, hipStream_t s) {
  hipLaunchKernelGGL((apply_kernel<OutT, D>), dim3((unsigned)ceil_div(dm.n, 64), dm.hq), dim3(256), 0, s, o_gm,
                     part.query_perm, fit.A, fit.B, fit.c0, fit.r_eff, dm.n, dm.g, dm.r, o);
  hipLaunchKernelGGL(probe_writeback_kernel<OutT>, dim3(dm.hq), dim3(256), 0, s, fit.o_dense, fit.probe_tokens,
                     dm.n, dm.g, dm.m, D, o);
}

void launch_apply(const Dims& dm, const float* o_gm, const sparsepr_partition_t& part, const sparsepr_fit_t& fit,
                  void* o, hipStream_t s) {
  if (dm.bf16) {
    if (dm.d == 128) apply_typed<bf16_t, 128>(dm, o_gm, part, fit, (bf16_t*)o, s);
    else apply_typed<bf16_t, 64>(dm, o_gm, part, fit, (bf16_t*)o, s);
  } else {
    if (dm.d == 128) apply_typed<float, 128>(dm, o_gm, part, fit, (float*)o, s);
    else apply_typed<float, 64>(dm, o_gm, part, fit, (float*)o, s);
  }
}

}  // namespace sp
