// Write-back (summary page of "Partition the Support, Reconstruct the Residual", execution
// paragraph lists write-back among the timed steps; the correction is the
// probe-fit residual reconstruction paragraph's affine fit with its feature-dependent part
// projected on the rank-r subspace): o_hat = o + c0 + (o A) B for every group-major row,
// scattered to token order through the query permutation and cast; then the probe rows
// are overwritten with their exact dense output.
#include "sp_common.hpp"
#include "sp_launch.hpp"

namespace sp {

// One block = 64 group-major rows of one query head.  The rows are staged in LDS, the
// rank-r coordinates T = O A are a 64 x r product, then o + c0 + T B is written to the
// token-order rows (4 threads per row, 16-byte stores).  RC bounds the correction rank
// (32, or 64 for the unprojected ridge); `rank` is the leading dimension of A and B.
// grid (ceil(n / 64), Hq), block 256.
template <typename OutT, int D, int RC>
__global__ __launch_bounds__(256) void apply_kernel(const float* __restrict__ o_gm, const int32_t* __restrict__ qperm,
                                                    const float* __restrict__ A, const float* __restrict__ B,
                                                    const float* __restrict__ c0, const int32_t* __restrict__ r_eff,
                                                    int n, int g, int rank, OutT* __restrict__ out) {
  constexpr int R = 64;
  constexpr int TPT = RC / 4;   // rank coordinates per thread
  __shared__ float Os[R][D + 4];
  __shared__ float As[D][RC];
  __shared__ float Bs[RC][D];
  __shared__ float Ts[R][RC + 1];
  __shared__ float cs[D];
  const int h = blockIdx.y, kv = h / g, j = h % g;
  const int tid = threadIdx.x;
  const int p0 = blockIdx.x * R;
  const int re = min(r_eff[h], min(rank, RC));
  for (int idx = tid; idx < D * RC; idx += 256) {
    const int c = idx / RC, k = idx % RC;
    As[c][k] = k < re ? A[((int64_t)h * D + c) * rank + k] : 0.f;
    const int kb = idx / D, cb = idx % D;
    Bs[kb][cb] = kb < re ? B[((int64_t)h * rank + kb) * D + cb] : 0.f;
  }
  for (int c = tid; c < D; c += 256) cs[c] = c0[(int64_t)h * D + c];
  for (int idx = tid; idx < R * (D / 4); idx += 256) {
    const int r = idx / (D / 4), c4 = idx % (D / 4);
    const int p = p0 + r;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (p < n) v = *reinterpret_cast<const float4*>(o_gm + (((int64_t)kv * n + p) * g + j) * D + 4 * c4);
    Os[r][4 * c4] = v.x; Os[r][4 * c4 + 1] = v.y; Os[r][4 * c4 + 2] = v.z; Os[r][4 * c4 + 3] = v.w;
  }
  __syncthreads();
  const int r = tid >> 2, q4 = tid & 3;
  {
    float t[TPT];
#pragma unroll
    for (int i = 0; i < TPT; ++i) t[i] = 0.f;
    for (int c = 0; c < D; ++c) {
      const float x = Os[r][c];
#pragma unroll
      for (int i = 0; i < TPT; ++i) t[i] = fmaf(x, As[c][TPT * q4 + i], t[i]);
    }
#pragma unroll
    for (int i = 0; i < TPT; ++i) Ts[r][TPT * q4 + i] = t[i];
  }
  __syncthreads();
  const int p = p0 + r;
  if (p < n) {
    constexpr int CW = D / 4;   // columns per thread
    const int cbase = q4 * CW;
    OutT* orow = out + ((int64_t)h * n + qperm[(int64_t)kv * n + p]) * D + cbase;
#pragma unroll
    for (int c8 = 0; c8 < CW; c8 += 8) {
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = cbase + c8 + e;
        float x = Os[r][c] + cs[c];
        for (int k = 0; k < re; ++k) x = fmaf(Ts[r][k], Bs[k][c], x);
        v[e] = x;
      }
      if constexpr (sizeof(OutT) == 4) {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(orow) + c8) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(orow) + c8 + 4) = make_float4(v[4], v[5], v[6], v[7]);
      } else {
        uint4 pk;
        pk.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
        pk.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
        pk.z = (uint32_t)f32_to_bf16(v[4]) | ((uint32_t)f32_to_bf16(v[5]) << 16);
        pk.w = (uint32_t)f32_to_bf16(v[6]) | ((uint32_t)f32_to_bf16(v[7]) << 16);
        *reinterpret_cast<uint4*>(reinterpret_cast<bf16_t*>(orow) + c8) = pk;
      }
    }
  }
}

// Fast path for correction rank 16 (the method's default): one lane = one group-major row
// of one query head, held in registers; a wave covers 64 consecutive rows.  T = o A and
// o + c0 + T B are computed with A, B and c0 read at wave-uniform addresses (scalar
// loads, no LDS) and the row is written to its token-order position with 16-byte stores.
// Coordinates beyond r_eff are zeroed once T is formed (A and B hold zeros there too).
// Same accumulation order as apply_kernel.  grid (ceil(n / 256), Hq), block 256.
constexpr int kApplyFastRank = 16;
template <typename OutT, int D>
__global__ __launch_bounds__(256) void apply_rows_kernel(const float* __restrict__ o_gm,
                                                         const int32_t* __restrict__ qperm,
                                                         const float* __restrict__ A, const float* __restrict__ B,
                                                         const float* __restrict__ c0,
                                                         const int32_t* __restrict__ r_eff, int n, int g,
                                                         OutT* __restrict__ out) {
  constexpr int RC = kApplyFastRank;
  const int h = blockIdx.y, kv = h / g, j = h % g;
  const int p = blockIdx.x * 256 + threadIdx.x;
  const int re = min(r_eff[h], RC);
  const float* Ah = A + (int64_t)h * D * RC;
  const float* Bh = B + (int64_t)h * RC * D;
  const float* ch = c0 + (int64_t)h * D;
  const bool valid = p < n;
  const float* orow = o_gm + (((int64_t)kv * n + (valid ? p : 0)) * g + j) * D;
  float o[D];
#pragma clang loop unroll(full)
  for (int c = 0; c < D; c += 4) {
    const float4 v = *reinterpret_cast<const float4*>(orow + c);
    o[c] = v.x; o[c + 1] = v.y; o[c + 2] = v.z; o[c + 3] = v.w;
  }
  float t[RC];
#pragma clang loop unroll(full)
  for (int k = 0; k < RC; ++k) t[k] = 0.f;
#pragma clang loop unroll(full)
  for (int c = 0; c < D; ++c) {
#pragma clang loop unroll(full)
    for (int k = 0; k < RC; ++k) t[k] = fmaf(o[c], Ah[c * RC + k], t[k]);
  }
#pragma clang loop unroll(full)
  for (int k = 0; k < RC; ++k) t[k] = k < re ? t[k] : 0.f;
  if (!valid) return;
  OutT* dst = out + ((int64_t)h * n + qperm[(int64_t)kv * n + p]) * D;
#pragma clang loop unroll(full)
  for (int c8 = 0; c8 < D; c8 += 8) {
    float v[8];
#pragma clang loop unroll(full)
    for (int e = 0; e < 8; ++e) v[e] = o[c8 + e] + ch[c8 + e];
#pragma clang loop unroll(full)
    for (int k = 0; k < RC; ++k) {
#pragma clang loop unroll(full)
      for (int e = 0; e < 8; ++e) v[e] = fmaf(t[k], Bh[k * D + c8 + e], v[e]);
    }
    if constexpr (sizeof(OutT) == 4) {
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(dst) + c8) = make_float4(v[0], v[1], v[2], v[3]);
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(dst) + c8 + 4) = make_float4(v[4], v[5], v[6], v[7]);
    } else {
      uint4 pk;
      pk.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
      pk.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
      pk.z = (uint32_t)f32_to_bf16(v[4]) | ((uint32_t)f32_to_bf16(v[5]) << 16);
      pk.w = (uint32_t)f32_to_bf16(v[6]) | ((uint32_t)f32_to_bf16(v[7]) << 16);
      *reinterpret_cast<uint4*>(reinterpret_cast<bf16_t*>(dst) + c8) = pk;
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
  const dim3 grid((unsigned)ceil_div(dm.n, 64), dm.hq);
  if (dm.rc == kApplyFastRank)
    hipLaunchKernelGGL((apply_rows_kernel<OutT, D>), dim3((unsigned)ceil_div(dm.n, 256), dm.hq), dim3(256), 0, s,
                       o_gm, part.query_perm, fit.A, fit.B, fit.c0, fit.r_eff, dm.n, dm.g, o);
  else if (dm.rc <= kMaxRank)
    hipLaunchKernelGGL((apply_kernel<OutT, D, kMaxRank>), grid, dim3(256), 0, s, o_gm, part.query_perm, fit.A, fit.B,
                       fit.c0, fit.r_eff, dm.n, dm.g, dm.rc, o);
  else
    hipLaunchKernelGGL((apply_kernel<OutT, D, kMaxCorrRank>), grid, dim3(256), 0, s, o_gm, part.query_perm, fit.A,
                       fit.B, fit.c0, fit.r_eff, dm.n, dm.g, dm.rc, o);
  if (dm.ablation != SPARSEPR_ABLATE_HARD_DROP)
    hipLaunchKernelGGL(probe_writeback_kernel<OutT>, dim3(dm.hq), dim3(256), 0, s, fit.o_dense, fit.probe_tokens,
                       dm.n, dm.g, dm.m, D, o);
}

void launch_probe_writeback(const Dims& dm, const sparsepr_fit_t& fit, void* o, hipStream_t s) {
  if (dm.bf16)
    hipLaunchKernelGGL(probe_writeback_kernel<bf16_t>, dim3(dm.hq), dim3(256), 0, s, fit.o_dense, fit.probe_tokens, dm.n,
                       dm.g, dm.m, dm.d, (bf16_t*)o);
  else
    hipLaunchKernelGGL(probe_writeback_kernel<float>, dim3(dm.hq), dim3(256), 0, s, fit.o_dense, fit.probe_tokens, dm.n,
                       dm.g, dm.m, dm.d, (float*)o);
}

void launch_apply(const Dims& dm, const float* o_gm, const sparsepr_partition_t& part, const sparsepr_fit_t& fit,
                  void* o, hipStream_t s) {
  if (dm.bf16 && dm.rc <= kMaxCorrRank) {
    // bf16 output: the matrix-core write-back (the fused epilogue's arithmetic; with split
    // hi/lo operands under GQA and for the unprojected ridge, whose corrections can reach the
    // size of the output), then the exact probe rows
    launch_apply_mfma(dm, o_gm, part, fit, o, s);
    if (dm.ablation != SPARSEPR_ABLATE_HARD_DROP) launch_probe_writeback(dm, fit, o, s);
  } else if (dm.bf16) {
    if (dm.d == 128) apply_typed<bf16_t, 128>(dm, o_gm, part, fit, (bf16_t*)o, s);
    else apply_typed<bf16_t, 64>(dm, o_gm, part, fit, (bf16_t*)o, s);
  } else {
    if (dm.d == 128) apply_typed<float, 128>(dm, o_gm, part, fit, (float*)o, s);
    else apply_typed<float, 64>(dm, o_gm, part, fit, (float*)o, s);
  }
}

}  // namespace sp
