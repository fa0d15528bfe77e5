// Block-sparse attention over the kept (query group x key group) cells, exact on those
// cells and renormalised over the kept K/V groups (summary page of "Partition the
// Support, Reconstruct the Residual", execution paragraph), and the dense attention
// baseline on the same tile schedule.
//
// This file holds the vector-ALU path: fp32 online softmax on the vector
// ALUs with K/V tiles staged in LDS.  It serves fp32 inputs (exact to fp32 rounding)
// and any shape the matrix-core path does not take.
#include "sp_attn.hpp"
#include "sp_common.hpp"
#include "sp_launch.hpp"

namespace sp {

// Block = 32 virtual rows x 64-key tiles; thread (row = tid / 8, sub = tid % 8) owns keys
// sub + 8 i of each tile and output columns sub + 8 c.
template <typename T, int D, typename OutT>
__global__ __launch_bounds__(256) void attn_valu_kernel(AttnArgs A) {
  constexpr int BM = 32, BN = 64, CPT = D / 8;
  __shared__ float qs[BM][D + 1];
  __shared__ float ks[BN][D + 1];
  __shared__ float vs[BN][D + 1];
  __shared__ float ps[BM][BN + 1];
  const int kv = blockIdx.y;
  TileInfo ti;
  if (!find_tile(A, kv, blockIdx.x, BM, ti)) return;
  const int tid = threadIdx.x, r = tid >> 3, sub = tid & 7;
  const T* qb = static_cast<const T*>(A.q);
  const T* kb = static_cast<const T*>(A.k) + (int64_t)kv * A.kv_skv;
  const T* vb = static_cast<const T*>(A.v) + (int64_t)kv * A.v_skv;
  for (int idx = tid; idx < BM * D; idx += 256) {
    const int rr = idx / D, c = idx % D, v = ti.v0 + rr;
    float x = 0.f;
    if (v < ti.v1) x = to_f32(qb[(int64_t)kv * A.q_skv + (int64_t)(v / A.g) * A.q_sp + (int64_t)(v % A.g) * A.q_sj + c]);
    qs[rr][c] = x;
  }
  float m_i = -INFINITY, l_i = 0.f;
  float o[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) o[c] = 0.f;
  int ci = ti.kbeg < 0 ? 0 : ti.kbeg, k0 = 0, k1 = 0;
  while (next_run(A, kv, ti, ci, k0, k1)) {
    for (int kt = k0; kt < k1; kt += BN) {
      const int nk = min(BN, k1 - kt);
      __syncthreads();
      for (int idx = tid; idx < BN * D; idx += 256) {
        const int kk = idx / D, c = idx % D;
        const bool in = kk < nk;
        ks[kk][c] = in ? to_f32(kb[(int64_t)(kt + kk) * D + c]) : 0.f;
        vs[kk][c] = in ? to_f32(vb[(int64_t)c * A.v_np + vt_pos(kt + kk)]) : 0.f;
      }
      __syncthreads();
      float s[8];
      float tmax = -INFINITY;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int key = sub + 8 * i;
        float acc = 0.f;
        for (int c = 0; c < D; ++c) acc = fmaf(qs[r][c], ks[key][c], acc);
        s[i] = key < nk ? acc * A.scale : -INFINITY;
        tmax = fmaxf(tmax, s[i]);
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 1));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 2));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 4));
      const float m_new = fmaxf(m_i, tmax);
      const float alpha = expf(m_i - m_new);
      float rs = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p = (s[i] == -INFINITY) ? 0.f : expf(s[i] - m_new);
        ps[r][sub + 8 * i] = p;
        rs += p;
      }
      rs += __shfl_xor(rs, 1);
      rs += __shfl_xor(rs, 2);
      rs += __shfl_xor(rs, 4);
      l_i = l_i * alpha + rs;
      m_i = m_new;
      __syncthreads();
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const int col = sub + 8 * c;
        float acc = o[c] * alpha;
        for (int key = 0; key < nk; ++key) acc = fmaf(ps[r][key], vs[key][col], acc);
        o[c] = acc;
      }
    }
  }
  const int v = ti.v0 + r;
  if (v < ti.v1) {
    const int p = v / A.g, j = v % A.g;
    const float inv = 1.f / l_i;
    OutT* ob = static_cast<OutT*>(A.o) + (int64_t)kv * A.o_skv + (int64_t)p * A.o_sp + (int64_t)j * A.o_sj;
#pragma unroll
    for (int c = 0; c < CPT; ++c) ob[sub + 8 * c] = from_f32<OutT>(o[c] * inv);
    if (A.lse && sub == 0) A.lse[((int64_t)kv * A.n + p) * A.g + j] = m_i + logf(l_i);
  }
}

template <typename T, int D, typename OutT>
static void launch_valu(AttnArgs a, int hkv, hipStream_t s) {
  constexpr int BM = 32;
  a.tiles_per_head = (int)ceil_div((int64_t)a.n * a.g, BM) + (a.qoff ? a.gq : 0);
  hipLaunchKernelGGL((attn_valu_kernel<T, D, OutT>), dim3(a.tiles_per_head, hkv), dim3(256), 0, s, a);
}

// bf16 inputs run on the matrix cores (attend_mfma.hip); fp32 inputs on the vector ALUs.
void launch_attention(const Dims& dm, AttnArgs a, bool out_is_input_dtype, hipStream_t s) {
  if (dm.bf16) {
    launch_attention_mfma(dm, a, out_is_input_dtype, s);
  } else {
    if (dm.d == 128) launch_valu<float, 128, float>(a, dm.hkv, s); else launch_valu<float, 64, float>(a, dm.hkv, s);
  }
}

}  // namespace sp
