// Probe-fit residual reconstruction (summary page of "Partition the Support, Reconstruct
// the Residual", probe-fit residual reconstruction paragraph): M probe rows per KV head
// stratified over query groups and drawn in radial order about each group's centroid,
// their exact attention against all keys and against the kept cells only (one pass,
// two online-softmax accumulators, split over key chunks), R = O_dense - O_sparse, the
// group-coverage-weighted ridge fit of R on O_sparse (dual M x M Cholesky) and the
// rank-r output subspace of the weighted probe residuals (parallel two-sided Jacobi on
// the M x M Gram matrix).  The fit runs in double precision, one block per query head.
#include <cmath>

#include "sp_common.hpp"
#include "sp_launch.hpp"

namespace sp {

constexpr int kSortMax = 8192;   // groups up to this size are sorted in LDS

// ---------------------------------------------------------------------------------------
// Probe rows for the ablations (PSRR, ablation paragraph): uniform over the raster order
// (tokens floor((2k+1) n / (2M))) or the caller's tokens in ptok (clamped into [0, n));
// weight 1, group = the token's query label.  grid Hkv, block 64.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(64) void probe_select_plain_kernel(const int32_t* __restrict__ qlabels, int n, int M,
                                                                int uniform, int32_t* __restrict__ ptok,
                                                                int32_t* __restrict__ pgrp,
                                                                double* __restrict__ pw) {
  const int kv = blockIdx.x;
  for (int k = threadIdx.x; k < M; k += 64) {
    int tok;
    if (uniform) tok = (int)(((int64_t)(2 * k + 1) * n) / (2 * M));
    else tok = min(max(ptok[kv * M + k], 0), n - 1);
    ptok[kv * M + k] = tok;
    pgrp[kv * M + k] = qlabels[(int64_t)kv * n + tok];
    pw[kv * M + k] = 1.0;
  }
}

// ---------------------------------------------------------------------------------------
// Probe selection.  grid (Gq, Hkv), block 256.
// Allocation: one probe at a time over the non-empty groups in the order (larger group
// first, smaller index first), skipping full groups.  Within group a the m_a probes are
// the members of rank floor((2k+1) n_a / (2 m_a)) in the order (squared distance of the
// integer query features (width F) to the group centroid, token index).
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void probe_select_kernel(const int8_t* __restrict__ XQ,
                                                           const int32_t* __restrict__ qcent,
                                                           const int32_t* __restrict__ qperm,
                                                           const int32_t* __restrict__ qoff, int n,
                                                           int Gq, int F, int M, int32_t* __restrict__ ptok,
                                                           int32_t* __restrict__ pgrp,
                                                           double* __restrict__ pw,
                                                           int32_t* __restrict__ radius) {
  __shared__ int alloc[kMaxGroups], start[kMaxGroups], tgt[kMaxProbe];
  __shared__ int sz[kMaxGroups];
  __shared__ int cent[kMaxSemFeat];
  __shared__ int lrad[1024];
  __shared__ uint64_t skey[kSortMax];
  const int a = blockIdx.x, kv = blockIdx.y, tid = threadIdx.x;
  const int32_t* qo = qoff + (int64_t)kv * (Gq + 1);
  if (tid < kMaxGroups) sz[tid] = tid < Gq ? qo[tid + 1] - qo[tid] : 0;
  __syncthreads();
  if (tid < 64) {
    // The one-at-a-time allocation in closed form: after p complete passes group b holds
    // min(n_b, p) probes, T(p) = sum_b min(n_b, p); p* is the last p with T(p) <= M, and
    // the R = M - T(p*) remaining probes go to the first R groups with n_b > p* in the
    // order (larger group first, smaller index first).
    const int b = tid, sb = sz[b];
    int maxs = sb;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) maxs = max(maxs, __shfl_xor(maxs, o));
    int pstar = 0, tp = 0;
    for (int p = 1; p <= min(maxs, M); ++p) {
      int t = min(sb, p);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) t += __shfl_xor(t, o);
      if (t > M) break;
      pstar = p;
      tp = t;
    }
    int rank = 0;
    for (int c = 0; c < kMaxGroups; ++c) {
      const int sc = sz[c];
      rank += (sc > pstar) && (sc > sb || (sc == sb && c < b));
    }
    const int al = min(sb, pstar) + ((sb > pstar && rank < M - tp) ? 1 : 0);
    int incl = al;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(incl, o);
      if (b >= o) incl += u;
    }
    alloc[b] = al;
    start[b] = incl - al;
  }
  __syncthreads();
  const int ma = alloc[a];
  if (ma == 0) return;
  const int na = qo[a + 1] - qo[a], off = qo[a];
  for (int f = tid; f < F; f += 256) cent[f] = qcent[((int64_t)kv * Gq + a) * F + f];
  for (int k = tid; k < ma; k += 256) tgt[k] = (int)(((int64_t)(2 * k + 1) * na) / (2 * ma));
  __syncthreads();
  int32_t* rad = radius + (int64_t)kv * n + off;
  for (int i = tid; i < na; i += 256) {
    const int tok = qperm[(int64_t)kv * n + off + i];
    const int8_t* x = XQ + ((int64_t)kv * n + tok) * F;
    int s = 0;
    if ((F & 15) == 0) {
      for (int f0 = 0; f0 < F; f0 += 16) {
        const uint4 v = *reinterpret_cast<const uint4*>(x + f0);
        const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int dd = (int)(int8_t)(wv[e >> 2] >> (8 * (e & 3))) - cent[f0 + e];
          s += dd * dd;
        }
      }
    } else {
      for (int f = 0; f < F; ++f) { int dd = (int)x[f] - cent[f]; s += dd * dd; }
    }
    rad[i] = s;
  }
  __syncthreads();
  if (na <= kSortMax) {
    // members fit in LDS: bitonic sort of (radius << 13 | position) keys, then read the
    // target ranks directly
    int P = 1;
    while (P < na) P <<= 1;
    for (int i = tid; i < P; i += 256)
      skey[i] = i < na ? (((uint64_t)(uint32_t)rad[i]) << 13) | (uint64_t)i : ~0ull;
    __syncthreads();
    for (int size = 2; size <= P; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int t = tid; t < P / 2; t += 256) {
          const int lo = 2 * t - (t & (stride - 1));
          const int hi = lo + stride;
          const bool up = (lo & size) == 0;
          const uint64_t x = skey[lo], y = skey[hi];
          if ((x > y) == up) { skey[lo] = y; skey[hi] = x; }
        }
        __syncthreads();
      }
    }
    for (int k = tid; k < ma; k += 256) {
      const int i = (int)(skey[tgt[k]] & (kSortMax - 1));
      const int slot = kv * M + start[a] + k;
      ptok[slot] = qperm[(int64_t)kv * n + off + i];
      pgrp[slot] = a;
      pw[slot] = (double)M * (double)na / ((double)ma * (double)n);
    }
    return;
  }
  // large group: rank of every member by counting smaller keys, tiled through LDS
  for (int i0 = 0; i0 < na; i0 += 256) {
    const int i = i0 + tid;
    const int my = i < na ? rad[i] : 0;
    int cnt = 0;
    for (int c0 = 0; c0 < na; c0 += 1024) {
      __syncthreads();
      for (int t = tid; t < 1024; t += 256) lrad[t] = (c0 + t < na) ? rad[c0 + t] : 0;
      __syncthreads();
      const int lim = min(1024, na - c0);
      if (i < na) {
        for (int t = 0; t < lim; ++t) {
          const int r2 = lrad[t];
          cnt += (r2 < my) || (r2 == my && c0 + t < i);
        }
      }
    }
    if (i < na) {
      int lo = 0, hi = ma - 1;
      while (lo < hi) {  // first target >= cnt
        int mid = (lo + hi) >> 1;
        if (tgt[mid] < cnt) lo = mid + 1; else hi = mid;
      }
      if (tgt[lo] == cnt) {
        const int slot = kv * M + start[a] + lo;
        ptok[slot] = qperm[(int64_t)kv * n + off + i];
        pgrp[slot] = a;
        pw[slot] = (double)M * (double)na / ((double)ma * (double)n);
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// Probe rows against one key chunk, dense and sparse accumulators.  grid (chunks, Hq),
// block 256: probe row r = tid / 4, sub = tid % 4 owns keys sub + 4 i of each 32-key tile
// and output columns sub + 4 c.  Partials [Hq][chunks][M][2][D + 2] = (o, m, l).
// ---------------------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void probe_attn_kernel(const T* __restrict__ q, const T* __restrict__ kgm,
                                                         const T* __restrict__ vgm,
                                                         const int32_t* __restrict__ koff,
                                                         const uint64_t* __restrict__ kept_mask,
                                                         const int32_t* __restrict__ ptok,
                                                         const int32_t* __restrict__ pgrp, int n, int g,
                                                         int Gq, int Gk, int M, float scale, int chunk,
                                                         float* __restrict__ partials) {
  constexpr int BN = 32, CPT = D / 4;
  __shared__ float qs[kMaxProbe][D + 1];
  __shared__ float ks[BN][D + 1];
  __shared__ float vs[BN][D + 1];
  __shared__ float pd[kMaxProbe][BN + 1];
  __shared__ float pq[kMaxProbe][BN + 1];
  __shared__ int klab[BN];
  __shared__ int ko[kMaxGroups + 1];
  __shared__ uint64_t msk[kMaxProbe];
  const int h = blockIdx.y, kv = h / g, ch = blockIdx.x;
  const int nch = gridDim.x;
  const int tid = threadIdx.x, r = tid >> 2, sub = tid & 3;
  const int k0 = ch * chunk, k1 = min(n, k0 + chunk);
  for (int idx = tid; idx < kMaxProbe * D; idx += 256) {
    const int rr = idx / D, c = idx % D;
    float x = 0.f;
    if (rr < M) x = to_f32(q[((int64_t)h * n + ptok[kv * M + rr]) * D + c]);
    qs[rr][c] = x;
  }
  if (tid < kMaxProbe) msk[tid] = tid < M ? kept_mask[(int64_t)kv * Gq + pgrp[kv * M + tid]] : 0ull;
  for (int b = tid; b <= Gk; b += 256) ko[b] = koff[(int64_t)kv * (Gk + 1) + b];
  const T* kb = kgm + (int64_t)kv * n * D;
  const int np = (int)vt_pad(n);
  const T* vb = vgm + (int64_t)kv * D * np;
  float md = -INFINITY, ld = 0.f, ms = -INFINITY, ls = 0.f;
  float od[CPT], os[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) { od[c] = 0.f; os[c] = 0.f; }
  for (int kt = k0; kt < k1; kt += BN) {
    const int nk = min(BN, k1 - kt);
    __syncthreads();
    for (int idx = tid; idx < BN * D; idx += 256) {
      const int kk = idx / D, c = idx % D;
      const bool in = kk < nk;
      ks[kk][c] = in ? to_f32(kb[(int64_t)(kt + kk) * D + c]) : 0.f;
      vs[kk][c] = in ? to_f32(vb[(int64_t)c * np + vt_pos(kt + kk)]) : 0.f;
    }
    if (tid < BN) {
      int lab = 0;
      if (tid < nk) {
        const int pos = kt + tid;
        int lo = 0, hi = Gk - 1;  // last b with ko[b] <= pos
        while (lo < hi) { int mid = (lo + hi + 1) >> 1; if (ko[mid] <= pos) lo = mid; else hi = mid - 1; }
        lab = lo;
      }
      klab[tid] = lab;
    }
    __syncthreads();
    float s[8];
    bool kp[8];
    float td = -INFINITY, ts = -INFINITY;
    const uint64_t mr = msk[r];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int key = sub + 4 * i;
      float acc = 0.f;
#pragma unroll 4
      for (int c = 0; c < D; ++c) acc = fmaf(qs[r][c], ks[key][c], acc);
      const bool valid = key < nk;
      s[i] = valid ? acc * scale : -INFINITY;
      kp[i] = valid && ((mr >> klab[key]) & 1ull);
      td = fmaxf(td, s[i]);
      if (kp[i]) ts = fmaxf(ts, s[i]);
    }
    td = fmaxf(td, __shfl_xor(td, 1));
    td = fmaxf(td, __shfl_xor(td, 2));
    ts = fmaxf(ts, __shfl_xor(ts, 1));
    ts = fmaxf(ts, __shfl_xor(ts, 2));
    const float mdn = fmaxf(md, td);
    const float ad = expf(md - mdn);
    const float msn = fmaxf(ms, ts);
    const float as = (msn == -INFINITY) ? 1.f : expf(ms - msn);
    float rd = 0.f, rsum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = (s[i] == -INFINITY) ? 0.f : expf(s[i] - mdn);
      const float pk = kp[i] ? expf(s[i] - msn) : 0.f;
      pd[r][sub + 4 * i] = p;
      pq[r][sub + 4 * i] = pk;
      rd += p;
      rsum += pk;
    }
    rd += __shfl_xor(rd, 1);
    rd += __shfl_xor(rd, 2);
    rsum += __shfl_xor(rsum, 1);
    rsum += __shfl_xor(rsum, 2);
    ld = ld * ad + rd;
    ls = ls * as + rsum;
    md = mdn;
    ms = msn;
    __syncthreads();
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int col = sub + 4 * c;
      float a1 = od[c] * ad, a2 = os[c] * as;
#pragma unroll 2
      for (int key = 0; key < nk; ++key) {
        const float vv = vs[key][col];
        a1 = fmaf(pd[r][key], vv, a1);
        a2 = fmaf(pq[r][key], vv, a2);
      }
      od[c] = a1;
      os[c] = a2;
    }
  }
  if (r < M) {
    float* pb = partials + (((int64_t)h * nch + ch) * M + r) * 2 * (D + 2);
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      pb[sub + 4 * c] = od[c];
      pb[D + 2 + sub + 4 * c] = os[c];
    }
    if (sub == 0) {
      pb[D] = md; pb[D + 1] = ld;
      pb[2 * D + 2] = ms; pb[2 * D + 3] = ls;
    }
  }
}

// ---------------------------------------------------------------------------------------
// Fit, one block (256 threads) per query head, double precision.
// fb: per-head scratch [X | Y | Z] (M x D each) followed by Vr (D x 32).
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ void jacobi_pair(int t, int i, int& p, int& q) {
  if (i == 0) { p = 0; q = 1 + t; }
  else { p = 1 + (t + i) % 63; q = 1 + (t - i + 63) % 63; }
}

// Merge of the per-chunk probe partials (log-sum-exp combination), one block per
// (probe row, query head), one thread per output column; writes O_dense / O_sparse
// (fp32 outputs) and X = O_sparse, Y = O_dense - O_sparse (float64 fit inputs).
template <int D>
__global__ __launch_bounds__(D) void probe_merge_kernel(const float* __restrict__ partials, int nch, int M,
                                                        double* __restrict__ fbuf, float* __restrict__ o_dense,
                                                        float* __restrict__ o_sparse) {
  const int r = blockIdx.x, h = blockIdx.y, c = threadIdx.x;
  double res[2];
  for (int which = 0; which < 2; ++which) {
    double mx = -INFINITY;
    for (int ch = 0; ch < nch; ++ch)
      mx = fmax(mx, (double)partials[(((int64_t)h * nch + ch) * M + r) * 2 * (D + 2) + which * (D + 2) + D]);
    double L = 0.0, O = 0.0;
    for (int ch = 0; ch < nch; ++ch) {
      const float* pb = partials + (((int64_t)h * nch + ch) * M + r) * 2 * (D + 2) + which * (D + 2);
      const double m = pb[D];
      if (m == -INFINITY) continue;
      const double sc = exp(m - mx);
      L += (double)pb[D + 1] * sc;
      O += (double)pb[c] * sc;
    }
    res[which] = O / L;
  }
  o_dense[((int64_t)h * M + r) * D + c] = (float)res[0];
  o_sparse[((int64_t)h * M + r) * D + c] = (float)res[1];
  double* X = fbuf + (size_t)h * (3 * kMaxProbe * D + D * kMaxRank);
  X[r * D + c] = res[1];
  X[kMaxProbe * D + r * D + c] = res[0] - res[1];
}

// ridge_only: write the unprojected ridge map as A = Xt^T [d, M], B = Z [M, d] (leading
// dimension M) and skip the subspace (PSRR, ablation paragraph).
template <int D>
__global__ __launch_bounds__(256) void probe_fit_kernel(const float* __restrict__ partials, int nch,
                                                        const double* __restrict__ pw, int g, int M,
                                                        int rank, int ridge_only, double lam,
                                                        double* __restrict__ fbuf,
                                                        float* __restrict__ o_dense,
                                                        float* __restrict__ o_sparse, float* __restrict__ Aout,
                                                        float* __restrict__ Bout, float* __restrict__ c0out,
                                                        int32_t* __restrict__ r_eff_out,
                                                        float* __restrict__ eig_out) {
  constexpr int MM = kMaxProbe;
  __shared__ double Km[MM][MM + 1];
  __shared__ double Vm[MM][MM + 1];
  __shared__ double w[MM], xbar[D], ybar[D], rc[32], rs[32], ev[MM], xa[kMaxRank], red[256];
  __shared__ int pp[32], qq[32], ord[MM];
  __shared__ int reff_s;
  __shared__ int stop_s;
  const int h = blockIdx.x, kv = h / g, tid = threadIdx.x;
  double* X = fbuf + (size_t)h * (3 * MM * D + D * kMaxRank);
  double* Y = X + MM * D;
  double* Z = Y + MM * D;
  double* Vr = Z + MM * D;
  if (tid < M) w[tid] = pw[kv * M + tid];
  __syncthreads();
  // 2. weighted centring and sqrt(w) scaling
  double sw = 0.0;
  for (int r = 0; r < M; ++r) sw += w[r];
  for (int c = tid; c < D; c += 256) {
    double sx = 0.0, sy = 0.0;
    for (int r = 0; r < M; ++r) { sx += w[r] * X[r * D + c]; sy += w[r] * Y[r * D + c]; }
    xbar[c] = sx / sw;
    ybar[c] = sy / sw;
  }
  __syncthreads();
  for (int idx = tid; idx < M * D; idx += 256) {
    const int r = idx / D, c = idx % D;
    const double sq = sqrt(w[r]);
    X[idx] = sq * (X[idx] - xbar[c]);
    Y[idx] = sq * (Y[idx] - ybar[c]);
  }
  __syncthreads();
  // 3. K = Xt Xt^T + lambda I
  for (int idx = tid; idx < M * M; idx += 256) {
    const int i = idx / M, j = idx % M;
    double s = 0.0;
    for (int c = 0; c < D; ++c) s += X[i * D + c] * X[j * D + c];
    Km[i][j] = s + (i == j ? lam : 0.0);
  }
  __syncthreads();
  // 4. Cholesky K = L L^T (lower triangle of Km)
  for (int k = 0; k < M; ++k) {
    if (tid == 0) Km[k][k] = sqrt(Km[k][k]);
    __syncthreads();
    for (int i = k + 1 + tid; i < M; i += 256) Km[i][k] /= Km[k][k];
    __syncthreads();
    const int rem = M - k - 1;
    for (int idx = tid; idx < rem * rem; idx += 256) {
      const int i = k + 1 + idx / rem, j = k + 1 + idx % rem;
      if (j <= i) Km[i][j] -= Km[i][k] * Km[j][k];
    }
    __syncthreads();
  }
  // 5. Z = K^{-1} Yt, one thread per column
  for (int c = tid; c < D; c += 256) {
    for (int i = 0; i < M; ++i) {
      double s = Y[i * D + c];
      for (int k = 0; k < i; ++k) s -= Km[i][k] * Z[k * D + c];
      Z[i * D + c] = s / Km[i][i];
    }
    for (int i = M - 1; i >= 0; --i) {
      double s = Z[i * D + c];
      for (int k = i + 1; k < M; ++k) s -= Km[k][i] * Z[k * D + c];
      Z[i * D + c] = s / Km[i][i];
    }
  }
  __syncthreads();
  if (ridge_only) {
    // xa[k] = xbar . Xt[k]; c0 = ybar - xa Z; A = Xt^T, B = Z (leading dimension M)
    double* xam = &Vm[0][0];
    for (int k = tid; k < M; k += 256) {
      double acc = 0.0;
      for (int c = 0; c < D; ++c) acc += xbar[c] * X[k * D + c];
      xam[k] = acc;
    }
    __syncthreads();
    for (int idx = tid; idx < D * M; idx += 256) {
      const int c = idx / M, k = idx % M;
      Aout[(int64_t)h * D * M + idx] = (float)X[k * D + c];
      Bout[(int64_t)h * M * D + (int64_t)k * D + c] = (float)Z[k * D + c];
    }
    for (int c = tid; c < D; c += 256) {
      double acc = ybar[c];
      for (int k = 0; k < M; ++k) acc -= xam[k] * Z[k * D + c];
      c0out[(int64_t)h * D + c] = (float)acc;
    }
    for (int k = tid; k <= rank; k += 256) eig_out[(int64_t)h * (rank + 1) + k] = 0.f;
    if (tid == 0) r_eff_out[h] = M;
    return;
  }
  // 6. G = Yt Yt^T (zero-padded to 64 x 64), V = I
  for (int idx = tid; idx < MM * MM; idx += 256) {
    const int i = idx / MM, j = idx % MM;
    double s = 0.0;
    if (i < M && j < M)
      for (int c = 0; c < D; ++c) s += Y[i * D + c] * Y[j * D + c];
    Km[i][j] = s;
    Vm[i][j] = (i == j) ? 1.0 : 0.0;
  }
  __syncthreads();
  // 7. parallel cyclic Jacobi (round-robin pairing: 32 disjoint rotations per step)
  for (int sweep = 0; sweep < 30; ++sweep) {
    double off = 0.0, dg = 0.0;
    for (int idx = tid; idx < MM * MM; idx += 256) {
      const int i = idx / MM, j = idx % MM;
      const double v = Km[i][j];
      if (i == j) dg += v * v; else off += v * v;
    }
    red[tid] = off;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) { if (tid < s) red[tid] += red[tid + s]; __syncthreads(); }
    const double off_all = red[0];
    __syncthreads();
    red[tid] = dg;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) { if (tid < s) red[tid] += red[tid + s]; __syncthreads(); }
    if (tid == 0) stop_s = (off_all <= 1e-24 * red[0]) || (off_all == 0.0);
    __syncthreads();
    if (stop_s) break;
    for (int t = 0; t < MM - 1; ++t) {
      if (tid < 32) {
        int p, q;
        jacobi_pair(t, tid, p, q);
        const double apq = Km[p][q];
        double c = 1.0, s = 0.0;
        if (apq != 0.0) {
          const double tau = (Km[q][q] - Km[p][p]) / (2.0 * apq);
          const double tt = tau >= 0.0 ? 1.0 / (tau + sqrt(1.0 + tau * tau)) : -1.0 / (-tau + sqrt(1.0 + tau * tau));
          c = 1.0 / sqrt(1.0 + tt * tt);
          s = tt * c;
        }
        pp[tid] = p; qq[tid] = q; rc[tid] = c; rs[tid] = s;
      }
      __syncthreads();
      for (int blk = tid; blk < 32 * 32; blk += 256) {
        const int bi = blk >> 5, bj = blk & 31;
        const int pi = pp[bi], qi = qq[bi], pj = pp[bj], qj = qq[bj];
        const double ci = rc[bi], si = rs[bi], cj = rc[bj], sj = rs[bj];
        const double a00 = Km[pi][pj], a01 = Km[pi][qj], a10 = Km[qi][pj], a11 = Km[qi][qj];
        const double t00 = a00 * cj - a01 * sj, t01 = a00 * sj + a01 * cj;
        const double t10 = a10 * cj - a11 * sj, t11 = a10 * sj + a11 * cj;
        Km[pi][pj] = ci * t00 - si * t10;
        Km[pi][qj] = ci * t01 - si * t11;
        Km[qi][pj] = si * t00 + ci * t10;
        Km[qi][qj] = si * t01 + ci * t11;
        if (bi == bj) { Km[pi][qj] = 0.0; Km[qi][pj] = 0.0; }
      }
      for (int idx = tid; idx < MM * 32; idx += 256) {
        const int row = idx >> 5, j = idx & 31;
        const int pj = pp[j], qj = qq[j];
        const double cj = rc[j], sj = rs[j];
        const double vp = Vm[row][pj], vq = Vm[row][qj];
        Vm[row][pj] = cj * vp - sj * vq;
        Vm[row][qj] = sj * vp + cj * vq;
      }
      __syncthreads();
    }
  }
  // 8. order the eigenvalues (descending, ties by index) and choose r_eff
  if (tid < MM) ev[tid] = Km[tid][tid];
  __syncthreads();
  if (tid < MM) {
    int cnt = 0;
    for (int j = 0; j < MM; ++j) cnt += (ev[j] > ev[tid]) || (ev[j] == ev[tid] && j < tid);
    ord[cnt] = tid;
  }
  __syncthreads();
  if (tid == 0) {
    const double l1 = ev[ord[0]];
    int re = 0;
    for (int k = 0; k < rank && k < M; ++k)
      if (l1 > 0.0 && ev[ord[k]] > 1e-8 * l1) ++re; else break;
    reff_s = re;
    r_eff_out[h] = re;
  }
  for (int k = tid; k <= rank; k += 256) eig_out[(int64_t)h * (rank + 1) + k] = k < MM ? (float)ev[ord[k]] : 0.f;
  __syncthreads();
  const int re = reff_s;
  // 9. V_r[:, k] = Yt^T a_k / sqrt(lambda_k)
  for (int idx = tid; idx < D * kMaxRank; idx += 256) {
    const int c = idx / kMaxRank, k = idx % kMaxRank;
    double s = 0.0;
    if (k < re) {
      const int e = ord[k];
      for (int i = 0; i < M; ++i) s += Y[i * D + c] * Vm[i][e];
      s /= sqrt(ev[e]);
    }
    Vr[c * kMaxRank + k] = s;
  }
  __syncthreads();
  // 10. ZV = Z V_r (M x r) into Km
  for (int idx = tid; idx < M * kMaxRank; idx += 256) {
    const int i = idx / kMaxRank, k = idx % kMaxRank;
    double s = 0.0;
    if (k < re)
      for (int c = 0; c < D; ++c) s += Z[i * D + c] * Vr[c * kMaxRank + k];
    Km[i][k] = s;
  }
  __syncthreads();
  // 11. A = Xt^T ZV (D x r) into Vm rows (D <= 128 rows -> two halves of 64 columns)
  double* Al = &Vm[0][0];  // D * kMaxRank doubles fit in Vm (64 * 65)
  for (int idx = tid; idx < D * kMaxRank; idx += 256) {
    const int c = idx / kMaxRank, k = idx % kMaxRank;
    double s = 0.0;
    if (k < re)
      for (int i = 0; i < M; ++i) s += X[i * D + c] * Km[i][k];
    Al[c * kMaxRank + k] = s;
  }
  __syncthreads();
  for (int k = tid; k < kMaxRank; k += 256) {
    double s = 0.0;
    for (int c = 0; c < D; ++c) s += xbar[c] * Al[c * kMaxRank + k];
    xa[k] = s;
  }
  __syncthreads();
  // 12. outputs: A [D][rank], B [rank][D], c0 = ybar - (xbar A) B
  for (int idx = tid; idx < D * rank; idx += 256) {
    const int c = idx / rank, k = idx % rank;
    Aout[(int64_t)h * D * rank + idx] = k < re ? (float)Al[c * kMaxRank + k] : 0.f;
    Bout[(int64_t)h * rank * D + (int64_t)k * D + c] = k < re ? (float)Vr[c * kMaxRank + k] : 0.f;
  }
  for (int c = tid; c < D; c += 256) {
    double s = ybar[c];
    for (int k = 0; k < re; ++k) s -= xa[k] * Vr[c * kMaxRank + k];
    c0out[(int64_t)h * D + c] = (float)s;
  }
}

void launch_probe_fit(const Dims& dm, const Workspace& wp, const void* q, const sparsepr_partition_t& part,
                      const sparsepr_route_t& route, const sparsepr_fit_t& out, char* ws, hipStream_t s) {
  int32_t* radius = reinterpret_cast<int32_t*>(ws + wp.probe_alloc);
  float* partials = reinterpret_cast<float*>(ws + wp.partials);
  double* fbuf = reinterpret_cast<double*>(ws + wp.fitbuf);
  if (dm.ablation == SPARSEPR_ABLATE_HARD_DROP) {
    // empty fit: nothing is reconstructed and no probe row is written back
    const size_t hq = (size_t)dm.hq, d = (size_t)dm.d;
    fill_u32(reinterpret_cast<uint32_t*>(out.probe_tokens), (size_t)dm.hkv * dm.m, 0xffffffffu, s);
    fill_u32(reinterpret_cast<uint32_t*>(out.probe_groups), (size_t)dm.hkv * dm.m, 0xffffffffu, s);
    fill_u32(reinterpret_cast<uint32_t*>(out.probe_weights), (size_t)dm.hkv * dm.m * 2, 0, s);
    fill_u32(reinterpret_cast<uint32_t*>(out.o_dense), hq * dm.m * d, 0, s);
    fill_u32(reinterpret_cast<uint32_t*>(out.o_sparse), hq * dm.m * d, 0, s);
    fill_u32(reinterpret_cast<uint32_t*>(out.A), hq * d * dm.rc, 0, s);
    fill_u32(reinterpret_cast<uint32_t*>(out.B), hq * dm.rc * d, 0, s);
    fill_u32(reinterpret_cast<uint32_t*>(out.c0), hq * d, 0, s);
    fill_u32(reinterpret_cast<uint32_t*>(out.r_eff), hq, 0, s);
    fill_u32(reinterpret_cast<uint32_t*>(out.eig), hq * (dm.r + 1), 0, s);
    return;
  }
  if (dm.probe_mode == SPARSEPR_PROBES_RADIAL)
    hipLaunchKernelGGL(probe_select_kernel, dim3(dm.gq, dm.hkv), dim3(256), 0, s, part.query_features,
                       part.query_centroids, part.query_perm, part.query_offsets, dm.n, dm.gq, dm.fq, dm.m,
                       out.probe_tokens, out.probe_groups, out.probe_weights, radius);
  else
    hipLaunchKernelGGL(probe_select_plain_kernel, dim3(dm.hkv), dim3(64), 0, s, part.query_labels, dm.n, dm.m,
                       dm.probe_mode == SPARSEPR_PROBES_UNIFORM ? 1 : 0, out.probe_tokens, out.probe_groups,
                       out.probe_weights);
  const dim3 pgrid(wp.nchunks, dm.hq);
  if (dm.bf16) {
    launch_probe_attn_mfma(dm, q, part, route, out, kProbeChunk, wp.nchunks, partials, s);
  } else {
    if (dm.d == 128)
      hipLaunchKernelGGL((probe_attn_kernel<float, 128>), pgrid, dim3(256), 0, s, (const float*)q,
                         (const float*)part.k_gm, (const float*)part.v_gm, part.key_offsets, route.kept_mask,
                         out.probe_tokens, out.probe_groups, dm.n, dm.g, dm.gq, dm.gk, dm.m, dm.scale,
                         kProbeChunk, partials);
    else
      hipLaunchKernelGGL((probe_attn_kernel<float, 64>), pgrid, dim3(256), 0, s, (const float*)q,
                         (const float*)part.k_gm, (const float*)part.v_gm, part.key_offsets, route.kept_mask,
                         out.probe_tokens, out.probe_groups, dm.n, dm.g, dm.gq, dm.gk, dm.m, dm.scale,
                         kProbeChunk, partials);
  }
  if (dm.d == 128)
    hipLaunchKernelGGL(probe_merge_kernel<128>, dim3(dm.m, dm.hq), dim3(128), 0, s, partials, wp.nchunks, dm.m,
                       fbuf, out.o_dense, out.o_sparse);
  else
    hipLaunchKernelGGL(probe_merge_kernel<64>, dim3(dm.m, dm.hq), dim3(64), 0, s, partials, wp.nchunks, dm.m,
                       fbuf, out.o_dense, out.o_sparse);
  if (dm.d == 128)
    hipLaunchKernelGGL(probe_fit_kernel<128>, dim3(dm.hq), dim3(256), 0, s, partials, wp.nchunks,
                       out.probe_weights, dm.g, dm.m, dm.r,
                       dm.ablation == SPARSEPR_ABLATE_RIDGE_ONLY ? 1 : 0, (double)dm.lambda, fbuf, out.o_dense, out.o_sparse,
                       out.A, out.B, out.c0, out.r_eff, out.eig);
  else
    hipLaunchKernelGGL(probe_fit_kernel<64>, dim3(dm.hq), dim3(256), 0, s, partials, wp.nchunks,
                       out.probe_weights, dm.g, dm.m, dm.r,
                       dm.ablation == SPARSEPR_ABLATE_RIDGE_ONLY ? 1 : 0, (double)dm.lambda, fbuf, out.o_dense, out.o_sparse,
                       out.A, out.B, out.c0, out.r_eff, out.eig);
}

}  // namespace sp
