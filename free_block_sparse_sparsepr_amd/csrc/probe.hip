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
  const double wgt = (double)M * (double)na / ((double)ma * (double)n);
  if (ma <= 4 || na > kSortMax) {
    // A few probes, or more members than the sort holds: each target rank of the order
    // (radius, position) by radix selection, four 8-bit digit passes over the radius (a
    // histogram of the members that match the digits found so far, then the bin that holds
    // the rank), then the ordered count, by position, of the members at that radius.
    __shared__ uint32_t hist[256];
    __shared__ int pick[2], wtot[4];
    const int lane = tid & 63, wv = tid >> 6;
    for (int k = 0; k < ma; ++k) {
      int r = tgt[k];
      uint32_t prefix = 0;
      for (int shift = 24; shift >= 0; shift -= 8) {
        hist[tid] = 0u;
        __syncthreads();
        for (int i = tid; i < na; i += 256) {
          const uint32_t x = (uint32_t)rad[i];
          if (shift == 24 || (x >> (shift + 8)) == prefix) atomicAdd(&hist[(x >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (tid < 64) {   // bins 4 tid .. 4 tid + 3 per lane, prefix sums across the wave
          const uint32_t hs[4] = {hist[4 * tid], hist[4 * tid + 1], hist[4 * tid + 2], hist[4 * tid + 3]};
          const uint32_t own = hs[0] + hs[1] + hs[2] + hs[3];
          uint32_t incl = own;
          for (int o = 1; o < 64; o <<= 1) {
            const uint32_t u = __shfl_up(incl, o);
            if (tid >= o) incl += u;
          }
          uint32_t c = incl - own;   // members in the bins below 4 tid
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if ((uint32_t)r >= c && (uint32_t)r < c + hs[j]) {
              pick[0] = 4 * tid + j;
              pick[1] = (int)c;
            }
            c += hs[j];
          }
        }
        __syncthreads();
        prefix = (prefix << 8) | (uint32_t)pick[0];
        r -= pick[1];
        __syncthreads();   // hist and pick are rewritten by the next pass
      }
      int base = 0;   // members at radius prefix among the positions before this chunk
      for (int i0 = 0; i0 < na; i0 += 256) {
        const int i = i0 + tid;
        const bool hit = i < na && (uint32_t)rad[i] == prefix;
        const uint64_t bal = __ballot(hit);
        if (lane == 0) wtot[wv] = __popcll(bal);
        __syncthreads();
        int woff = 0;
        for (int u = 0; u < wv; ++u) woff += wtot[u];
        const int tot = wtot[0] + wtot[1] + wtot[2] + wtot[3];
        if (hit && base + woff + __popcll(bal & ((1ull << lane) - 1ull)) == r) {
          const int slot = kv * M + start[a] + k;
          ptok[slot] = qperm[(int64_t)kv * n + off + i];
          pgrp[slot] = a;
          pw[slot] = wgt;
        }
        base += tot;
        __syncthreads();   // wtot is rewritten by the next chunk
        if (base > r) break;
      }
    }
    return;
  }
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
    pw[slot] = wgt;
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
  // each chunk's scale exp(m - max) is formed once, by one thread, into LDS; every thread
  // then adds its column over the chunks in chunk order (chunks without keys skipped)
  __shared__ double red[D], scs[D];
  const int r = blockIdx.x, h = blockIdx.y, c = threadIdx.x;
  const int64_t cstride = (int64_t)M * 2 * (D + 2);
  double res[2];
  for (int which = 0; which < 2; ++which) {
    const float* base = partials + (((int64_t)h * nch) * M + r) * 2 * (D + 2) + which * (D + 2);
    double mx = -INFINITY;
    for (int ch = c; ch < nch; ch += D) mx = fmax(mx, (double)base[ch * cstride + D]);
    red[c] = mx;
    __syncthreads();
    for (int s2 = D / 2; s2 > 0; s2 >>= 1) {
      if (c < s2) red[c] = fmax(red[c], red[c + s2]);
      __syncthreads();
    }
    mx = red[0];
    double L = 0.0, O = 0.0;
    for (int b0 = 0; b0 < nch; b0 += D) {
      const int ch = b0 + c;
      double sc = -1.0;   // no keys in the chunk
      if (ch < nch) {
        const double m = base[ch * cstride + D];
        if (m != -INFINITY) sc = exp(m - mx);
      }
      scs[c] = sc;
      __syncthreads();
      const int lim = min(D, nch - b0);
      for (int k = 0; k < lim; ++k) {
        const double s2 = scs[k];
        if (s2 < 0.0) continue;
        const float* pb = base + (int64_t)(b0 + k) * cstride;
        L += (double)pb[D + 1] * s2;
        O += (double)pb[c] * s2;
      }
      __syncthreads();   // scs and red are rewritten by the next pass
    }
    res[which] = O / L;
  }
  o_dense[((int64_t)h * M + r) * D + c] = (float)res[0];
  o_sparse[((int64_t)h * M + r) * D + c] = (float)res[1];
  double* fb = fbuf + (size_t)h * FitBuf::per_head(D);
  fb[FitBuf::x(D) + r * D + c] = res[1];
  fb[FitBuf::y(D) + r * D + c] = res[0] - res[1];
}

// The fit of each query head in float64, as three kernels.
//
// fit_gram_kernel, grid (4, Hq), block 256: blocks 0-1 stage X = O_sparse of the probe
// rows in LDS, form the weighted mean xbar and Xt = sqrt(w) (X - xbar) and each compute 32
// rows of the dual matrix K = Xt Xt^T + lambda I; blocks 2-3 do the same for the residuals
// Y (ybar, Yt) and the Gram matrix G = Yt Yt^T (zero-padded to 64 x 64).  Blocks 0 and 2
// also store Xt, xbar and Yt, ybar.
template <int D>
__global__ __launch_bounds__(256) void fit_gram_kernel(const double* __restrict__ pw, int g, int M, double lam,
                                                       double* __restrict__ fbuf) {
  constexpr int MM = kMaxProbe;
  __shared__ double S[MM][D + 1];
  __shared__ double w[MM], mean[D];
  const int h = blockIdx.y, kv = h / g, part = blockIdx.x, tid = threadIdx.x;
  const bool isK = part < 2;
  double* fb = fbuf + (size_t)h * FitBuf::per_head(D);
  const double* src = fb + (isK ? FitBuf::x(D) : FitBuf::y(D));
  if (tid < MM) w[tid] = tid < M ? pw[kv * M + tid] : 0.0;
  __syncthreads();
  double sw = 0.0;
  for (int r = 0; r < M; ++r) sw += w[r];
  for (int c = tid; c < D; c += 256) {
    double sx = 0.0;
    for (int r = 0; r < M; ++r) sx += w[r] * src[r * D + c];
    mean[c] = sx / sw;
  }
  __syncthreads();
  for (int idx = tid; idx < MM * D; idx += 256) {
    const int r = idx / D, c = idx % D;
    S[r][c] = r < M ? sqrt(w[r]) * (src[idx] - mean[c]) : 0.0;
  }
  __syncthreads();
  if ((part & 1) == 0) {
    double* dst = fb + (isK ? FitBuf::xt(D) : FitBuf::yt(D));
    for (int idx = tid; idx < M * D; idx += 256) dst[idx] = S[idx / D][idx % D];
    for (int c = tid; c < D; c += 256) fb[(isK ? FitBuf::xbar(D) : FitBuf::ybar(D)) + c] = mean[c];
  }
  double* out = fb + (isK ? FitBuf::k(D) : FitBuf::g(D));
  const int r0 = 32 * (part & 1);
  for (int idx = tid; idx < 32 * MM; idx += 256) {
    const int i = r0 + idx / MM, j = idx % MM;
    double v = 0.0;
    if (i < M && j < M)
      for (int c = 0; c < D; ++c) v += S[i][c] * S[j][c];
    if (isK && i == j) v += lam;
    out[i * MM + j] = v;
  }
}

// fit_factor_kernel, grid (2, Hq), block 256: block 0 factors K = L L^T (Cholesky, lower
// triangle in place); block 1 diagonalises G by parallel cyclic Jacobi (round-robin
// pairing: 32 disjoint rotations per step; a thread applies a step to four 2x2 blocks of G
// and to one pair's two columns in eight rows of V, every read issued before its writes),
// orders the eigenvalues (descending, ties by index), keeps those above 1e-8 of the largest
// (at most rank) and stores them with their
// eigenvectors a.  With ridge_only (the unprojected ridge) block 1 writes r_eff = M and
// zero eigenvalues.
template <int D>
__global__ __launch_bounds__(256) void fit_factor_kernel(int M, int rank, int ridge_only, double* __restrict__ fbuf,
                                                         int32_t* __restrict__ r_eff_out,
                                                         float* __restrict__ eig_out) {
  constexpr int MM = kMaxProbe;
  __shared__ double Km[MM][MM + 1];
  __shared__ double Vm[MM][MM + 1];
  __shared__ double rc[32], rs[32], ev[MM], red[256];
  __shared__ int ord[MM];
  __shared__ int stop_s;
  const int h = blockIdx.y, tid = threadIdx.x;
  double* fb = fbuf + (size_t)h * FitBuf::per_head(D);
  if (blockIdx.x == 0) {
    double* K = fb + FitBuf::k(D);
    for (int idx = tid; idx < MM * MM; idx += 256) Km[idx / MM][idx % MM] = K[idx];
    __syncthreads();
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
    for (int idx = tid; idx < MM * MM; idx += 256) K[idx] = Km[idx / MM][idx % MM];
    return;
  }
  if (ridge_only) {
    for (int k = tid; k <= rank; k += 256) eig_out[(int64_t)h * (rank + 1) + k] = 0.f;
    if (tid == 0) {
      r_eff_out[h] = M;
      fb[FitBuf::reff(D)] = (double)M;
    }
    return;
  }
  const double* G = fb + FitBuf::g(D);
  for (int idx = tid; idx < MM * MM; idx += 256) {
    const int i = idx / MM, j = idx % MM;
    Km[i][j] = G[idx];
    Vm[i][j] = (i == j) ? 1.0 : 0.0;
  }
  __syncthreads();
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
    // stop once the off-diagonal energy is below 1e-12 of the diagonal's (a relative norm
    // of 1e-6): on real probe residuals the rank-16 projector then agrees with a full
    // eigendecomposition to about 1e-7, and the sweeps that would tidy the small
    // eigenvalues' block (up to three of eleven) are skipped
    if (tid == 0) stop_s = (off_all <= 1e-12 * red[0]) || (off_all == 0.0);
    __syncthreads();
    if (stop_s) break;
    for (int t = 0; t < MM - 1; ++t) {
      if (tid < 32) {
        int p, q;
        jacobi_pair(t, tid, p, q);
        // t = tan(theta), the smaller root of t^2 + 2 tau t - 1 = 0 with tau = (a_qq - a_pp) /
        // (2 a_pq), written as |2 a_pq| / (|a_qq - a_pp| + hypot) with the sign of tau (+ for
        // tau = 0): one square root and one division, then c = 1 / sqrt(1 + t^2), s = t c
        const double apq = Km[p][q];
        double c = 1.0, s = 0.0;
        if (apq != 0.0) {
          const double dd = Km[q][q] - Km[p][p], a2 = 2.0 * apq;
          const double r = sqrt(fma(dd, dd, a2 * a2));
          if (r > 0.0) {
            double tt = fabs(a2) / (fabs(dd) + r);
            if (dd != 0.0 && ((dd < 0.0) != (a2 < 0.0))) tt = -tt;
            c = rsqrt(fma(tt, tt, 1.0));
            s = tt * c;
          }
        }
        rc[tid] = c;
        rs[tid] = s;
      }
      __syncthreads();
      {  // thread: column pair bj, row pairs r0 + 8k of G and rows r0 + 8m of V; every
         // operand read is issued before the first write (the blocks are disjoint)
        const int bj = tid & 31, r0 = tid >> 5;
        int pj, qj;
        jacobi_pair(t, bj, pj, qj);
        const double cj = rc[bj], sj = rs[bj];
        int pi[4], qi[4];
        double ci[4], si[4], a[4][4], vp[8], vq[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int bi = r0 + 8 * k;
          jacobi_pair(t, bi, pi[k], qi[k]);
          ci[k] = rc[bi];
          si[k] = rs[bi];
          a[k][0] = Km[pi[k]][pj];
          a[k][1] = Km[pi[k]][qj];
          a[k][2] = Km[qi[k]][pj];
          a[k][3] = Km[qi[k]][qj];
        }
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          vp[m] = Vm[r0 + 8 * m][pj];
          vq[m] = Vm[r0 + 8 * m][qj];
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const double t00 = a[k][0] * cj - a[k][1] * sj, t01 = a[k][0] * sj + a[k][1] * cj;
          const double t10 = a[k][2] * cj - a[k][3] * sj, t11 = a[k][2] * sj + a[k][3] * cj;
          const bool diag = r0 + 8 * k == bj;
          Km[pi[k]][pj] = ci[k] * t00 - si[k] * t10;
          Km[pi[k]][qj] = diag ? 0.0 : ci[k] * t01 - si[k] * t11;
          Km[qi[k]][pj] = diag ? 0.0 : si[k] * t00 + ci[k] * t10;
          Km[qi[k]][qj] = si[k] * t01 + ci[k] * t11;
        }
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          Vm[r0 + 8 * m][pj] = cj * vp[m] - sj * vq[m];
          Vm[r0 + 8 * m][qj] = sj * vp[m] + cj * vq[m];
        }
      }
      __syncthreads();
    }
  }
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
    r_eff_out[h] = re;
    fb[FitBuf::reff(D)] = (double)re;
  }
  for (int k = tid; k <= rank; k += 256) eig_out[(int64_t)h * (rank + 1) + k] = k < MM ? (float)ev[ord[k]] : 0.f;
  for (int idx = tid; idx < MM * kMaxRank; idx += 256) {
    const int i = idx / kMaxRank, k = idx % kMaxRank;
    fb[FitBuf::a(D) + idx] = Vm[i][ord[k]];
  }
  for (int k = tid; k < MM; k += 256) fb[FitBuf::ev(D) + k] = ev[ord[k]];
}

// fit_solve_kernel, grid Hq, block 256: Z = K^{-1} Yt by forward and back substitution
// with L and Z resident in LDS (one thread per output column), then either the
// unprojected ridge (A = Xt^T, B = Z, c0 = ybar - (xbar Xt^T) Z) or the projected fit:
// V_r[:, k] = Yt^T a_k / sqrt(lambda_k), A = Xt^T (Z V_r), B = V_r^T, c0 = ybar - (xbar A) B.
template <int D>
__global__ __launch_bounds__(256) void fit_solve_kernel(int M, int rank, int ridge_only,
                                                        const double* __restrict__ fbuf, float* __restrict__ Aout,
                                                        float* __restrict__ Bout, float* __restrict__ c0out) {
  constexpr int MM = kMaxProbe;
  __shared__ double La[MM][MM + 1];         // L, then a, then Z V_r
  __shared__ double Zs[MM * D];             // Z, then A
  __shared__ double Vr[D][kMaxRank + 1];
  __shared__ double xa[MM];
  const int h = blockIdx.x, tid = threadIdx.x;
  const double* fb = fbuf + (size_t)h * FitBuf::per_head(D);
  const double* Xt = fb + FitBuf::xt(D);
  const double* Yt = fb + FitBuf::yt(D);
  const double* xbar = fb + FitBuf::xbar(D);
  const double* ybar = fb + FitBuf::ybar(D);
  for (int idx = tid; idx < MM * MM; idx += 256) La[idx / MM][idx % MM] = fb[FitBuf::k(D) + idx];
  for (int idx = tid; idx < M * D; idx += 256) Zs[idx] = Yt[idx];
  __syncthreads();
  for (int c = tid; c < D; c += 256) {
    for (int i = 0; i < M; ++i) {
      double s = Zs[i * D + c];
      for (int k = 0; k < i; ++k) s -= La[i][k] * Zs[k * D + c];
      Zs[i * D + c] = s / La[i][i];
    }
    for (int i = M - 1; i >= 0; --i) {
      double s = Zs[i * D + c];
      for (int k = i + 1; k < M; ++k) s -= La[k][i] * Zs[k * D + c];
      Zs[i * D + c] = s / La[i][i];
    }
  }
  __syncthreads();
  if (ridge_only) {
    // xa[k] = xbar . Xt[k]; c0 = ybar - xa Z; A = Xt^T, B = Z (leading dimension M)
    for (int k = tid; k < M; k += 256) {
      double acc = 0.0;
      for (int c = 0; c < D; ++c) acc += xbar[c] * Xt[k * D + c];
      xa[k] = acc;
    }
    __syncthreads();
    for (int idx = tid; idx < D * M; idx += 256) {
      const int c = idx / M, k = idx % M;
      Aout[(int64_t)h * D * M + idx] = (float)Xt[k * D + c];
      Bout[(int64_t)h * M * D + (int64_t)k * D + c] = (float)Zs[k * D + c];
    }
    for (int c = tid; c < D; c += 256) {
      double acc = ybar[c];
      for (int k = 0; k < M; ++k) acc -= xa[k] * Zs[k * D + c];
      c0out[(int64_t)h * D + c] = (float)acc;
    }
    return;
  }
  const int re = (int)fb[FitBuf::reff(D)];
  for (int idx = tid; idx < MM * kMaxRank; idx += 256) La[idx / kMaxRank][idx % kMaxRank] = fb[FitBuf::a(D) + idx];
  __syncthreads();
  for (int c = tid; c < D; c += 256) {
    double acc[kMaxRank];
#pragma unroll
    for (int k = 0; k < kMaxRank; ++k) acc[k] = 0.0;
    for (int i = 0; i < M; ++i) {
      const double y = Yt[i * D + c];
#pragma unroll
      for (int k = 0; k < kMaxRank; ++k) acc[k] += y * La[i][k];
    }
#pragma unroll
    for (int k = 0; k < kMaxRank; ++k) Vr[c][k] = k < re ? acc[k] / sqrt(fb[FitBuf::ev(D) + k]) : 0.0;
  }
  __syncthreads();
  // Z V_r (M x r) into La
  for (int idx = tid; idx < M * kMaxRank; idx += 256) {
    const int i = idx / kMaxRank, k = idx % kMaxRank;
    double s = 0.0;
    if (k < re)
      for (int c = 0; c < D; ++c) s += Zs[i * D + c] * Vr[c][k];
    La[i][k] = s;
  }
  __syncthreads();
  // A = Xt^T (Z V_r) (D x r) into Zs
  for (int c = tid; c < D; c += 256) {
    double acc[kMaxRank];
#pragma unroll
    for (int k = 0; k < kMaxRank; ++k) acc[k] = 0.0;
    for (int i = 0; i < M; ++i) {
      const double x = Xt[i * D + c];
#pragma unroll
      for (int k = 0; k < kMaxRank; ++k) acc[k] += x * La[i][k];
    }
#pragma unroll
    for (int k = 0; k < kMaxRank; ++k) Zs[c * kMaxRank + k] = k < re ? acc[k] : 0.0;
  }
  __syncthreads();
  for (int k = tid; k < kMaxRank; k += 256) {
    double s = 0.0;
    for (int c = 0; c < D; ++c) s += xbar[c] * Zs[c * kMaxRank + k];
    xa[k] = s;
  }
  __syncthreads();
  // outputs: A [D][rank], B [rank][D], c0 = ybar - (xbar A) B
  for (int idx = tid; idx < D * rank; idx += 256) {
    const int c = idx / rank, k = idx % rank;
    Aout[(int64_t)h * D * rank + idx] = k < re ? (float)Zs[c * kMaxRank + k] : 0.f;
    Bout[(int64_t)h * rank * D + (int64_t)k * D + c] = k < re ? (float)Vr[c][k] : 0.f;
  }
  for (int c = tid; c < D; c += 256) {
    double s = ybar[c];
    for (int k = 0; k < re; ++k) s -= xa[k] * Vr[c][k];
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
    launch_probe_attn_mfma(dm, q, part, route, out, probe_chunk(dm.n), wp.nchunks, partials, s);
  } else {
    if (dm.d == 128)
      hipLaunchKernelGGL((probe_attn_kernel<float, 128>), pgrid, dim3(256), 0, s, (const float*)q,
                         (const float*)part.k_gm, (const float*)part.v_gm, part.key_offsets, route.kept_mask,
                         out.probe_tokens, out.probe_groups, dm.n, dm.g, dm.gq, dm.gk, dm.m, dm.scale,
                         probe_chunk(dm.n), partials);
    else
      hipLaunchKernelGGL((probe_attn_kernel<float, 64>), pgrid, dim3(256), 0, s, (const float*)q,
                         (const float*)part.k_gm, (const float*)part.v_gm, part.key_offsets, route.kept_mask,
                         out.probe_tokens, out.probe_groups, dm.n, dm.g, dm.gq, dm.gk, dm.m, dm.scale,
                         probe_chunk(dm.n), partials);
  }
  if (dm.d == 128)
    hipLaunchKernelGGL(probe_merge_kernel<128>, dim3(dm.m, dm.hq), dim3(128), 0, s, partials, wp.nchunks, dm.m,
                       fbuf, out.o_dense, out.o_sparse);
  else
    hipLaunchKernelGGL(probe_merge_kernel<64>, dim3(dm.m, dm.hq), dim3(64), 0, s, partials, wp.nchunks, dm.m,
                       fbuf, out.o_dense, out.o_sparse);
  const int ridge = dm.ablation == SPARSEPR_ABLATE_RIDGE_ONLY ? 1 : 0;
  if (dm.d == 128) {
    hipLaunchKernelGGL(fit_gram_kernel<128>, dim3(4, dm.hq), dim3(256), 0, s, out.probe_weights, dm.g, dm.m,
                       (double)dm.lambda, fbuf);
    hipLaunchKernelGGL(fit_factor_kernel<128>, dim3(2, dm.hq), dim3(256), 0, s, dm.m, dm.r, ridge, fbuf, out.r_eff,
                       out.eig);
    hipLaunchKernelGGL(fit_solve_kernel<128>, dim3(dm.hq), dim3(256), 0, s, dm.m, dm.r, ridge, fbuf, out.A, out.B,
                       out.c0);
  } else {
    hipLaunchKernelGGL(fit_gram_kernel<64>, dim3(4, dm.hq), dim3(256), 0, s, out.probe_weights, dm.g, dm.m,
                       (double)dm.lambda, fbuf);
    hipLaunchKernelGGL(fit_factor_kernel<64>, dim3(2, dm.hq), dim3(256), 0, s, dm.m, dm.r, ridge, fbuf, out.r_eff,
                       out.eig);
    hipLaunchKernelGGL(fit_solve_kernel<64>, dim3(dm.hq), dim3(256), 0, s, dm.m, dm.r, ridge, fbuf, out.A, out.B,
                       out.c0);
  }
}

}  // namespace sp
