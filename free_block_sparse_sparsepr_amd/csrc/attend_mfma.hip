// Matrix-core flash attention for bf16 (gfx950 MFMA 32x32x16), used both for the
// block-sparse SparsePR attention over the kept cells (summary page of "Partition the
// Support, Reconstruct the Residual", execution paragraph: exact on the selected cells,
// renormalised over the kept K/V groups) and for the dense baseline.
//
// Work decomposition: one block = 128 virtual query rows of one query group (4 waves x
// 32 rows); the block walks the group's kept key runs in 64-key tiles staged through LDS
// (double-buffered: the next tile's global loads are in flight while the current one is
// consumed).  Each wave computes S^T = K Q^T so that a lane owns one query and 32 of the
// tile's keys: the row max and sum are in-register plus one exchange with the partner
// lane (l ^ 32), and the probabilities are already laid out as the B operand of
// O^T += V^T P^T, so P never leaves registers.  V is stored transposed in LDS for that
// A operand.  Softmax runs in the log2 domain with scale * log2(e) folded in; P is
// rounded to bf16 for the second product and accumulation is fp32.
//
// Blocks are remapped so that consecutive tiles of one query group run on the same XCD
// (the hardware deals blocks round-robin over the 8 XCDs), keeping a group's key runs
// hot in that XCD's L2.
#include "sp_attn.hpp"
#include "sp_common.hpp"
#include "sp_launch.hpp"

namespace sp {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kXcds = 8;

template <int D>
struct MfmaCfg {
  static constexpr int BM = 128;           // virtual query rows per block
  static constexpr int BN = 64;            // keys per tile
  static constexpr int KROW = D + 8;       // LDS row of K (bf16), padded: conflict-free 16-byte reads
  static constexpr int VROW = BN + 4;      // LDS row of V^T (bf16), padded: conflict-free 8-byte reads
  static constexpr int KSTEPS = D / 16;    // MFMA k-steps over d
  static constexpr int DBLK = D / 32;      // 32-wide output blocks over d
};

// Key-tile iterator over the kept runs of a tile (uniform across the block).
struct TileIter {
  int ci, k0, k1, kt;
  bool valid;
};

__device__ __forceinline__ void iter_first(const AttnArgs& A, int kv, const TileInfo& ti, TileIter& it) {
  it.ci = ti.kbeg < 0 ? 0 : ti.kbeg;
  it.valid = next_run(A, kv, ti, it.ci, it.k0, it.k1);
  it.kt = it.k0;
}

__device__ __forceinline__ void iter_next(const AttnArgs& A, int kv, const TileInfo& ti, TileIter& it, int BN) {
  it.kt += BN;
  if (it.kt < it.k1) return;
  it.valid = next_run(A, kv, ti, it.ci, it.k0, it.k1);
  it.kt = it.k0;
}

__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }

template <int D>
struct Stage {
  uint4 k[4];
  uint4 v[4];
};

// Global -> registers for one K/V tile.  K: thread t loads D / 2 contiguous bytes of key
// t % 64 at d = (t / 64) D / 4; V (d = 128): 16 bytes of each of keys 4 (t % 16) .. +3
// at d = 8 (t / 16); V (d = 64): keys 2 (t % 32), +1 at d = 8 (t / 32).  Rows at or beyond
// k1 are zero.
template <int D>
__device__ __forceinline__ void stage_load(const bf16_t* __restrict__ kb, const bf16_t* __restrict__ vb, int kt,
                                           int k1, int tid, Stage<D>& st) {
  static_assert(D == 128 || D == 64, "head dim");
  constexpr int KV = D / 64;                  // 16-byte chunks per thread per operand / 2
  const int key = tid & 63, c = (tid >> 6) * (D / 4);
  const bool in = kt + key < k1;
  const uint4* src = reinterpret_cast<const uint4*>(kb + (int64_t)(kt + key) * D + c);
#pragma unroll
  for (int i = 0; i < 2 * KV; ++i) st.k[i] = in ? src[i] : make_uint4(0, 0, 0, 0);
  if constexpr (D == 128) {
    const int kq = tid & 15, dc = (tid >> 4) * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key2 = 4 * kq + i;
      st.v[i] = (kt + key2 < k1) ? *reinterpret_cast<const uint4*>(vb + (int64_t)(kt + key2) * D + dc)
                                 : make_uint4(0, 0, 0, 0);
    }
  } else {
    const int kp = tid & 31, dc = (tid >> 5) * 8;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int key2 = 2 * kp + i;
      st.v[i] = (kt + key2 < k1) ? *reinterpret_cast<const uint4*>(vb + (int64_t)(kt + key2) * D + dc)
                                 : make_uint4(0, 0, 0, 0);
    }
  }
}

// Registers -> LDS (K row-major, V transposed).  Consecutive lanes write consecutive
// keys (K rows 272 bytes apart, V^T words 8 bytes apart), so the stores are free of bank
// conflicts.
template <int D>
__device__ __forceinline__ void stage_store(bf16_t* __restrict__ Ks, bf16_t* __restrict__ Vt, int tid,
                                            const Stage<D>& st) {
  using C = MfmaCfg<D>;
  constexpr int KV = D / 64;
  const int key = tid & 63, c = (tid >> 6) * (D / 4);
  uint4* dst = reinterpret_cast<uint4*>(Ks + key * C::KROW + c);
#pragma unroll
  for (int i = 0; i < 2 * KV; ++i) dst[i] = st.k[i];
  if constexpr (D == 128) {
    const int kq = tid & 15, dc = (tid >> 4) * 8;
    const uint32_t* x0 = reinterpret_cast<const uint32_t*>(&st.v[0]);
    const uint32_t* x1 = reinterpret_cast<const uint32_t*>(&st.v[1]);
    const uint32_t* x2 = reinterpret_cast<const uint32_t*>(&st.v[2]);
    const uint32_t* x3 = reinterpret_cast<const uint32_t*>(&st.v[3]);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint2 lo = make_uint2(pack_lo(x0[w], x1[w]), pack_lo(x2[w], x3[w]));
      uint2 hi = make_uint2(pack_hi(x0[w], x1[w]), pack_hi(x2[w], x3[w]));
      *reinterpret_cast<uint2*>(Vt + (dc + 2 * w) * C::VROW + 4 * kq) = lo;
      *reinterpret_cast<uint2*>(Vt + (dc + 2 * w + 1) * C::VROW + 4 * kq) = hi;
    }
  } else {
    const int kp = tid & 31, dc = (tid >> 5) * 8;
    const uint32_t* x0 = reinterpret_cast<const uint32_t*>(&st.v[0]);
    const uint32_t* x1 = reinterpret_cast<const uint32_t*>(&st.v[1]);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      *reinterpret_cast<uint32_t*>(Vt + (dc + 2 * w) * C::VROW + 2 * kp) = pack_lo(x0[w], x1[w]);
      *reinterpret_cast<uint32_t*>(Vt + (dc + 2 * w + 1) * C::VROW + 2 * kp) = pack_hi(x0[w], x1[w]);
    }
  }
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
union PackP {
  bf16x8_t v;
  bf16x2_t h[4];
};

// A row max may go stale by up to this much (log2 units) before O and l are rescaled:
// probabilities stay below 2^8 and most tiles skip the rescale entirely.
constexpr float kStaleMax = 8.f;

// One 64-key tile of the online softmax for a wave's 32 queries: S^T = K Q^T on the
// matrix cores (two independent accumulation chains), masking (keys at or beyond nk,
// only on partial tiles; with MASK, keys whose group bit is clear in rowmask), the row
// max (in-register plus the partner lane), p = exp2(s c2 - m) with one FMA and the raw
// hardware exp2, bf16 packing, the row sum as bf16 dot products of the packed p (the
// same values the second product consumes), a lazy rescale, and O^T += V^T P^T.
template <int D, bool MASK>
__device__ __forceinline__ void mfma_tile_step(const bf16_t* __restrict__ ks, const bf16_t* __restrict__ vt,
                                               const bf16x8_t* qreg, int nk, float c2,
                                               const uint8_t* __restrict__ klab, uint64_t rowmask, float& m_i,
                                               float& l_i, f32x16_t* o, int l32, int hf) {
  using C = MfmaCfg<D>;
  f32x16_t s0, s1;
#pragma unroll
  for (int r = 0; r < 16; ++r) { s0[r] = 0.f; s1[r] = 0.f; }
  {
    const bf16_t* k0 = ks + l32 * C::KROW + 8 * hf;
    const bf16_t* k1 = ks + (32 + l32) * C::KROW + 8 * hf;
#pragma unroll
    for (int kk = 0; kk < C::KSTEPS; ++kk) {
      const bf16x8_t a0 = *reinterpret_cast<const bf16x8_t*>(k0 + 16 * kk);
      const bf16x8_t a1 = *reinterpret_cast<const bf16x8_t*>(k1 + 16 * kk);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qreg[kk], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qreg[kk], s1, 0, 0, 0);
    }
  }
  f32x16_t sv[2] = {s0, s1};
  if (MASK || nk < C::BN) {
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * kb2 + 8 * (r >> 2) + 4 * hf + (r & 3);
        bool keep = key < nk;
        if constexpr (MASK) keep = keep && ((rowmask >> klab[key]) & 1ull);
        sv[kb2][r] = keep ? sv[kb2][r] : -INFINITY;
      }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sv[kb2][r]);
  mx = fmaxf(mx, __shfl_xor(mx, 32)) * c2;
  const float m_use = (mx > m_i + kStaleMax) ? mx : m_i;
  float alpha;
  if constexpr (MASK) alpha = (m_use == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_i - m_use);
  else alpha = __builtin_amdgcn_exp2f(m_i - m_use);
  const float neg = -m_use;
  bf16x2_t ones;
  ones[0] = (__bf16)1.f;
  ones[1] = (__bf16)1.f;
  float rs = 0.f;
  PackP p[2][2];
#pragma unroll
  for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      float e0 = __builtin_amdgcn_exp2f(fmaf(sv[kb2][r], c2, neg));
      float e1 = __builtin_amdgcn_exp2f(fmaf(sv[kb2][r + 1], c2, neg));
      if constexpr (MASK) {
        e0 = (sv[kb2][r] == -INFINITY) ? 0.f : e0;
        e1 = (sv[kb2][r + 1] == -INFINITY) ? 0.f : e1;
      }
      bf16x2_t pr;
      pr[0] = (__bf16)e0;
      pr[1] = (__bf16)e1;
      p[kb2][r >> 3].h[(r & 7) >> 1] = pr;
      rs = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, rs, false);
    }
  l_i = l_i * alpha + rs;
  m_i = m_use;
  if (__ballot(alpha != 1.f)) {
#pragma unroll
    for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
  }
  // O^T += V^T P^T over the 4 key k-steps of the tile
#pragma unroll
  for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int koff = 32 * kb2 + 16 * s2 + 4 * hf;
#pragma unroll
      for (int db = 0; db < C::DBLK; ++db) {
        const bf16_t* vr = vt + (32 * db + l32) * C::VROW + koff;
        uint2 lo = *reinterpret_cast<const uint2*>(vr);
        uint2 hi = *reinterpret_cast<const uint2*>(vr + 8);
        uint4 av = make_uint4(lo.x, lo.y, hi.x, hi.y);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, av), p[kb2][s2].v, o[db], 0,
                                                        0, 0);
      }
    }
}

template <int D, typename OutT>
__global__ __launch_bounds__(256, 2) void attn_mfma_kernel(AttnArgs A) {
  using C = MfmaCfg<D>;
  __shared__ __attribute__((aligned(16))) bf16_t Ks[2][C::BN * C::KROW];
  __shared__ __attribute__((aligned(16))) bf16_t Vt[2][D * C::VROW];

  // XCD-aware remap of the linear block id (consecutive logical tiles on one XCD)
  const int total = gridDim.x;
  const int per_xcd = total / kXcds;
  const int b = blockIdx.x;
  const int logical = (b % kXcds) * per_xcd + b / kXcds;
  const int kv = logical / A.tiles_per_head;
  const int t = logical % A.tiles_per_head;
  if (kv >= A.n_heads_kv) return;
  TileInfo ti;
  if (!find_tile(A, kv, t, C::BM, ti)) return;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const bf16_t* qb = static_cast<const bf16_t*>(A.q);
  const bf16_t* kb = static_cast<const bf16_t*>(A.k) + (int64_t)kv * A.kv_skv;
  const bf16_t* vb = static_cast<const bf16_t*>(A.v) + (int64_t)kv * A.kv_skv;

  // Q operand (B of S^T = K Q^T): lane holds Q[row l32][16 kk + 8 hf .. +7]
  const int vrow = ti.v0 + 32 * w + l32;
  const bool qvalid = vrow < ti.v1;
  bf16x8_t qreg[C::KSTEPS];
  {
    const bf16_t* qr = qb + (int64_t)kv * A.q_skv + (int64_t)(vrow / A.g) * A.q_sp + (int64_t)(vrow % A.g) * A.q_sj;
#pragma unroll
    for (int kk = 0; kk < C::KSTEPS; ++kk) {
      uint4 x = qvalid ? *reinterpret_cast<const uint4*>(qr + 16 * kk + 8 * hf) : make_uint4(0, 0, 0, 0);
      qreg[kk] = __builtin_bit_cast(bf16x8_t, x);
    }
  }

  const float c2 = A.scale * 1.4426950408889634f;   // scale * log2(e)
  float m_i = -INFINITY, l_i = 0.f;
  f32x16_t o[C::DBLK];
#pragma unroll
  for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;

  TileIter it;
  iter_first(A, kv, ti, it);
  Stage<D> st;
  if (it.valid) {
    stage_load<D>(kb, vb, it.kt, it.k1, tid, st);
    stage_store<D>(Ks[0], Vt[0], tid, st);
  }
  __syncthreads();
  int cur = 0;
  while (it.valid) {
    TileIter nx = it;
    iter_next(A, kv, ti, nx, C::BN);
    if (nx.valid) stage_load<D>(kb, vb, nx.kt, nx.k1, tid, st);

    mfma_tile_step<D, false>(Ks[cur], Vt[cur], qreg, it.k1 - it.kt, c2, nullptr, 0ull, m_i, l_i, o, l32, hf);
    if (nx.valid) stage_store<D>(Ks[cur ^ 1], Vt[cur ^ 1], tid, st);
    __syncthreads();
    cur ^= 1;
    it = nx;
  }

  // epilogue: O / l, LSE; lane writes query l32's d = 32 db + 8 j + 4 hf + 0..3
  const float l_tot = l_i + __shfl_xor(l_i, 32);
  if (qvalid) {
    const float inv = 1.f / l_tot;
    OutT* orow = static_cast<OutT*>(A.o) + (int64_t)kv * A.o_skv + (int64_t)(vrow / A.g) * A.o_sp +
                 (int64_t)(vrow % A.g) * A.o_sj;
#pragma unroll
    for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d0 = 32 * db + 8 * j + 4 * hf;
        if constexpr (sizeof(OutT) == 4) {
          float4 v4 = make_float4(o[db][4 * j] * inv, o[db][4 * j + 1] * inv, o[db][4 * j + 2] * inv,
                                  o[db][4 * j + 3] * inv);
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(orow) + d0) = v4;
        } else {
          uint2 v2 = make_uint2((uint32_t)f32_to_bf16(o[db][4 * j] * inv) |
                                    ((uint32_t)f32_to_bf16(o[db][4 * j + 1] * inv) << 16),
                                (uint32_t)f32_to_bf16(o[db][4 * j + 2] * inv) |
                                    ((uint32_t)f32_to_bf16(o[db][4 * j + 3] * inv) << 16));
          *reinterpret_cast<uint2*>(reinterpret_cast<bf16_t*>(orow) + d0) = v2;
        }
      }
    if (A.lse && hf == 0) A.lse[((int64_t)kv * A.n + vrow / A.g) * A.g + vrow % A.g] = (m_i + log2f(l_tot)) * 0.6931471805599453f;
  }
}


// ---------------------------------------------------------------------------------------
// Probe rows (summary page of "Partition the Support, Reconstruct the Residual",
// probe-fit residual reconstruction paragraph): the M <= 64 probe rows of a query head
// against one chunk of keys (group-major order), as two online softmaxes: waves 0-1 over
// every key (dense rows) and waves 2-3 over the keys whose group is kept for the probe's
// query group (sparse rows).  Writes unnormalised partials (o, m, l) with m in natural
// log units: partials [Hq][chunks][M][2][D + 2].  grid (chunks, Hq), block 256.
// ---------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 2) void probe_attn_mfma_kernel(const bf16_t* __restrict__ q,
                                                               const bf16_t* __restrict__ kgm,
                                                               const bf16_t* __restrict__ vgm,
                                                               const int32_t* __restrict__ koff,
                                                               const uint64_t* __restrict__ kept_mask,
                                                               const int32_t* __restrict__ ptok,
                                                               const int32_t* __restrict__ pgrp, int n, int g,
                                                               int Gq, int Gk, int M, float scale, int chunk,
                                                               float* __restrict__ partials) {
  using C = MfmaCfg<D>;
  __shared__ __attribute__((aligned(16))) bf16_t Ks[2][C::BN * C::KROW];
  __shared__ __attribute__((aligned(16))) bf16_t Vt[2][D * C::VROW];
  __shared__ uint8_t klab[2][C::BN];
  __shared__ int ko[kMaxGroups + 1];
  const int h = blockIdx.y, kv = h / g, ch = blockIdx.x, nch = gridDim.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int row = 32 * (w & 1) + l32;
  const bool sparse = (w >> 1) != 0;
  const int k0 = ch * chunk, k1 = min(n, k0 + chunk);
  for (int b = tid; b <= Gk; b += 256) ko[b] = koff[(int64_t)kv * (Gk + 1) + b];
  const bool rvalid = row < M;
  const uint64_t rowmask = rvalid ? kept_mask[(int64_t)kv * Gq + pgrp[kv * M + row]] : 0ull;
  bf16x8_t qreg[C::KSTEPS];
  {
    const bf16_t* qr = q + ((int64_t)h * n + (rvalid ? ptok[kv * M + row] : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < C::KSTEPS; ++kk) {
      uint4 x = rvalid ? *reinterpret_cast<const uint4*>(qr + 16 * kk + 8 * hf) : make_uint4(0, 0, 0, 0);
      qreg[kk] = __builtin_bit_cast(bf16x8_t, x);
    }
  }
  const bf16_t* kb = kgm + (int64_t)kv * n * D;
  const bf16_t* vb = vgm + (int64_t)kv * n * D;
  const float c2 = scale * 1.4426950408889634f;
  float m_i = -INFINITY, l_i = 0.f;
  f32x16_t o[C::DBLK];
#pragma unroll
  for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  __syncthreads();
  auto label_of = [&](int pos) {
    int lo = 0, hi = Gk - 1;  // last group b with ko[b] <= pos (always non-empty)
    while (lo < hi) { int mid = (lo + hi + 1) >> 1; if (ko[mid] <= pos) lo = mid; else hi = mid - 1; }
    return lo;
  };
  Stage<D> st;
  int kt = k0;
  if (kt < k1) {
    stage_load<D>(kb, vb, kt, k1, tid, st);
    stage_store<D>(Ks[0], Vt[0], tid, st);
    if (tid < C::BN) klab[0][tid] = (uint8_t)(kt + tid < k1 ? label_of(kt + tid) : 0);
  }
  __syncthreads();
  int cur = 0;
  while (kt < k1) {
    const int nt = kt + C::BN;
    if (nt < k1) stage_load<D>(kb, vb, nt, k1, tid, st);
    if (sparse)
      mfma_tile_step<D, true>(Ks[cur], Vt[cur], qreg, k1 - kt, c2, klab[cur], rowmask, m_i, l_i, o, l32, hf);
    else
      mfma_tile_step<D, false>(Ks[cur], Vt[cur], qreg, k1 - kt, c2, nullptr, 0ull, m_i, l_i, o, l32, hf);
    if (nt < k1) {
      stage_store<D>(Ks[cur ^ 1], Vt[cur ^ 1], tid, st);
      if (tid < C::BN) klab[cur ^ 1][tid] = (uint8_t)(nt + tid < k1 ? label_of(nt + tid) : 0);
    }
    __syncthreads();
    cur ^= 1;
    kt = nt;
  }
  const float l_tot = l_i + __shfl_xor(l_i, 32);
  if (rvalid) {
    float* pb = partials + (((int64_t)h * nch + ch) * M + row) * 2 * (D + 2) + (sparse ? D + 2 : 0);
#pragma unroll
    for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d0 = 32 * db + 8 * j + 4 * hf;
#pragma unroll
        for (int e = 0; e < 4; ++e) pb[d0 + e] = o[db][4 * j + e];
      }
    if (hf == 0) {
      pb[D] = m_i == -INFINITY ? -INFINITY : m_i * 0.6931471805599453f;
      pb[D + 1] = l_tot;
    }
  }
}

void launch_probe_attn_mfma(const Dims& dm, const void* q, const sparsepr_partition_t& part,
                            const sparsepr_route_t& route, const sparsepr_fit_t& fit, int chunk, int nchunks,
                            float* partials, hipStream_t s) {
  const dim3 grid(nchunks, dm.hq);
  if (dm.d == 128)
    hipLaunchKernelGGL(probe_attn_mfma_kernel<128>, grid, dim3(256), 0, s, (const bf16_t*)q,
                       (const bf16_t*)part.k_gm, (const bf16_t*)part.v_gm, part.key_offsets, route.kept_mask,
                       fit.probe_tokens, fit.probe_groups, dm.n, dm.g, dm.gq, dm.gk, dm.m, dm.scale, chunk,
                       partials);
  else
    hipLaunchKernelGGL(probe_attn_mfma_kernel<64>, grid, dim3(256), 0, s, (const bf16_t*)q,
                       (const bf16_t*)part.k_gm, (const bf16_t*)part.v_gm, part.key_offsets, route.kept_mask,
                       fit.probe_tokens, fit.probe_groups, dm.n, dm.g, dm.gq, dm.gk, dm.m, dm.scale, chunk,
                       partials);
}

template <int D, typename OutT>
void launch_mfma_typed(AttnArgs a, int hkv, hipStream_t s) {
  a.tiles_per_head = (int)ceil_div((int64_t)a.n * a.g, MfmaCfg<D>::BM) + (a.qoff ? a.gq : 0);
  a.n_heads_kv = hkv;
  int64_t total = (int64_t)a.tiles_per_head * hkv;
  total = ceil_div(total, kXcds) * kXcds;
  hipLaunchKernelGGL((attn_mfma_kernel<D, OutT>), dim3((unsigned)total), dim3(256), 0, s, a);
}

void launch_attention_mfma(const Dims& dm, AttnArgs a, bool out_is_input_dtype, hipStream_t s) {
  if (out_is_input_dtype) {
    if (dm.d == 128) launch_mfma_typed<128, bf16_t>(a, dm.hkv, s); else launch_mfma_typed<64, bf16_t>(a, dm.hkv, s);
  } else {
    if (dm.d == 128) launch_mfma_typed<128, float>(a, dm.hkv, s); else launch_mfma_typed<64, float>(a, dm.hkv, s);
  }
}

}  // namespace sp
