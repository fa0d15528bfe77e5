// Matrix-core flash attention for bf16 (gfx950 MFMA 32x32x16), used both for the
// block-sparse SparsePR attention over the kept cells (summary page of "Partition the
// Support, Reconstruct the Residual", execution paragraph: exact on the selected cells,
// renormalised over the kept K/V groups) and for the dense baseline.
//
// Work decomposition: one block = 256 virtual query rows of one query group (8 waves x
// 32 rows); the block walks the group's kept key runs in 64-key tiles staged through LDS
// (four stages filled by direct global-to-LDS copies two tiles ahead).  Each wave computes
// S^T = K Q^T so that a lane owns one query and 32 of the tile's keys: the row max and sum
// are in-register plus one exchange with the partner lane (l ^ 32), and the probabilities
// are already laid out as the B operand of O^T += V^T P^T, so P never leaves registers.
// V is stored transposed in LDS for that A operand.  Softmax runs in the log2 domain with
// scale * log2(e) folded in; P is rounded to bf16 for the second product and accumulation
// is fp32.  The two waves of every SIMD run anti-phased, one block barrier per tile: while
// one issues a tile's matrix products (with its LDS operand reads kept six deep, as one
// assembly block for d = 128), the other runs its softmax; one of the two also copies the
// tiles.
//
// Blocks are remapped so that consecutive tiles of one query group run on the same XCD
// (the hardware deals blocks round-robin over the 8 XCDs), keeping a group's key runs
// hot in that XCD's L2; a head's tiles stay together, its query groups longest first.
#include "sp_attn.hpp"
#include "sp_common.hpp"
#include "sp_launch.hpp"

namespace sp {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kXcds = 8;
// A row max may go stale by up to this much (log2 units) before O and l are rescaled:
// probabilities stay below 2^8 and most tiles skip the rescale entirely.
constexpr float kStaleMax = 8.f;

template <int D, int BN_ = 32, int NW_ = 4>
struct MfmaCfg {
  static constexpr int NW = NW_;            // waves per block (32 query rows each)
  static constexpr int BM = 32 * NW;        // virtual query rows per block
  static constexpr int BN = BN_;            // keys per tile (32 or 64)
  static constexpr int NB = BN / 32;        // 32-key score blocks per tile
  static constexpr int KCH = D / 8;         // 16-byte chunks per K row
  static constexpr int VCH = BN / 8;        // 16-byte chunks per V^T row
  static constexpr int KBYTES = BN * D * 2; // K stage: BN rows, chunk c of row r at slot c ^ kswz(r)
  static constexpr int VBYTES = D * BN * 2; // V^T stage: D rows of BN keys, chunk c of row d at slot c ^ vswz(d)
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int KIPW = BN * KCH / (64 * NW);   // K copy instructions per wave
  static constexpr int VIPW = D * VCH / (64 * NW);
  static_assert(KIPW >= 1 && VIPW >= 1, "tile too small for the block's copy lanes");
  static constexpr int KSTEPS = D / 16;
  static constexpr int DBLK = D / 32;
  // chunk swizzle of K row r: 16 consecutive rows read at one chunk offset (the 16 lanes
  // of one LDS cycle of a 16-byte read) hit distinct banks; 256-byte rows (d = 128) each
  // fill the bank window, 128-byte rows (d = 64) share it in pairs
  __device__ static int kswz(int r) { return KCH == 16 ? (r & 15) : ((r >> 1) & 7); }
  // chunk swizzle of V^T row d: rows that share a bank window (every second row for
  // 128-byte rows, every fourth for 64-byte rows) see distinct chunk slots, so 16
  // consecutive rows read at one chunk offset hit distinct banks
  __device__ static int vswz(int d) { return VCH == 8 ? ((d >> 1) & 7) : ((d >> 2) & 3); }
};

// Key tiles walk the kept runs of a query tile (uniform across the block).  Tiles start
// on 16-key boundaries so that the transposed V's 16-key groups are aligned; keys of a
// tile outside its run [k0, k1) are masked.
// The runs of next_run, listed once per block in LDS by one wave: lane t takes CSR column t
// of the query group; a column starts a run unless it follows its predecessor's group, a run
// ends before the next start, and runs without keys are dropped (ballot + rank).  The
// block's iterators then read one LDS entry per run: loads of the CSR columns from global
// memory would wait behind the tile copies in flight (the counter of vector memory
// operations is in order).
__device__ __forceinline__ void build_runs(const AttnArgs& A, int kv, const TileInfo& ti, int lane, int2* runs,
                                           int* nruns) {
  if (ti.kbeg < 0) {   // the dense schedule: one run over every key
    if (lane == 0) {
      runs[0] = make_int2(0, A.n);
      *nruns = 1;
    }
    return;
  }
  const int32_t* cl = A.cols + (int64_t)kv * A.gq * A.gk;
  const int32_t* ko = A.koff + (int64_t)kv * (A.gk + 1);
  const int cnt = ti.kend - ti.kbeg;   // <= G_K <= 64
  const int b = lane < cnt ? cl[ti.kbeg + lane] : 0;
  const int pb = __shfl(b, lane > 0 ? lane - 1 : 0);
  const bool start = lane < cnt && (lane == 0 || pb + 1 != b);
  const uint64_t sm = __ballot(start);
  const uint64_t after = sm & ~((2ull << lane) - 1ull);   // starts above this lane
  const int e = after ? __ffsll((unsigned long long)after) - 2 : cnt - 1;
  const int be = __shfl(b, e < 0 ? 0 : e);
  int k0 = 0, k1 = 0;
  if (start) {
    k0 = ko[b];
    k1 = ko[be + 1];
  }
  const bool keep = start && k1 > k0;
  const uint64_t km = __ballot(keep);
  if (keep) runs[__popcll(km & ((1ull << lane) - 1ull))] = make_int2(k0, k1);
  if (lane == 0) *nruns = __popcll(km);
}

// Advances (ri, k0, k1, kt) to the next tile (ri: the next run); false after the last one.
__device__ __forceinline__ bool next_tile_lds(const int2* runs, int nruns, int BN, int& ri, int& k0, int& k1,
                                              int& kt) {
  kt += BN;
  if (kt < k1) return true;
  if (ri >= nruns) return false;
  const int2 r = runs[ri++];
  k0 = __builtin_amdgcn_readfirstlane(r.x);
  k1 = __builtin_amdgcn_readfirstlane(r.y);
  kt = k0 & ~15;
  return true;
}

// Global -> LDS copy of one tile (K rows kt.., V^T columns kt..) with the direct
// global-to-LDS path: lane i of a copy instruction lands at the instruction's LDS base +
// 16 i, so each lane fetches the global chunk that belongs at its LDS slot.  A lane's
// source offsets relative to the tile (CopyPlan, fixed for the whole kernel) and a
// wave-uniform tile base make an interior tile's copies address arithmetic-free; the
// last tile of the sequence clamps rows beyond n (those keys are masked).
__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// 32-bit LDS byte address of a pointer into a __shared__ array
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

template <int D, int BN, int NW>
struct CopyPlan {
  using C = MfmaCfg<D, BN, NW>;
  uint32_t koff[C::KIPW];   // bytes from the tile's first K row
  uint32_t voff[C::VIPW];   // bytes from the tile's first V^T column
  int w, lane;

  __device__ CopyPlan(int w_, int lane_, int np) : w(w_), lane(lane_) {
#pragma unroll
    for (int i = 0; i < C::KIPW; ++i) koff[i] = (uint32_t)(krow(i) * D + 8 * kchunk(i)) * 2u;
#pragma unroll
    for (int i = 0; i < C::VIPW; ++i) voff[i] = (uint32_t)(vrow(i) * np + vcol(i)) * 2u;
  }
  // K row within the tile and its chunk for copy instruction i (recomputed where needed,
  // so that only the byte offsets stay in registers)
  __device__ int krow(int i) const { return ((w * C::KIPW + i) * 64 + lane) / C::KCH; }
  __device__ int kchunk(int i) const {
    const int L = (w * C::KIPW + i) * 64 + lane;
    return (L % C::KCH) ^ C::kswz(L / C::KCH);
  }
  // V^T row (d) and column (key within the tile) for copy instruction i
  __device__ int vrow(int i) const { return ((w * C::VIPW + i) * 64 + lane) / C::VCH; }
  __device__ int vcol(int i) const {
    const int L = (w * C::VIPW + i) * 64 + lane;
    return 8 * ((L % C::VCH) ^ C::vswz(L / C::VCH));
  }
};

template <int D, int BN, int NW>
__device__ __forceinline__ void stage_copy(const CopyPlan<D, BN, NW>& cp, const bf16_t* __restrict__ kb,
                                           const bf16_t* __restrict__ vtb, int n, int np, int kt, char* stage,
                                           int wu) {
  using C = MfmaCfg<D, BN, NW>;
  char* vst = stage + C::KBYTES;
  if (kt + BN <= n) {
    const char* kbase = reinterpret_cast<const char*>(kb + (int64_t)kt * D);
    const char* vbase = reinterpret_cast<const char*>(vtb + kt);
#pragma unroll
    for (int i = 0; i < C::KIPW; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(kbase + cp.koff[i]),
                                       (lds_void_t*)(stage + (wu * C::KIPW + i) * 1024), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < C::VIPW; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(vbase + cp.voff[i]),
                                       (lds_void_t*)(vst + (wu * C::VIPW + i) * 1024), 16, 0, 0);
    return;
  }
  // ragged tail: rows past n read row n - 1.  Byte offsets from the head's base are formed in
  // 32 bits (wrapping; the sums are the in-bounds offsets, below 2^30 at the largest n), so
  // that only koff / voff stay in registers across the loop.
#pragma unroll
  for (int i = 0; i < C::KIPW; ++i) {
    const int kr = cp.krow(i);
    const int row = min(kt + kr, n - 1);
    const uint32_t off = cp.koff[i] + (uint32_t)(row - kr) * (uint32_t)(D * 2);
    const char* src = reinterpret_cast<const char*>(kb) + off;
    __builtin_amdgcn_global_load_lds((const void*)src, (lds_void_t*)(stage + (wu * C::KIPW + i) * 1024), 16, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < C::VIPW; ++i) {
    const int vc = cp.vcol(i);
    const int pos = kt + vc;
    const int base = pos + 8 <= np ? kt : -vc;   // chunks past n_pad read the row's first chunk
    const uint32_t off = cp.voff[i] + (uint32_t)base * 2u;
    const char* src = reinterpret_cast<const char*>(vtb) + off;
    __builtin_amdgcn_global_load_lds((const void*)src, (lds_void_t*)(vst + (wu * C::VIPW + i) * 1024), 16, 0, 0);
  }
}

union PackP {
  bf16x8_t v;
  bf16x2_t h[4];
};

// The three parts of one tile (BN keys) of the online softmax for a wave's 32 queries.
// scores_mfma: S^T = K Q^T on the matrix cores (one accumulation chain per 32-key block).
template <int D, int BN>
__device__ __forceinline__ void scores_mfma(const char* __restrict__ stage, const bf16x8_t* qreg, f32x16_t* sv,
                                            int l32, int hf) {
  using C = MfmaCfg<D, BN>;
#pragma unroll
  for (int kb = 0; kb < C::NB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) sv[kb][r] = 0.f;
#pragma unroll
  for (int kk = 0; kk < C::KSTEPS; ++kk) {
#pragma unroll
    for (int kb = 0; kb < C::NB; ++kb) {
      const int row = 32 * kb + l32;
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(stage + row * (D * 2) + (((2 * kk + hf) ^ C::kswz(row)) << 4));
      sv[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[kk], sv[kb], 0, 0, 0);
    }
  }
}

// softmax_step: masking (keys outside [lo, hi) of the tile; with MASK also keys whose
// group bit is clear in rowmask), the row max (in-register plus the partner lane l ^ 32),
// p = exp2(s c2 - m) with one FMA and the hardware exp2, bf16 packing into the B-operand
// layout of the second product, the row sum as bf16 dot products of the packed p (the
// values the second product consumes) and a lazy rescale of O.
template <int D, int BN, bool MASK>
__device__ __forceinline__ void softmax_step(f32x16_t* sv, int lo, int hi, float c2, const uint8_t* __restrict__ klab,
                                             uint64_t rowmask, float& m_i, float& l_i, f32x16_t* o,
                                             PackP (*p)[2], int hf) {
  using C = MfmaCfg<D, BN>;
  if (MASK || lo > 0 || hi < C::BN) {
#pragma unroll
    for (int kb = 0; kb < C::NB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * kb + 8 * (r >> 2) + 4 * hf + (r & 3);
        bool keep = key >= lo && key < hi;
        if constexpr (MASK) keep = keep && ((rowmask >> klab[key]) & 1ull);
        sv[kb][r] = keep ? sv[kb][r] : -INFINITY;
      }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < C::NB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sv[kb][r]);
  mx = max_xor32(mx) * c2;
  const float m_use = (mx > m_i + kStaleMax) ? mx : m_i;
  float alpha;
  if constexpr (MASK) alpha = (m_use == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_i - m_use);
  else alpha = __builtin_amdgcn_exp2f(m_i - m_use);
  const float neg = -m_use;
  bf16x2_t ones;
  ones[0] = (__bf16)1.f;
  ones[1] = (__bf16)1.f;
  float rs = 0.f;
#pragma unroll
  for (int kb = 0; kb < C::NB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      float e0 = __builtin_amdgcn_exp2f(fmaf(sv[kb][r], c2, neg));
      float e1 = __builtin_amdgcn_exp2f(fmaf(sv[kb][r + 1], c2, neg));
      if constexpr (MASK) {
        e0 = (sv[kb][r] == -INFINITY) ? 0.f : e0;
        e1 = (sv[kb][r + 1] == -INFINITY) ? 0.f : e1;
      }
      bf16x2_t pr;
      pr[0] = (__bf16)e0;
      pr[1] = (__bf16)e1;
      p[kb][r >> 3].h[(r & 7) >> 1] = pr;
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
}

// pv_mfma: O^T += V^T P^T.  Key k-step (kb, s2) covers keys 32 kb + 16 s2 + {4 hf + 0..3,
// 8 + 4 hf + 0..3}, which the V^T layout keeps as chunk 2 (2 kb + s2) + hf of the row.
template <int D, int BN>
__device__ __forceinline__ void pv_mfma(const char* __restrict__ stage, const PackP (*p)[2], f32x16_t* o, int l32,
                                        int hf) {
  using C = MfmaCfg<D, BN>;
  const char* vst = stage + C::KBYTES;
#pragma unroll
  for (int kb = 0; kb < C::NB; ++kb)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
      for (int db = 0; db < C::DBLK; ++db) {
        const int d = 32 * db + l32;
        const char* vr = vst + d * (C::BN * 2);
        const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(vr + (((4 * kb + 2 * s2 + hf) ^ C::vswz(d)) << 4));
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, p[kb][s2].v, o[db], 0, 0, 0);
      }
    }
}

// The probe rows' softmax: as softmax_step, but the probabilities are split into a bf16
// high part and a bf16 remainder (p = hi + lo to about 2^-16 relative), both laid out as
// B operands, and the row sum is formed from the float probabilities, so that the probe
// rows' O^T += V^T (hi + lo)^T carries no bf16 rounding of P.
template <int D, int BN, bool MASK>
__device__ __forceinline__ void softmax_step_split(f32x16_t* sv, int hi_key, float c2,
                                                   const uint8_t* __restrict__ klab, uint64_t rowmask, float& m_i,
                                                   float& l_i, f32x16_t* o, PackP (*ph)[2], PackP (*pl)[2],
                                                   int hf) {
  using C = MfmaCfg<D, BN>;
#pragma unroll
  for (int kb = 0; kb < C::NB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 32 * kb + 8 * (r >> 2) + 4 * hf + (r & 3);
      bool keep = key < hi_key;
      if constexpr (MASK) keep = keep && ((rowmask >> klab[key]) & 1ull);
      sv[kb][r] = keep ? sv[kb][r] : -INFINITY;
    }
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < C::NB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sv[kb][r]);
  mx = max_xor32(mx) * c2;
  const float m_use = (mx > m_i + kStaleMax) ? mx : m_i;
  const float alpha = (m_use == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_i - m_use);
  const float neg = -m_use;
  float rs = 0.f;
#pragma unroll
  for (int kb = 0; kb < C::NB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      float e0 = __builtin_amdgcn_exp2f(fmaf(sv[kb][r], c2, neg));
      float e1 = __builtin_amdgcn_exp2f(fmaf(sv[kb][r + 1], c2, neg));
      e0 = (sv[kb][r] == -INFINITY) ? 0.f : e0;
      e1 = (sv[kb][r + 1] == -INFINITY) ? 0.f : e1;
      bf16x2_t h, l;
      h[0] = (__bf16)e0;
      h[1] = (__bf16)e1;
      l[0] = (__bf16)(e0 - (float)h[0]);
      l[1] = (__bf16)(e1 - (float)h[1]);
      ph[kb][r >> 3].h[(r & 7) >> 1] = h;
      pl[kb][r >> 3].h[(r & 7) >> 1] = l;
      rs += e0 + e1;
    }
  l_i = l_i * alpha + rs;
  m_i = m_use;
  if (__ballot(alpha != 1.f)) {
#pragma unroll
    for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
  }
}

template <int D, int BN, bool MASK>
__device__ __forceinline__ void probe_tile_step(const char* __restrict__ stage, const bf16x8_t* qreg, int hi_key,
                                                float c2, const uint8_t* __restrict__ klab, uint64_t rowmask,
                                                float& m_i, float& l_i, f32x16_t* o, int l32, int hf) {
  using C = MfmaCfg<D, BN>;
  f32x16_t sv[C::NB];
  PackP ph[C::NB][2], pl[C::NB][2];
  scores_mfma<D, BN>(stage, qreg, sv, l32, hf);
  softmax_step_split<D, BN, MASK>(sv, hi_key, c2, klab, rowmask, m_i, l_i, o, ph, pl, hf);
  pv_mfma<D, BN>(stage, ph, o, l32, hf);
  pv_mfma<D, BN>(stage, pl, o, l32, hf);
}

// The matrix phase of the anti-phased schedule: O^T += V^T P^T of the previous tile and
// S^T = K Q^T of the current one as one straight-line block, with the LDS operand reads
// issued LA products ahead of their use (the partner wave of the SIMD runs its softmax
// meanwhile, so this wave must hide its own LDS latency).
template <int D, int BN, int LA>
__device__ __forceinline__ void matrix_phase(const char* __restrict__ kstage, const char* __restrict__ vstage,
                                             const bf16x8_t* qreg, const PackP (*p)[2], f32x16_t* o,
                                             f32x16_t* sv, int l32, int hf) {
  using C = MfmaCfg<D, BN>;
  constexpr int NPV = C::NB * 2 * C::DBLK, NS = C::NB * C::KSTEPS, T = NPV + NS;
  bf16x8_t va[NPV], ka[NS];
  const char* vst = vstage + C::KBYTES;
#pragma unroll
  for (int kb = 0; kb < C::NB; ++kb)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int db = 0; db < C::DBLK; ++db) {
        const int d = 32 * db + l32;
        va[(kb * 2 + s2) * C::DBLK + db] = *reinterpret_cast<const bf16x8_t*>(
            vst + d * (C::BN * 2) + (((4 * kb + 2 * s2 + hf) ^ C::vswz(d)) << 4));
      }
#pragma unroll
  for (int kk = 0; kk < C::KSTEPS; ++kk)
#pragma unroll
    for (int kb = 0; kb < C::NB; ++kb) {
      const int row = 32 * kb + l32;
      ka[kk * C::NB + kb] =
          *reinterpret_cast<const bf16x8_t*>(kstage + row * (D * 2) + (((2 * kk + hf) ^ C::kswz(row)) << 4));
    }
#pragma unroll
  for (int kb = 0; kb < C::NB; ++kb)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int db = 0; db < C::DBLK; ++db)
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[(kb * 2 + s2) * C::DBLK + db], p[kb][s2].v, o[db], 0, 0, 0);
#pragma unroll
  for (int kb = 0; kb < C::NB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) sv[kb][r] = 0.f;
#pragma unroll
  for (int kk = 0; kk < C::KSTEPS; ++kk)
#pragma unroll
    for (int kb = 0; kb < C::NB; ++kb)
      sv[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kk * C::NB + kb], qreg[kk], sv[kb], 0, 0, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, LA, 0);   // LA operand reads
#pragma unroll
  for (int i = 0; i < T - LA; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one product
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // the read LA products ahead
  }
  __builtin_amdgcn_sched_group_barrier(0x008, LA, 0);
}

// The matrix phase for d = 128 and 64-key tiles as one self-contained assembly block: O^T +=
// V^T P^T of the previous tile (V^T rows d = 32 db + l32 at (vb ^ 32 m) + 16384 + 4096 db for
// key k-step m = 2 kb + s2), then S^T = K Q^T of the current one (K rows 32 kb + l32 at
// (kb ^ 32 kk) + 8192 kb for d k-step kk), with six LDS operand reads in flight across both
// products and exact partial waits (a read is issued into the buffer the product before it
// has just consumed; the xor-ed addresses are formed in two temporaries just before their
// first read; the block waits for all of its reads before it ends).  With one wave per SIMD
// in this phase, a 16-byte operand read per 32x32x16 product keeps the matrix pipe about
// 69 % busy at four reads in flight and 76 % at six (deeper rings add nothing), measured on
// MI355X with the ring restarted every 16 products.  The leading s_nop covers the wait
// states between the softmax phase's vector writes (P, the rescaled O) and their first
// matrix read; the trailing ones those between the last product and the vector reads of S.
__device__ __forceinline__ void matrix_phase_d128(uint32_t kb, uint32_t vb, const bf16x8_t* qreg,
                                                  const PackP (*p)[2], f32x16_t* o, f32x16_t* sv) {
  bf16x8_t t0, t1, t2, t3, t4, t5;
  uint32_t ta, tb;
  asm volatile(
      "s_nop 4\n"
      "ds_read_b128 %[t0], %[vb] offset:16384\n"
      "ds_read_b128 %[t1], %[vb] offset:20480\n"
      "ds_read_b128 %[t2], %[vb] offset:24576\n"
      "ds_read_b128 %[t3], %[vb] offset:28672\n"
      "v_xor_b32 %[ta], 32, %[vb]\n"
      "ds_read_b128 %[t4], %[ta] offset:16384\n"
      "ds_read_b128 %[t5], %[ta] offset:20480\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[o0], %[t0], %[p0], %[o0]\n"
      "ds_read_b128 %[t0], %[ta] offset:24576\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[o1], %[t1], %[p0], %[o1]\n"
      "ds_read_b128 %[t1], %[ta] offset:28672\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[o2], %[t2], %[p0], %[o2]\n"
      "v_xor_b32 %[tb], 64, %[vb]\n"
      "ds_read_b128 %[t2], %[tb] offset:16384\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[o3], %[t3], %[p0], %[o3]\n"
      "ds_read_b128 %[t3], %[tb] offset:20480\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[o0], %[t4], %[p1], %[o0]\n"
      "ds_read_b128 %[t4], %[tb] offset:24576\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[o1], %[t5], %[p1], %[o1]\n"
      "ds_read_b128 %[t5], %[tb] offset:28672\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[o2], %[t0], %[p1], %[o2]\n"
      "v_xor_b32 %[ta], 96, %[vb]\n"
      "ds_read_b128 %[t0], %[ta] offset:16384\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[o3], %[t1], %[p1], %[o3]\n"
      "ds_read_b128 %[t1], %[ta] offset:20480\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[o0], %[t2], %[p2], %[o0]\n"
      "ds_read_b128 %[t2], %[ta] offset:24576\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[o1], %[t3], %[p2], %[o1]\n"
      "ds_read_b128 %[t3], %[ta] offset:28672\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[o2], %[t4], %[p2], %[o2]\n"
      "ds_read_b128 %[t4], %[kb] offset:0\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[o3], %[t5], %[p2], %[o3]\n"
      "ds_read_b128 %[t5], %[kb] offset:8192\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[o0], %[t0], %[p3], %[o0]\n"
      "v_xor_b32 %[tb], 32, %[kb]\n"
      "ds_read_b128 %[t0], %[tb] offset:0\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[o1], %[t1], %[p3], %[o1]\n"
      "ds_read_b128 %[t1], %[tb] offset:8192\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[o2], %[t2], %[p3], %[o2]\n"
      "v_xor_b32 %[ta], 64, %[kb]\n"
      "ds_read_b128 %[t2], %[ta] offset:0\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[o3], %[t3], %[p3], %[o3]\n"
      "ds_read_b128 %[t3], %[ta] offset:8192\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[s0], %[t4], %[q0], 0\n"
      "v_xor_b32 %[tb], 96, %[kb]\n"
      "ds_read_b128 %[t4], %[tb] offset:0\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[s1], %[t5], %[q0], 0\n"
      "ds_read_b128 %[t5], %[tb] offset:8192\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[s0], %[t0], %[q1], %[s0]\n"
      "v_xor_b32 %[ta], 128, %[kb]\n"
      "ds_read_b128 %[t0], %[ta] offset:0\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[s1], %[t1], %[q1], %[s1]\n"
      "ds_read_b128 %[t1], %[ta] offset:8192\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[s0], %[t2], %[q2], %[s0]\n"
      "v_xor_b32 %[tb], 160, %[kb]\n"
      "ds_read_b128 %[t2], %[tb] offset:0\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[s1], %[t3], %[q2], %[s1]\n"
      "ds_read_b128 %[t3], %[tb] offset:8192\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[s0], %[t4], %[q3], %[s0]\n"
      "v_xor_b32 %[ta], 192, %[kb]\n"
      "ds_read_b128 %[t4], %[ta] offset:0\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[s1], %[t5], %[q3], %[s1]\n"
      "ds_read_b128 %[t5], %[ta] offset:8192\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[s0], %[t0], %[q4], %[s0]\n"
      "v_xor_b32 %[tb], 224, %[kb]\n"
      "ds_read_b128 %[t0], %[tb] offset:0\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[s1], %[t1], %[q4], %[s1]\n"
      "ds_read_b128 %[t1], %[tb] offset:8192\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[s0], %[t2], %[q5], %[s0]\n"
      "s_waitcnt lgkmcnt(4)\n"
      "v_mfma_f32_32x32x16_bf16 %[s1], %[t3], %[q5], %[s1]\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %[s0], %[t4], %[q6], %[s0]\n"
      "s_waitcnt lgkmcnt(2)\n"
      "v_mfma_f32_32x32x16_bf16 %[s1], %[t5], %[q6], %[s1]\n"
      "s_waitcnt lgkmcnt(1)\n"
      "v_mfma_f32_32x32x16_bf16 %[s0], %[t0], %[q7], %[s0]\n"
      "s_waitcnt lgkmcnt(0)\n"
      "v_mfma_f32_32x32x16_bf16 %[s1], %[t1], %[q7], %[s1]\n"
      "s_nop 7\n"
      "s_nop 7\n"
      "s_nop 4\n"
      : [o0] "+v"(o[0]), [o1] "+v"(o[1]), [o2] "+v"(o[2]), [o3] "+v"(o[3]), [s0] "=&v"(sv[0]), [s1] "=&v"(sv[1]),
        [t0] "=&v"(t0), [t1] "=&v"(t1), [t2] "=&v"(t2), [t3] "=&v"(t3), [t4] "=&v"(t4), [t5] "=&v"(t5),
        [ta] "=&v"(ta), [tb] "=&v"(tb)
      : [p0] "v"(p[0][0].v), [p1] "v"(p[0][1].v), [p2] "v"(p[1][0].v), [p3] "v"(p[1][1].v), [q0] "v"(qreg[0]),
        [q1] "v"(qreg[1]), [q2] "v"(qreg[2]), [q3] "v"(qreg[3]), [q4] "v"(qreg[4]), [q5] "v"(qreg[5]),
        [q6] "v"(qreg[6]), [q7] "v"(qreg[7]), [vb] "v"(vb), [kb] "v"(kb)
      : "memory");
}

// One whole tile: scores, softmax and O^T += V^T P^T in sequence (the probe rows).
template <int D, int BN, bool MASK>
__device__ __forceinline__ void mfma_tile_step(const char* __restrict__ stage, const bf16x8_t* qreg, int lo, int hi,
                                               float c2, const uint8_t* __restrict__ klab, uint64_t rowmask,
                                               float& m_i, float& l_i, f32x16_t* o, int l32, int hf) {
  using C = MfmaCfg<D, BN>;
  f32x16_t sv[C::NB];
  PackP p[C::NB][2];
  scores_mfma<D, BN>(stage, qreg, sv, l32, hf);
  softmax_step<D, BN, MASK>(sv, lo, hi, c2, klab, rowmask, m_i, l_i, o, p, hf);
  pv_mfma<D, BN>(stage, p, o, l32, hf);
}

// Fused write-back for one query head per KV head (summary page of "Partition the
// Support, Reconstruct the Residual": the affine probe-fit correction, write-back):
// o_hat = o + c0 + (o A) B on the matrix cores straight from the output accumulators.
// O^T's accumulator layout is already a valid B operand over d (the k-index permutation
// is applied to both operands), so t^T = A^T O^T (k x q) and then O^T += B^T t^T need no
// data movement; A^T, B^T (bf16) and c0 are staged in LDS.  With SPLIT every bf16 operand
// (O, A, t, B) is carried as a bf16 high part and a bf16 remainder and each product as
// three (hi hi + hi lo + lo hi), which keeps the correction to about 2^-16 of its size
// where it grows as large as the output itself (grouped query heads, the unprojected
// ridge).  Rows are scattered to token order through the query permutation.
template <int D, bool SPLIT>
struct FusedLds {
  static constexpr int RCM = kMaxCorrRank;  // up to 64 correction directions (two 32-row blocks of t)
  static constexpr int AROW = D + 8;        // At[k][d] bf16, padded rows (conflict-free 16-byte reads)
  static constexpr int BROW = RCM + 4;      // Bt[d][k] bf16, padded rows (conflict-free 8-byte reads)
  static constexpr int PART = (RCM * AROW + D * BROW) * 2;   // one copy of At and Bt
  static constexpr int BYTES = PART * (SPLIT ? 2 : 1) + D * 4;
};

template <int D, int LDS_BYTES, int NT, bool SPLIT = false>
__device__ __forceinline__ void fused_stage(const AttnArgs& A, int h, char* lds, int tid) {
  using F = FusedLds<D, SPLIT>;
  static_assert(F::BYTES <= LDS_BYTES, "fused write-back staging");
  bf16_t* At = reinterpret_cast<bf16_t*>(lds);
  bf16_t* Bt = At + F::RCM * F::AROW;
  float* c0s = reinterpret_cast<float*>(lds + F::PART * (SPLIT ? 2 : 1));
  const int re = min(A.r_eff[h], min(A.rank, F::RCM));
  const float* Ah = A.fitA + (int64_t)h * D * A.rank;
  const float* Bh = A.fitB + (int64_t)h * A.rank * D;
  // only the rows of A^T (columns of B^T) the products read: one 32-row block of t, or two
  const int kr = re > 32 ? F::RCM : 32;
  auto put = [&](bf16_t* dst, int off, float v) {
    const bf16_t hi = f32_to_bf16(v);
    dst[off] = hi;
    if constexpr (SPLIT) dst[F::PART / 2 + off] = f32_to_bf16(v - bf16_to_f32(hi));
  };
  if ((A.rank & 3) == 0) {   // 16-byte loads: four k of a row of A, four d of a row of B
    const int kq = kr / 4;
    for (int idx = tid; idx < kq * D; idx += NT) {
      const int d = idx / kq, k = 4 * (idx % kq);
      const float4 a4 = k < re ? *reinterpret_cast<const float4*>(Ah + (int64_t)d * A.rank + k)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
      put(At, k * F::AROW + d, a4.x);
      put(At, (k + 1) * F::AROW + d, k + 1 < re ? a4.y : 0.f);
      put(At, (k + 2) * F::AROW + d, k + 2 < re ? a4.z : 0.f);
      put(At, (k + 3) * F::AROW + d, k + 3 < re ? a4.w : 0.f);
    }
    for (int idx = tid; idx < kr * (D / 4); idx += NT) {
      const int k = idx / (D / 4), d = 4 * (idx % (D / 4));
      const float4 b4 = k < re ? *reinterpret_cast<const float4*>(Bh + (int64_t)k * D + d)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
      put(Bt, d * F::BROW + k, b4.x);
      put(Bt, (d + 1) * F::BROW + k, b4.y);
      put(Bt, (d + 2) * F::BROW + k, b4.z);
      put(Bt, (d + 3) * F::BROW + k, b4.w);
    }
  } else {
    for (int idx = tid; idx < kr * D; idx += NT) {
      const int k = idx / D, d = idx % D;
      put(At, k * F::AROW + d, k < re ? Ah[d * A.rank + k] : 0.f);
      put(Bt, d * F::BROW + k, k < re ? Bh[k * D + d] : 0.f);
    }
  }
  for (int d = tid; d < D; d += NT) c0s[d] = A.fitc0[(int64_t)h * D + d];
  __syncthreads();
}

// 8 bf16 of a staged row (two 8-byte reads 8 elements apart: the k-permuted operand layout)
__device__ __forceinline__ bf16x8_t staged8(const bf16_t* r) {
  const uint2 lo8 = *reinterpret_cast<const uint2*>(r);
  const uint2 hi8 = *reinterpret_cast<const uint2*>(r + 8);
  return __builtin_bit_cast(bf16x8_t, make_uint4(lo8.x, lo8.y, hi8.x, hi8.y));
}

// The correction and scatter of one wave's 32 rows of query head h (group-major position
// p of KV head kv) from A^T, B^T and c0 staged by fused_stage.
template <int D, bool SPLIT = false>
__device__ __forceinline__ void fused_apply(const AttnArgs& A, int h, int kv, int p, bool qvalid, float inv,
                                            f32x16_t* o, const char* lds, int l32, int hf) {
  using F = FusedLds<D, SPLIT>;
  constexpr int DBLK = D / 32;
  const bf16_t* At = reinterpret_cast<const bf16_t*>(lds);
  const bf16_t* Bt = At + F::RCM * F::AROW;
  const float* c0s = reinterpret_cast<const float*>(lds + F::PART * (SPLIT ? 2 : 1));
  const int re = min(A.r_eff[h], min(A.rank, F::RCM));
  // normalise and pack O (bf16) as the B operand over d; t^T = A^T O^T in one or two 32-row
  // blocks of correction directions
  const bool two = re > 32;
  f32x16_t t[2];
#pragma unroll
  for (int r = 0; r < 16; ++r) { t[0][r] = 0.f; t[1][r] = 0.f; }
#pragma unroll
  for (int db = 0; db < DBLK; ++db) {
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] *= inv;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      bf16x8_t ob, obl;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ob[e] = (__bf16)o[db][8 * s2 + e];
        if constexpr (SPLIT) obl[e] = (__bf16)(o[db][8 * s2 + e] - (float)ob[e]);
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (kb == 1 && !two) break;
        const bf16_t* ar = At + (32 * kb + l32) * F::AROW + 32 * db + 16 * s2 + 4 * hf;
        const bf16x8_t av = staged8(ar);
        t[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, ob, t[kb], 0, 0, 0);
        if constexpr (SPLIT) {
          t[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(staged8(ar + F::PART / 2), ob, t[kb], 0, 0, 0);
          t[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, obl, t[kb], 0, 0, 0);
        }
      }
    }
  }
  // t^T[k][q] in the accumulator layout is the B operand over k of O^T += B^T t^T
  bf16x8_t tb[4], tbl[4];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    tb[0][e] = (__bf16)t[0][e];
    tb[1][e] = (__bf16)t[0][8 + e];
    tb[2][e] = (__bf16)t[1][e];
    tb[3][e] = (__bf16)t[1][8 + e];
    if constexpr (SPLIT) {
      tbl[0][e] = (__bf16)(t[0][e] - (float)tb[0][e]);
      tbl[1][e] = (__bf16)(t[0][8 + e] - (float)tb[1][e]);
      tbl[2][e] = (__bf16)(t[1][e] - (float)tb[2][e]);
      tbl[3][e] = (__bf16)(t[1][8 + e] - (float)tb[3][e]);
    }
  }
  const int ksteps = (re + 15) / 16;
#pragma unroll
  for (int db = 0; db < DBLK; ++db) {
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      if (s2 >= ksteps) break;
      const bf16_t* br = Bt + (32 * db + l32) * F::BROW + 16 * s2 + 4 * hf;
      const bf16x8_t bv = staged8(br);
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv, tb[s2], o[db], 0, 0, 0);
      if constexpr (SPLIT) {
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(staged8(br + F::PART / 2), tb[s2], o[db], 0, 0, 0);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv, tbl[s2], o[db], 0, 0, 0);
      }
    }
  }
  if (qvalid) {
    const int64_t tok = A.qperm[(int64_t)kv * A.n + p];
    bf16_t* orow = static_cast<bf16_t*>(A.out_tok) + ((int64_t)h * A.n + tok) * D;
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d0 = 32 * db + 8 * j + 4 * hf;
        uint2 v2 = make_uint2((uint32_t)f32_to_bf16(o[db][4 * j] + c0s[d0]) |
                                  ((uint32_t)f32_to_bf16(o[db][4 * j + 1] + c0s[d0 + 1]) << 16),
                              (uint32_t)f32_to_bf16(o[db][4 * j + 2] + c0s[d0 + 2]) |
                                  ((uint32_t)f32_to_bf16(o[db][4 * j + 3] + c0s[d0 + 3]) << 16));
        *reinterpret_cast<uint2*>(orow + d0) = v2;
      }
  }
}

template <int D, int LDS_BYTES, int NT>
__device__ __forceinline__ void fused_writeback(const AttnArgs& A, int kv, int vrow, bool qvalid, float inv,
                                                f32x16_t* o, char* lds, int tid, int l32, int hf) {
  fused_stage<D, LDS_BYTES, NT>(A, kv, lds, tid);   // one query head per KV head
  fused_apply<D>(A, kv, kv, vrow, qvalid, inv, o, lds, l32, hf);
}

// The fused write-back under GQA (summary page of "Partition the Support, Reconstruct the
// Residual", execution paragraph: the route is shared by the query heads of a KV head, so
// one attention block holds rows of all of them; virtual row v is query head v mod g at
// group-major position v / g).  The g heads' corrections are applied in turn: head j's A^T,
// B^T (split into a bf16 high part and remainder, as the GQA write-back kernel does) are
// staged, t^T = A_j^T O^T is formed for the wave's 32 columns and the columns of other heads'
// rows are zeroed, so O^T += B_j^T t^T changes only head j's columns (a column of the
// products depends on that column of O^T alone).  Then c0 of each row's head is added and
// the rows are scattered to token order.
template <int D, int LDS_BYTES, int NT>
__device__ __forceinline__ void fused_writeback_gqa(const AttnArgs& A, int kv, int vrow, bool qvalid, float inv,
                                                    f32x16_t* o, char* lds, int tid, int l32, int hf) {
  using F = FusedLds<D, true>;
  constexpr int DBLK = D / 32;
  const bf16_t* At = reinterpret_cast<const bf16_t*>(lds);
  const bf16_t* Bt = At + F::RCM * F::AROW;
  const int jrow = vrow % A.g;
#pragma unroll
  for (int db = 0; db < DBLK; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] *= inv;
  for (int j = 0; j < A.g; ++j) {
    const int h = kv * A.g + j;
    if (j > 0) __syncthreads();   // every wave is done reading head j - 1's staging
    fused_stage<D, LDS_BYTES, NT, true>(A, h, lds, tid);
    const int re = min(A.r_eff[h], min(A.rank, F::RCM));
    const bool two = re > 32;
    f32x16_t t[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) { t[0][r] = 0.f; t[1][r] = 0.f; }
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        bf16x8_t ob, obl;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          ob[e] = (__bf16)o[db][8 * s2 + e];
          obl[e] = (__bf16)(o[db][8 * s2 + e] - (float)ob[e]);
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          if (kb == 1 && !two) break;
          const bf16_t* ar = At + (32 * kb + l32) * F::AROW + 32 * db + 16 * s2 + 4 * hf;
          const bf16x8_t av = staged8(ar);
          t[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, ob, t[kb], 0, 0, 0);
          t[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(staged8(ar + F::PART / 2), ob, t[kb], 0, 0, 0);
          t[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, obl, t[kb], 0, 0, 0);
        }
      }
    const bool mine = jrow == j;   // lane l32's column is this head's row
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      t[0][r] = mine ? t[0][r] : 0.f;
      t[1][r] = mine ? t[1][r] : 0.f;
    }
    bf16x8_t tb[4], tbl[4];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      tb[0][e] = (__bf16)t[0][e];
      tb[1][e] = (__bf16)t[0][8 + e];
      tb[2][e] = (__bf16)t[1][e];
      tb[3][e] = (__bf16)t[1][8 + e];
      tbl[0][e] = (__bf16)(t[0][e] - (float)tb[0][e]);
      tbl[1][e] = (__bf16)(t[0][8 + e] - (float)tb[1][e]);
      tbl[2][e] = (__bf16)(t[1][e] - (float)tb[2][e]);
      tbl[3][e] = (__bf16)(t[1][8 + e] - (float)tb[3][e]);
    }
    const int ksteps = (re + 15) / 16;
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
        if (s2 >= ksteps) break;
        const bf16_t* br = Bt + (32 * db + l32) * F::BROW + 16 * s2 + 4 * hf;
        const bf16x8_t bv = staged8(br);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv, tb[s2], o[db], 0, 0, 0);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(staged8(br + F::PART / 2), tb[s2], o[db], 0, 0, 0);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv, tbl[s2], o[db], 0, 0, 0);
      }
  }
  if (qvalid) {
    const int h = kv * A.g + jrow;
    const int64_t tok = A.qperm[(int64_t)kv * A.n + vrow / A.g];
    const float* c0 = A.fitc0 + (int64_t)h * D;
    bf16_t* orow = static_cast<bf16_t*>(A.out_tok) + ((int64_t)h * A.n + tok) * D;
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d0 = 32 * db + 8 * j + 4 * hf;
        uint2 v2 = make_uint2((uint32_t)f32_to_bf16(o[db][4 * j] + c0[d0]) |
                                  ((uint32_t)f32_to_bf16(o[db][4 * j + 1] + c0[d0 + 1]) << 16),
                              (uint32_t)f32_to_bf16(o[db][4 * j + 2] + c0[d0 + 2]) |
                                  ((uint32_t)f32_to_bf16(o[db][4 * j + 3] + c0[d0 + 3]) << 16));
        *reinterpret_cast<uint2*>(orow + d0) = v2;
      }
  }
}

constexpr int kAttnWaves = 8;    // waves per block of the main attention kernel
constexpr int kAttnStages = 4;   // K/V tile stages in LDS; tile j + 2 is copied while tile j runs
constexpr int kMatLookahead = 5; // LDS operand reads in flight ahead of the matrix products (d = 64)

// Waits until at most `later` tiles' copies of this wave are still in flight (each tile is
// C::KIPW + C::VIPW direct-to-LDS loads, which complete in order for the counter).
template <int PER_TILE>
__device__ __forceinline__ void wait_tiles_in_flight(int later) {
  static_assert(2 * PER_TILE <= 63, "vmcnt immediate");
  // s_waitcnt immediate: vmcnt bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at
  // their maxima
  constexpr int V2 = 2 * PER_TILE, V1 = PER_TILE;
  if (later >= 2) __builtin_amdgcn_s_waitcnt(0x0F70 | (V2 & 15) | ((V2 >> 4) << 14));
  else if (later == 1) __builtin_amdgcn_s_waitcnt(0x0F70 | (V1 & 15) | ((V1 >> 4) << 14));
  else __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Claims the next unstarted tile of the tail of XCD x's range, else of the other XCDs' ranges
// in turn; -1 when none is left.  A claimed slot past a head's tiles (its padding) moves that
// counter on to the next head's first slot.
__device__ int claim_tile(const AttnArgs& A, int x) {
  for (int k = 0; k < kXcds; ++k) {
    const int y = (x + k) & (kXcds - 1);
    for (;;) {
      const int j = atomicAdd(&A.claim[y], 1);
      if (j >= A.per_xcd) break;
      const int logical = y * A.per_xcd + j;
      const int kv = logical / A.tiles_per_head;
      if (kv >= A.n_heads_kv) break;   // the grid's rounding past the last head
      if (A.order_count == nullptr || logical % A.tiles_per_head < A.order_count[kv]) return logical;
      atomicMax(&A.claim[y], (kv + 1) * A.tiles_per_head - y * A.per_xcd);
    }
  }
  return -1;
}

template <int D, int BN, typename OutT>
__global__ __launch_bounds__(64 * kAttnWaves, 1) void attn_mfma_kernel(AttnArgs A) {
  using C = MfmaCfg<D, BN, kAttnWaves>;
  constexpr int PER_TILE = C::KIPW + C::VIPW;
  __shared__ __attribute__((aligned(1024))) char stages[kAttnStages][C::STAGE];

  // XCD-aware remap of the linear block id (consecutive logical tiles on one XCD)
  const int b = blockIdx.x;
  int logical;
  if (A.claim == nullptr) {
    logical = (b % kXcds) * (gridDim.x / kXcds) + b / kXcds;
  } else if (b / kXcds < A.tail_start) {
    logical = (b % kXcds) * A.per_xcd + b / kXcds;
  } else {   // the tail of the XCD's range, then of the others' ranges (block-uniform branch)
    __shared__ int claimed_s;
    if (threadIdx.x == 0) claimed_s = claim_tile(A, b % kXcds);
    __syncthreads();
    logical = claimed_s;
    if (logical < 0) return;
  }
  int kv;
  TileInfo ti;
  if (A.order != nullptr) {   // the head's groups longest first
    kv = logical / A.tiles_per_head;
    if (kv >= A.n_heads_kv) return;
    const int idx = logical % A.tiles_per_head;
    if (idx >= A.order_count[kv]) return;
    const int32_t* e = A.order + 2 * ((int64_t)kv * A.tiles_per_head + idx);
    if (!group_tile(A, kv, e[0], e[1], C::BM, ti)) return;
  } else {
    kv = logical / A.tiles_per_head;
    if (kv >= A.n_heads_kv) return;
    if (!find_tile(A, kv, logical % A.tiles_per_head, C::BM, ti)) return;
  }

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int wu = wave_uniform(w);
  const bf16_t* qb = static_cast<const bf16_t*>(A.q);
  const bf16_t* kb = static_cast<const bf16_t*>(A.k) + (int64_t)kv * A.kv_skv;
  const bf16_t* vtb = static_cast<const bf16_t*>(A.v) + (int64_t)kv * A.v_skv;

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
  const bool wave_rows = ti.v0 + 32 * wu < ti.v1;
  float m_i = -INFINITY, l_i = 0.f;
  f32x16_t o[C::DBLK];
#pragma unroll
  for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;

  // Tile iterators: (ci, k0, k1, kt) is the tile being computed (ci: its next run), (fci, fk0,
  // fk1, fkt) the copy frontier two tiles ahead; tile j lives in stage j % kAttnStages.
  __shared__ int2 runs[kMaxGroups];
  __shared__ int nruns_s;
  if (wu == 0) build_runs(A, kv, ti, lane, runs, &nruns_s);
  __syncthreads();
  const int nruns = __builtin_amdgcn_readfirstlane(nruns_s);
  int ci = 0, k0 = 0, k1 = 0, kt = -BN;
  bool valid = next_tile_lds(runs, nruns, BN, ci, k0, k1, kt);
  int fci = ci, fk0 = k0, fk1 = k1, fkt = kt;
  bool fvalid = valid;
  // Anti-phased schedule: waves 0-3 and 4-7 (one of each per SIMD) alternate between a
  // matrix phase (S_j = K_j Q^T and O += V_{j-1} P_{j-1}) and a softmax phase (S_j ->
  // P_j), so that one wave of every SIMD issues matrix products while the other runs its
  // exponentials.  One block barrier per tile: between barriers j and j + 1, waves 0-3 run
  // the matrix phase of tile j and then its softmax; waves 4-7 run the softmax of tile
  // j - 1 and then the matrix phase of tile j (their first interval has no softmax, and the
  // last tile's softmax follows the loop).  K_j and V_{j-1} are the only stages read in
  // interval j.  Waves 0-3 alone copy the tiles, between their matrix phase and their
  // softmax (which reads no LDS): tile j + 2 in interval j, into the stage of tile j - 2
  // (last read in interval j - 1), and each waits for its copies of tile j + 1 before the
  // barrier that ends interval j.
  constexpr int CW = kAttnWaves / 2;   // copying waves
  using CC = MfmaCfg<D, BN, CW>;
  constexpr int PT = CC::KIPW + CC::VIPW;
  const bool lag = wu >= CW;
  const CopyPlan<D, BN, CW> cpa(wu & (CW - 1), lane, A.v_np);
  int ncopied = 0;
  for (int i = 0; i < 2 && fvalid; ++i) {
    if (!lag) stage_copy<D, BN, CW>(cpa, kb, vtb, A.n, A.v_np, fkt, stages[i], wu);
    ++ncopied;
    fvalid = next_tile_lds(runs, nruns, BN, fci, fk0, fk1, fkt);
  }
  if (!lag) wait_tiles_in_flight<PT>(ncopied - 1);   // tile 0 has landed
  __syncthreads();
  f32x16_t sv[C::NB];
  PackP pp[C::NB][2];
#pragma unroll
  for (int kb = 0; kb < C::NB; ++kb)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int e = 0; e < 8; ++e) pp[kb][s2].v[e] = (__bf16)0.f;
  // per-lane LDS byte offsets of the matrix phase's first K and V^T operand reads within a
  // stage (d = 128); k-step i reads at the offset xor 32 i (the swizzles of K rows and V^T
  // rows act on the chunk's low bit and the lane only, so the k-step moves bits 5-7 alone)
  const uint32_t koff0 = (uint32_t)(l32 * 256 + ((hf ^ (l32 & 15)) << 4));
  const uint32_t voff0 = (uint32_t)(l32 * 128 + ((hf ^ ((l32 >> 1) & 7)) << 4));
  int cur = 0, prev = 0, fst = 2;
  bool have_prev = false;
  int plo = 0, phi = 0;   // valid keys of the previous tile (the lagging waves' softmax)
  while (valid) {
    const int lo = max(k0 - kt, 0), hi = min(k1 - kt, BN);
    if (lag && have_prev && wave_rows)   // waves 4-7: the previous tile's softmax first
      softmax_step<D, BN, false>(sv, plo, phi, c2, nullptr, 0ull, m_i, l_i, o, pp, hf);
    if (wave_rows) {   // matrix phase (the first one multiplies tile 0's V by zero probabilities)
      if constexpr (D == 128 && BN == 64) {
        // stages are 1024-byte aligned, so adding the stage base commutes with the xor
        matrix_phase_d128(lds_addr(stages[cur]) + koff0, lds_addr(stages[prev]) + voff0, qreg, pp, o, sv);
      } else {
        matrix_phase<D, BN, kMatLookahead>(stages[cur], stages[prev], qreg, pp, o, sv, l32, hf);
      }
    }
    bool issued = false;
    if (fvalid) {
      if (!lag) stage_copy<D, BN, CW>(cpa, kb, vtb, A.n, A.v_np, fkt, stages[fst], wu);
      issued = true;
      fst = fst == kAttnStages - 1 ? 0 : fst + 1;
      fvalid = next_tile_lds(runs, nruns, BN, fci, fk0, fk1, fkt);
    }
    if (!lag && wave_rows)   // waves 0-3: this tile's softmax
      softmax_step<D, BN, false>(sv, lo, hi, c2, nullptr, 0ull, m_i, l_i, o, pp, hf);
    have_prev = true;
    plo = lo;
    phi = hi;
    prev = cur;
    cur = cur == kAttnStages - 1 ? 0 : cur + 1;
    valid = next_tile_lds(runs, nruns, BN, ci, k0, k1, kt);
    if (!lag) wait_tiles_in_flight<PT>(issued ? 1 : 0);   // tile j + 1 has landed
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
  if (lag && have_prev && wave_rows) softmax_step<D, BN, false>(sv, plo, phi, c2, nullptr, 0ull, m_i, l_i, o, pp, hf);
  if (wave_rows && have_prev) pv_mfma<D, BN>(stages[prev], pp, o, l32, hf);

  const float l_tot = add_xor32(l_i);
  const float inv = 1.f / l_tot;
  if (A.fitA != nullptr) {
    __syncthreads();   // every wave is done reading its last V tile from the stages
    if (A.g == 1)
      fused_writeback<D, C::STAGE * kAttnStages, 64 * kAttnWaves>(A, kv, vrow, qvalid, inv, o, &stages[0][0], tid,
                                                                     l32, hf);
    else
      fused_writeback_gqa<D, C::STAGE * kAttnStages, 64 * kAttnWaves>(A, kv, vrow, qvalid, inv, o, &stages[0][0],
                                                                         tid, l32, hf);
    return;
  }
  // epilogue: O / l, LSE; lane writes query l32's d = 32 db + 8 j + 4 hf + 0..3
  if (qvalid) {
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
    if (A.lse && hf == 0)
      A.lse[((int64_t)kv * A.n + vrow / A.g) * A.g + vrow % A.g] = (m_i + log2f(l_tot)) * 0.6931471805599453f;
  }
}

// Write-back of the unfused order on the matrix cores (bf16 output): the fp32 group-major
// rows of one query head are loaded in the accumulator layout of O^T and corrected and
// scattered exactly as in the fused epilogue.  grid (ceil(n / (128 kApplyTiles)), Hq), block
// 256 (4 waves x 32 rows per tile); one staging of the correction per block.
constexpr int kApplyTiles = 4;

template <int D, bool SPLIT>
__global__ __launch_bounds__(256, 2) void apply_mfma_kernel(AttnArgs A, const float* __restrict__ o_gm) {
  constexpr int LDS = FusedLds<D, SPLIT>::BYTES;
  __shared__ __attribute__((aligned(16))) char lds[LDS];
  const int h = blockIdx.y, kv = h / A.g, j = h % A.g;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  // rows of tile it in the accumulator layout (the next tile's loads are issued before the
  // current tile's products, and the first tile's before the staging, to hide HBM latency)
  auto load_tile = [&](int it, f32x16_t* o) {
    const int p = (blockIdx.x * kApplyTiles + it) * 128 + 32 * w + l32;
    const bool valid = p < A.n;
    const float* row = o_gm + (((int64_t)kv * A.n + (valid ? p : 0)) * A.g + j) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float4 v = valid ? *reinterpret_cast<const float4*>(row + 32 * db + 8 * jj + 4 * hf)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
        o[db][4 * jj] = v.x;
        o[db][4 * jj + 1] = v.y;
        o[db][4 * jj + 2] = v.z;
        o[db][4 * jj + 3] = v.w;
      }
  };
  f32x16_t ob[2][D / 32];
  load_tile(0, ob[0]);
  fused_stage<D, LDS, 256, SPLIT>(A, h, lds, tid);
  // the staged A^T, B^T and c0 serve kApplyTiles tiles of 128 rows
#pragma unroll
  for (int it = 0; it < kApplyTiles; ++it) {
    const int p0 = (blockIdx.x * kApplyTiles + it) * 128;
    if (p0 < A.n) {
      if (it + 1 < kApplyTiles && p0 + 128 < A.n) load_tile(it + 1, ob[(it + 1) & 1]);
      const int p = p0 + 32 * w + l32;
      fused_apply<D, SPLIT>(A, h, kv, p, p < A.n, 1.f, ob[it & 1], lds, l32, hf);
    }
  }
}

void launch_apply_mfma(const Dims& dm, const float* o_gm, const sparsepr_partition_t& part,
                       const sparsepr_fit_t& fit, void* o, hipStream_t s) {
  AttnArgs a{};
  a.n = dm.n;
  a.g = dm.g;
  a.fitA = fit.A;
  a.fitB = fit.B;
  a.fitc0 = fit.c0;
  a.r_eff = fit.r_eff;
  a.rank = dm.rc;
  a.qperm = part.query_perm;
  a.out_tok = o;
  const dim3 grid((unsigned)ceil_div(dm.n, 128 * kApplyTiles), dm.hq);
  // the split operands where the correction may grow as large as the output: grouped query
  // heads and the unprojected ridge (one query head per KV head with the projected fit keeps
  // the fused epilogue's single bf16 products)
  const bool split = dm.g > 1 || dm.rc > kMaxRank;
  if (dm.d == 128) {
    if (split) hipLaunchKernelGGL((apply_mfma_kernel<128, true>), grid, dim3(256), 0, s, a, o_gm);
    else hipLaunchKernelGGL((apply_mfma_kernel<128, false>), grid, dim3(256), 0, s, a, o_gm);
  } else {
    if (split) hipLaunchKernelGGL((apply_mfma_kernel<64, true>), grid, dim3(256), 0, s, a, o_gm);
    else hipLaunchKernelGGL((apply_mfma_kernel<64, false>), grid, dim3(256), 0, s, a, o_gm);
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
                                                               const bf16_t* __restrict__ vtgm,
                                                               const int32_t* __restrict__ koff,
                                                               const uint64_t* __restrict__ kept_mask,
                                                               const int32_t* __restrict__ ptok,
                                                               const int32_t* __restrict__ pgrp, int n, int g,
                                                               int Gq, int Gk, int M, float scale, int chunk,
                                                               float* __restrict__ partials) {
  using C = MfmaCfg<D>;
  __shared__ __attribute__((aligned(1024))) char stages[2][C::STAGE];
  __shared__ uint8_t klab[2][C::BN];
  __shared__ int ko[kMaxGroups + 1];
  const int h = blockIdx.y, kv = h / g, ch = blockIdx.x, nch = gridDim.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int row = 32 * (w & 1) + l32;
  const bool sparse = (w >> 1) != 0;
  const int k0 = ch * chunk, k1 = min(n, k0 + chunk);
  const int np = (int)vt_pad(n);
  const int wu = wave_uniform(w);
  const CopyPlan<D, 32, 4> cp(wu, lane, np);
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
  const bf16_t* vtb = vtgm + (int64_t)kv * D * np;
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
  int kt = k0;
  if (kt < k1) {
    stage_copy<D, 32, 4>(cp, kb, vtb, n, np, kt, stages[0], wu);
    if (tid < C::BN) klab[0][tid] = (uint8_t)(kt + tid < k1 ? label_of(kt + tid) : 0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  int cur = 0;
  while (kt < k1) {
    const int nt = kt + C::BN;
    if (nt < k1) {
      stage_copy<D, 32, 4>(cp, kb, vtb, n, np, nt, stages[cur ^ 1], wu);
      if (tid < C::BN) klab[cur ^ 1][tid] = (uint8_t)(nt + tid < k1 ? label_of(nt + tid) : 0);
    }
    const int hi = min(k1 - kt, C::BN);
    if (sparse)
      probe_tile_step<D, 32, true>(stages[cur], qreg, hi, c2, klab[cur], rowmask, m_i, l_i, o, l32, hf);
    else
      probe_tile_step<D, 32, false>(stages[cur], qreg, hi, c2, nullptr, 0ull, m_i, l_i, o, l32, hf);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    cur ^= 1;
    kt = nt;
  }
  const float l_tot = add_xor32(l_i);
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

constexpr int kAttnBN = 64;   // keys per tile of the main attention kernel

// Longest-first schedule of the block-sparse attention within each KV head: a head's query
// groups are ranked by the number of key tiles each of their query tiles walks (descending,
// ties to the smaller group) and their query tiles laid out in that order.  Heads keep their
// place in the grid (a head's tiles stay together on one XCD, where its K/V runs are shared
// in L2); only the order of its groups changes, so the last blocks of a head are its
// shortest.  The order changes the schedule, never a result.  grid Hkv, block 64.
__global__ __launch_bounds__(64) void tile_order_kernel(const int32_t* __restrict__ qoff,
                                                        const int32_t* __restrict__ koff,
                                                        const int32_t* __restrict__ row_ptr,
                                                        const int32_t* __restrict__ cols, int gq, int gk, int g,
                                                        int BM, int BN, int tiles_per_head,
                                                        int32_t* __restrict__ order, int32_t* __restrict__ count,
                                                        int* __restrict__ claim, int tail_start) {
  __shared__ int nkt[kMaxGroups], nqt[kMaxGroups], start[kMaxGroups];
  __shared__ int cl[kMaxGroups * kMaxGroups], ko[kMaxGroups + 1], rp[kMaxGroups + 1];
  const int kv = blockIdx.x, a = threadIdx.x;
  if (kv == 0 && a < kXcds) claim[a] = tail_start;   // the attention's tile claims start afresh
  // the head's CSR and key offsets, staged with coalesced loads
  for (int i = a; i <= gk; i += 64) ko[i] = koff[(int64_t)kv * (gk + 1) + i];
  for (int i = a; i <= gq; i += 64) rp[i] = row_ptr[(int64_t)kv * (gq + 1) + i];
  __syncthreads();
  for (int i = a; i < rp[gq]; i += 64) cl[i] = cols[(int64_t)kv * gq * gk + i];
  __syncthreads();
  if (a < gq) {
    const int32_t* qo = qoff + (int64_t)kv * (gq + 1);
    nqt[a] = (int)ceil_div((int64_t)(qo[a + 1] - qo[a]) * g, BM);
    int t = 0;
    for (int ci = rp[a], ce = rp[a + 1]; ci < ce;) {   // runs of adjacent kept key groups, as next_run
      const int b = cl[ci++];
      int e = b;
      while (ci < ce && cl[ci] == e + 1) { ++e; ++ci; }
      const int k0 = ko[b], k1 = ko[e + 1];
      if (k1 > k0) t += (k1 - (k0 & ~15) + BN - 1) / BN;
    }
    nkt[a] = t;
  }
  __syncthreads();
  if (a < gq) {   // tiles of the groups ranked before this one
    int before = 0;
    for (int b = 0; b < gq; ++b)
      if (nkt[b] > nkt[a] || (nkt[b] == nkt[a] && b < a)) before += nqt[b];
    start[a] = before;
  }
  __syncthreads();
  if (a < gq) {
    int32_t* oh = order + 2 * (int64_t)kv * tiles_per_head;
    for (int t = 0; t < nqt[a]; ++t) {
      oh[2 * (start[a] + t)] = a;
      oh[2 * (start[a] + t) + 1] = t;
    }
  }
  if (a == 0) {
    int tot = 0;
    for (int b = 0; b < gq; ++b) tot += nqt[b];
    count[kv] = tot;
  }
}

static int attn_tiles_per_head(int n, int g, int gq) {
  return (int)ceil_div((int64_t)n * g, MfmaCfg<128, kAttnBN, kAttnWaves>::BM) + gq;
}

size_t attn_order_bytes(int n, int g, int hkv, int gq) {
  return (size_t)(2 * (int64_t)attn_tiles_per_head(n, g, gq) * hkv + 64 + hkv) * 4;
}

// XCD ranges of tph tiles per head over hkv heads: the last eighth of each XCD's range is
// claimed, with half as many spare blocks per XCD (launch_mfma_typed).
static void claim_plan(int tph, int hkv, AttnArgs& a) {
  a.per_xcd = (int)ceil_div((int64_t)tph * hkv, kXcds);
  a.tail_start = a.per_xcd - a.per_xcd / 8;
}

void launch_tile_order(const Dims& dm, AttnArgs& a, char* region, hipStream_t s) {
  const int tph = attn_tiles_per_head(dm.n, dm.g, dm.gq);
  int32_t* order = reinterpret_cast<int32_t*>(region);
  int32_t* count = order + 2 * (int64_t)tph * dm.hkv;
  int* claim = count + dm.hkv;   // kXcds counters in the region's last 64 words
  claim_plan(tph, dm.hkv, a);
  hipLaunchKernelGGL(tile_order_kernel, dim3(dm.hkv), dim3(64), 0, s, a.qoff, a.koff, a.row_ptr, a.cols, dm.gq, dm.gk,
                     dm.g, MfmaCfg<128, kAttnBN, kAttnWaves>::BM, kAttnBN, tph, order, count, claim, a.tail_start);
  a.order = order;
  a.order_count = count;
  a.claim = claim;
}

// The dense schedule (every tile of a head, no order) with the same claimed XCD tails; the
// counters are set by a fill kernel on the call's stream.
void launch_dense_claims(const Dims& dm, AttnArgs& a, int* claim, hipStream_t s) {
  const int tph = (int)ceil_div((int64_t)dm.n * dm.g, MfmaCfg<128, kAttnBN, kAttnWaves>::BM);
  claim_plan(tph, dm.hkv, a);
  fill_u32(reinterpret_cast<uint32_t*>(claim), kXcds, (uint32_t)a.tail_start, s);
  a.claim = claim;
}

template <int D, typename OutT>
void launch_mfma_typed(AttnArgs a, int hkv, hipStream_t s) {
  a.tiles_per_head = (int)ceil_div((int64_t)a.n * a.g, MfmaCfg<D, kAttnBN, kAttnWaves>::BM) + (a.qoff ? a.gq : 0);
  a.n_heads_kv = hkv;
  int64_t total = (int64_t)a.tiles_per_head * hkv;
  total = ceil_div(total, kXcds) * kXcds;
  if (a.claim != nullptr)   // spare blocks: half the claimed tail of each XCD
    total = (int64_t)kXcds * (a.per_xcd + (a.per_xcd - a.tail_start) / 2);
  hipLaunchKernelGGL((attn_mfma_kernel<D, kAttnBN, OutT>), dim3((unsigned)total), dim3(64 * kAttnWaves), 0, s, a);
}

void launch_attention_mfma(const Dims& dm, AttnArgs a, bool out_is_input_dtype, hipStream_t s) {
  if (out_is_input_dtype) {
    if (dm.d == 128) launch_mfma_typed<128, bf16_t>(a, dm.hkv, s); else launch_mfma_typed<64, bf16_t>(a, dm.hkv, s);
  } else {
    if (dm.d == 128) launch_mfma_typed<128, float>(a, dm.hkv, s); else launch_mfma_typed<64, float>(a, dm.hkv, s);
  }
}

}  // namespace sp
