// Matrix-core flash attention for bf16 (gfx950 MFMA 32x32x16), used both for the
// block-sparse SparsePR attention over the kept cells (summary page of "Partition the
// Support, Reconstruct the Residual", execution paragraph: exact on the selected cells,
// renormalised over the kept K/V groups) and for the dense baseline.
//
// Work decomposition: one block = 256 virtual query rows of one query group (8 waves x
// 32 rows); the block walks the group's kept key runs in 64-key tiles staged through LDS
// (four stages, direct global-to-LDS copies two tiles ahead of the tile being consumed).  Each wave computes S^T = K Q^T so that a lane owns one query and 32 of the
// tile's keys: the row max and sum are in-register plus one exchange with the partner
// lane (l ^ 32), and the probabilities are already laid out as the B operand of
// O^T += V^T P^T, so P never leaves registers.  V is stored transposed in LDS for that
// A operand.  Softmax runs in the log2 domain with scale * log2(e) folded in; P is
// rounded to bf16 for the second product and accumulation is fp32.
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
// tile outside its run [k0, k1) are masked.  Advances (ci, k0, k1, kt) to the next tile;
// returns false after the last one.
__device__ __forceinline__ bool next_tile(const AttnArgs& A, int kv, const TileInfo& ti, int BN, int& ci, int& k0,
                                          int& k1, int& kt) {
  kt += BN;
  if (kt < k1) return true;
  if (!next_run(A, kv, ti, ci, k0, k1)) return false;
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

template <int D, int BN, int NW>
struct CopyPlan {
  using C = MfmaCfg<D, BN, NW>;
  uint32_t koff[C::KIPW];   // bytes from the tile's first K row
  uint32_t voff[C::VIPW];   // bytes from the tile's first V^T column
  int krow[C::KIPW];        // K row within the tile
  int vcol[C::VIPW];        // V^T column (key) within the tile

  __device__ CopyPlan(int w, int lane, int np) {
#pragma unroll
    for (int i = 0; i < C::KIPW; ++i) {
      const int L = (w * C::KIPW + i) * 64 + lane;
      const int r = L / C::KCH, slot = L % C::KCH, c = slot ^ C::kswz(r);
      krow[i] = r;
      koff[i] = (uint32_t)(r * D + 8 * c) * 2u;
    }
#pragma unroll
    for (int i = 0; i < C::VIPW; ++i) {
      const int L = (w * C::VIPW + i) * 64 + lane;
      const int d = L / C::VCH, slot = L % C::VCH, c = slot ^ C::vswz(d);
      vcol[i] = 8 * c;
      voff[i] = (uint32_t)(d * np + 8 * c) * 2u;
    }
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
#pragma unroll
  for (int i = 0; i < C::KIPW; ++i) {
    const int row = min(kt + cp.krow[i], n - 1);
    const char* src = reinterpret_cast<const char*>(kb + (int64_t)(row - cp.krow[i]) * D) + cp.koff[i];
    __builtin_amdgcn_global_load_lds((const void*)src, (lds_void_t*)(stage + (wu * C::KIPW + i) * 1024), 16, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < C::VIPW; ++i) {
    const int pos = kt + cp.vcol[i];
    const int base = pos + 8 <= np ? kt : -cp.vcol[i];   // chunks past n_pad read the row's first chunk
    const char* src = reinterpret_cast<const char*>(vtb + base) + cp.voff[i];
    __builtin_amdgcn_global_load_lds((const void*)src, (lds_void_t*)(vst + (wu * C::VIPW + i) * 1024), 16, 0, 0);
  }
}

union PackP {
  bf16x8_t v;
  bf16x2_t h[4];
};

// One tile (BN keys) of the online softmax for a wave's 32 queries: S^T = K Q^T on the
// matrix cores (one accumulation chain per 32-key block), masking (keys outside [lo, hi)
// of the tile; with MASK also keys whose group bit is clear in rowmask), the row max
// (in-register plus the partner lane l ^ 32), p = exp2(s c2 - m) with one FMA and the
// hardware exp2, bf16 packing, the row sum as bf16 dot products of the packed p (the
// values the second product consumes), a lazy rescale, and O^T += V^T P^T.
template <int D, int BN, bool MASK>
__device__ __forceinline__ void mfma_tile_step(const char* __restrict__ stage, const bf16x8_t* qreg, int lo, int hi,
                                               float c2, const uint8_t* __restrict__ klab, uint64_t rowmask,
                                               float& m_i, float& l_i, f32x16_t* o, int l32, int hf) {
  using C = MfmaCfg<D, BN>;
  f32x16_t sv[C::NB];
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
  PackP p[C::NB][2];
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
  // O^T += V^T P^T: key k-step (kb, s2) covers keys 32 kb + 16 s2 + {4 hf + 0..3, 8 + 4 hf + 0..3},
  // which the V^T layout keeps as chunk 2 (2 kb + s2) + hf of the row
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

// Fused write-back for one query head per KV head (summary page of "Partition the
// Support, Reconstruct the Residual": the affine probe-fit correction, write-back):
// o_hat = o + c0 + (o A) B on the matrix cores straight from the output accumulators.
// O^T's accumulator layout is already a valid B operand over d (the k-index permutation
// is applied to both operands), so t^T = A^T O^T (k x q) and then O^T += B^T t^T need no
// data movement; A^T, B^T (bf16) and c0 are staged in the free LDS stages.  Rows are
// scattered to token order through the query permutation.
template <int D, int LDS_BYTES, int NT>
__device__ __forceinline__ void fused_stage(const AttnArgs& A, int h, char* lds, int tid) {
  constexpr int RCM = kMaxCorrRank;  // up to 64 correction directions (two 32-row blocks of t)
  constexpr int AROW = D + 8;        // At[k][d] bf16, padded rows (conflict-free 16-byte reads)
  constexpr int BROW = RCM + 4;      // Bt[d][k] bf16, padded rows (conflict-free 8-byte reads)
  static_assert((RCM * AROW + D * BROW) * 2 + D * 4 <= LDS_BYTES, "fused write-back staging");
  bf16_t* At = reinterpret_cast<bf16_t*>(lds);
  bf16_t* Bt = At + RCM * AROW;
  float* c0s = reinterpret_cast<float*>(Bt + D * BROW);
  const int re = min(A.r_eff[h], min(A.rank, RCM));
  const float* Ah = A.fitA + (int64_t)h * D * A.rank;
  const float* Bh = A.fitB + (int64_t)h * A.rank * D;
  for (int idx = tid; idx < RCM * D; idx += NT) {
    const int k = idx / D, d = idx % D;
    At[k * AROW + d] = f32_to_bf16(k < re ? Ah[d * A.rank + k] : 0.f);
    Bt[d * BROW + k] = f32_to_bf16(k < re ? Bh[k * D + d] : 0.f);
  }
  for (int d = tid; d < D; d += NT) c0s[d] = A.fitc0[(int64_t)h * D + d];
  __syncthreads();
}

// The correction and scatter of one wave's 32 rows of query head h (group-major position
// p of KV head kv) from A^T, B^T and c0 staged by fused_stage.
template <int D>
__device__ __forceinline__ void fused_apply(const AttnArgs& A, int h, int kv, int p, bool qvalid, float inv,
                                            f32x16_t* o, const char* lds, int l32, int hf) {
  constexpr int DBLK = D / 32;
  constexpr int RCM = kMaxCorrRank;
  constexpr int AROW = D + 8;
  constexpr int BROW = RCM + 4;
  const bf16_t* At = reinterpret_cast<const bf16_t*>(lds);
  const bf16_t* Bt = At + RCM * AROW;
  const float* c0s = reinterpret_cast<const float*>(Bt + D * BROW);
  const int re = min(A.r_eff[h], min(A.rank, RCM));
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
      bf16x8_t ob;
#pragma unroll
      for (int e = 0; e < 8; ++e) ob[e] = (__bf16)o[db][8 * s2 + e];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (kb == 1 && !two) break;
        const bf16_t* ar = At + (32 * kb + l32) * AROW + 32 * db + 16 * s2 + 4 * hf;
        const uint2 lo8 = *reinterpret_cast<const uint2*>(ar);
        const uint2 hi8 = *reinterpret_cast<const uint2*>(ar + 8);
        const uint4 av = make_uint4(lo8.x, lo8.y, hi8.x, hi8.y);
        t[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, av), ob, t[kb], 0, 0, 0);
      }
    }
  }
  // t^T[k][q] in the accumulator layout is the B operand over k of O^T += B^T t^T
  bf16x8_t tb[4];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    tb[0][e] = (__bf16)t[0][e];
    tb[1][e] = (__bf16)t[0][8 + e];
    tb[2][e] = (__bf16)t[1][e];
    tb[3][e] = (__bf16)t[1][8 + e];
  }
  const int ksteps = (re + 15) / 16;
#pragma unroll
  for (int db = 0; db < DBLK; ++db) {
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      if (s2 >= ksteps) break;
      const bf16_t* br = Bt + (32 * db + l32) * BROW + 16 * s2 + 4 * hf;
      const uint2 lo8 = *reinterpret_cast<const uint2*>(br);
      const uint2 hi8 = *reinterpret_cast<const uint2*>(br + 8);
      const uint4 bv = make_uint4(lo8.x, lo8.y, hi8.x, hi8.y);
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, bv), tb[s2], o[db], 0, 0, 0);
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

constexpr int kAttnWaves = 8;    // waves per block of the main attention kernel
constexpr int kAttnStages = 4;   // K/V tile stages in LDS; tile j + 2 is copied while tile j runs

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

template <int D, int BN, typename OutT>
__global__ __launch_bounds__(64 * kAttnWaves, 1) void attn_mfma_kernel(AttnArgs A) {
  using C = MfmaCfg<D, BN, kAttnWaves>;
  constexpr int PER_TILE = C::KIPW + C::VIPW;
  __shared__ __attribute__((aligned(1024))) char stages[kAttnStages][C::STAGE];

  // XCD-aware remap of the linear block id (consecutive logical tiles on one XCD)
  const int total = gridDim.x;
  const int per_xcd = total / kXcds;
  const int b = blockIdx.x;
  const int logical = (b % kXcds) * per_xcd + b / kXcds;
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
  const CopyPlan<D, BN, kAttnWaves> cp(wu, lane, A.v_np);
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

  // Tile iterators: (ci, k0, k1, kt) is the tile being computed; (fci, fk0, fk1, fkt) the
  // copy frontier, kAttnStages - 2 tiles ahead.  Tile j lives in stage j % kAttnStages.
  // The block meets at a barrier after every second tile (odd j) and after the last one:
  // a wave working on tile j has then passed the barrier after tile j - 1 or j - 2, so
  // every wave is done with tile j - 2, whose stage the copy of tile j + 2 reuses; and
  // before the barrier after an odd tile j each wave waits for its copies of tiles j + 1
  // and j + 2, the two tiles computed before the next barrier.  The barrier is a bare
  // s_barrier after the counted waits: the workgroup fence of __syncthreads() would also
  // drain the copies still in flight.
  int ci = ti.kbeg < 0 ? 0 : ti.kbeg, k0 = 0, k1 = 0, kt = 0;
  bool valid = next_run(A, kv, ti, ci, k0, k1);
  if (valid) kt = k0 & ~15;
  int fci = ci, fk0 = k0, fk1 = k1, fkt = kt;
  bool fvalid = valid;
  int nfront = 0;           // copied tiles not yet computed
  int fst = 0;              // stage of the frontier tile
  for (int i = 0; i < kAttnStages - 2 && fvalid; ++i) {
    stage_copy<D, BN, kAttnWaves>(cp, kb, vtb, A.n, A.v_np, fkt, stages[fst], wu);
    ++nfront;
    fst = fst == kAttnStages - 1 ? 0 : fst + 1;
    fvalid = next_tile(A, kv, ti, C::BN, fci, fk0, fk1, fkt);
  }
  wait_tiles_in_flight<PER_TILE>(nfront - 2);   // tiles 0 and 1 have landed
  __syncthreads();
  int cur = 0, j = 0;
  while (valid) {
    if (fvalid) {
      stage_copy<D, BN, kAttnWaves>(cp, kb, vtb, A.n, A.v_np, fkt, stages[fst], wu);
      ++nfront;
      fst = fst == kAttnStages - 1 ? 0 : fst + 1;
      fvalid = next_tile(A, kv, ti, C::BN, fci, fk0, fk1, fkt);
    }
    const int lo = max(k0 - kt, 0), hi = min(k1 - kt, BN);
    if (wave_rows)   // a wave whose rows all lie past the tile's end only keeps the copies and barriers
      mfma_tile_step<D, BN, false>(stages[cur], qreg, lo, hi, c2, nullptr, 0ull, m_i, l_i, o, l32, hf);
    --nfront;
    valid = next_tile(A, kv, ti, C::BN, ci, k0, k1, kt);
    if ((j & 1) || !valid) {
      wait_tiles_in_flight<PER_TILE>(nfront - 2);   // tiles j + 1 and j + 2 have landed
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    ++j;
    cur = cur == kAttnStages - 1 ? 0 : cur + 1;
  }

  const float l_tot = add_xor32(l_i);
  const float inv = 1.f / l_tot;
  if (A.fitA != nullptr) {
    fused_writeback<D, C::STAGE * kAttnStages, 64 * kAttnWaves>(A, kv, vrow, qvalid, inv, o, &stages[0][0], tid,
                                                                   l32, hf);
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

template <int D>
__global__ __launch_bounds__(256) void apply_mfma_kernel(AttnArgs A, const float* __restrict__ o_gm) {
  constexpr int LDS = (kMaxCorrRank * (D + 8) + D * (kMaxCorrRank + 4)) * 2 + D * 4;
  __shared__ __attribute__((aligned(16))) char lds[LDS];
  const int h = blockIdx.y, kv = h / A.g, j = h % A.g;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  fused_stage<D, LDS, 256>(A, h, lds, tid);
  // the staged A^T, B^T and c0 serve kApplyTiles tiles of 128 rows
  for (int it = 0; it < kApplyTiles; ++it) {
    const int p0 = (blockIdx.x * kApplyTiles + it) * 128;
    if (p0 >= A.n) break;
    const int p = p0 + 32 * w + l32;
    const bool valid = p < A.n;
    const float* row = o_gm + (((int64_t)kv * A.n + (valid ? p : 0)) * A.g + j) * D;
    f32x16_t o[D / 32];
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
    fused_apply<D>(A, h, kv, p, valid, 1.f, o, lds, l32, hf);
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
  if (dm.d == 128) hipLaunchKernelGGL(apply_mfma_kernel<128>, grid, dim3(256), 0, s, a, o_gm);
  else hipLaunchKernelGGL(apply_mfma_kernel<64>, grid, dim3(256), 0, s, a, o_gm);
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
      mfma_tile_step<D, 32, true>(stages[cur], qreg, 0, hi, c2, klab[cur], rowmask, m_i, l_i, o, l32, hf);
    else
      mfma_tile_step<D, 32, false>(stages[cur], qreg, 0, hi, c2, nullptr, 0ull, m_i, l_i, o, l32, hf);
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
                                                        int32_t* __restrict__ order, int32_t* __restrict__ count) {
  __shared__ int nkt[kMaxGroups], nqt[kMaxGroups], start[kMaxGroups];
  __shared__ int cl[kMaxGroups * kMaxGroups], ko[kMaxGroups + 1], rp[kMaxGroups + 1];
  const int kv = blockIdx.x, a = threadIdx.x;
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

void launch_tile_order(const Dims& dm, AttnArgs& a, char* region, hipStream_t s) {
  const int tph = attn_tiles_per_head(dm.n, dm.g, dm.gq);
  int32_t* order = reinterpret_cast<int32_t*>(region);
  int32_t* count = order + 2 * (int64_t)tph * dm.hkv;
  hipLaunchKernelGGL(tile_order_kernel, dim3(dm.hkv), dim3(64), 0, s, a.qoff, a.koff, a.row_ptr, a.cols, dm.gq, dm.gk,
                     dm.g, MfmaCfg<128, kAttnBN, kAttnWaves>::BM, kAttnBN, tph, order, count);
  a.order = order;
  a.order_count = count;
}

template <int D, typename OutT>
void launch_mfma_typed(AttnArgs a, int hkv, hipStream_t s) {
  a.tiles_per_head = (int)ceil_div((int64_t)a.n * a.g, MfmaCfg<D, kAttnBN, kAttnWaves>::BM) + (a.qoff ? a.gq : 0);
  a.n_heads_kv = hkv;
  int64_t total = (int64_t)a.tiles_per_head * hkv;
  total = ceil_div(total, kXcds) * kXcds;
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
