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

// Global -> registers for one K/V tile.  K: thread t loads 64 contiguous bytes of key
// t / 4; V: thread t loads 16 bytes of each of keys 4 (t / 16) .. +3 at d = 8 (t % 16).
// Rows at or beyond k1 are zero.
template <int D>
__device__ __forceinline__ void stage_load(const bf16_t* __restrict__ kb, const bf16_t* __restrict__ vb, int kt,
                                           int k1, int tid, Stage<D>& st) {
  static_assert(D == 128 || D == 64, "head dim");
  if constexpr (D == 128) {
    const int key = tid >> 2, c = (tid & 3) * 32;
    const bool in = kt + key < k1;
    const uint4* src = reinterpret_cast<const uint4*>(kb + (int64_t)(kt + key) * D + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) st.k[i] = in ? src[i] : make_uint4(0, 0, 0, 0);
    const int kq = tid >> 4, dc = (tid & 15) * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key2 = 4 * kq + i;
      st.v[i] = (kt + key2 < k1) ? *reinterpret_cast<const uint4*>(vb + (int64_t)(kt + key2) * D + dc)
                                 : make_uint4(0, 0, 0, 0);
    }
  } else {
    // D = 64: thread t loads 32 contiguous bytes of key t / 4 (K) and 16 bytes of keys
    // 2 (t / 8) and 2 (t / 8) + 1 at d = 8 (t % 8) (V)
    const int key = tid >> 2, c = (tid & 3) * 16;
    const bool in = kt + key < k1;
    const uint4* src = reinterpret_cast<const uint4*>(kb + (int64_t)(kt + key) * D + c);
#pragma unroll
    for (int i = 0; i < 2; ++i) st.k[i] = in ? src[i] : make_uint4(0, 0, 0, 0);
    const int kp = tid >> 3, dc = (tid & 7) * 8;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int key2 = 2 * kp + i;
      st.v[i] = (kt + key2 < k1) ? *reinterpret_cast<const uint4*>(vb + (int64_t)(kt + key2) * D + dc)
                                 : make_uint4(0, 0, 0, 0);
    }
  }
}

// Registers -> LDS (K row-major, V transposed).
template <int D>
__device__ __forceinline__ void stage_store(bf16_t* __restrict__ Ks, bf16_t* __restrict__ Vt, int tid,
                                            const Stage<D>& st) {
  using C = MfmaCfg<D>;
  if constexpr (D == 128) {
    const int key = tid >> 2, c = (tid & 3) * 32;
    uint4* dst = reinterpret_cast<uint4*>(Ks + key * C::KROW + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = st.k[i];
    const int kq = tid >> 4, dc = (tid & 15) * 8;
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
    const int key = tid >> 2, c = (tid & 3) * 16;
    uint4* dst = reinterpret_cast<uint4*>(Ks + key * C::KROW + c);
#pragma unroll
    for (int i = 0; i < 2; ++i) dst[i] = st.k[i];
    // D = 64 V: thread t holds keys 2 (t / 8) and 2 (t / 8) + 1 at d = 8 (t % 8) .. +7;
    // each d row receives the key pair as one 32-bit word.
    const int kp = tid >> 3, dc = (tid & 7) * 8;
    const int keyb = 2 * kp;
    const uint32_t* x0 = reinterpret_cast<const uint32_t*>(&st.v[0]);
    const uint32_t* x1 = reinterpret_cast<const uint32_t*>(&st.v[1]);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      *reinterpret_cast<uint32_t*>(Vt + (dc + 2 * w) * C::VROW + keyb) = pack_lo(x0[w], x1[w]);
      *reinterpret_cast<uint32_t*>(Vt + (dc + 2 * w + 1) * C::VROW + keyb) = pack_hi(x0[w], x1[w]);
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

    const bf16_t* ks = Ks[cur];
    const bf16_t* vt = Vt[cur];
    // S^T blocks: keys 32 kb + (8 (r / 4) + 4 hf + r % 4), query l32
    f32x16_t s[2];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb2][r] = 0.f;
      const bf16_t* krow = ks + (32 * kb2 + l32) * C::KROW + 8 * hf;
#pragma unroll
      for (int kk = 0; kk < C::KSTEPS; ++kk) {
        bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(krow + 16 * kk);
        s[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[kk], s[kb2], 0, 0, 0);
      }
    }
    // scale to the log2 domain, mask keys beyond the run, tile max
    const int nk = it.k1 - it.kt;
    float mx = -INFINITY;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * kb2 + 8 * (r >> 2) + 4 * hf + (r & 3);
        float x = s[kb2][r] * c2;
        x = key < nk ? x : -INFINITY;
        s[kb2][r] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_i, mx);
    const float alpha = exp2f(m_i - m_new);
    float rs = 0.f;
    bf16x8_t p[2][2];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = exp2f(s[kb2][r] - m_new);
        rs += e;
        p[kb2][r >> 3][r & 7] = (__bf16)e;
      }
    l_i = l_i * alpha + rs;
    m_i = m_new;
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
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, av), p[kb2][s2], o[db],
                                                          0, 0, 0);
        }
      }
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
