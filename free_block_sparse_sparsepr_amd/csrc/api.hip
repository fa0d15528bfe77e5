// C ABI of the SparsePR call: argument validation, workspace planning and launch order.
// The operations themselves are documented in include/sparsepr.h.
#include <cmath>
#include <mutex>
#include <unordered_set>

#include "sp_common.hpp"
#include "sp_launch.hpp"

namespace sp {

Dims dims_of(const sparsepr_params& p) {
  Dims d;
  d.hq = p.heads_q;
  d.hkv = p.heads_kv;
  d.g = p.heads_q / p.heads_kv;
  d.n = p.n;
  d.d = p.d;
  d.gq = p.groups_q;
  d.gk = p.groups_k;
  d.rk = p.r_k;
  d.m = p.n_probe;
  d.r = p.rank;
  d.iters = p.kmeans_iters;
  d.ablation = p.ablation;
  d.probe_mode = p.probe_mode;
  d.semantic = p.partition_mode == SPARSEPR_PARTITION_SEMANTIC;
  d.fq = d.semantic ? p.d : p.groups_k;
  d.rc = p.ablation == SPARSEPR_ABLATE_RIDGE_ONLY ? p.n_probe : p.rank;
  d.global_budget = p.budget_mode == SPARSEPR_BUDGET_GLOBAL;
  d.tile = p.cost_mode == SPARSEPR_COST_TILES ? p.block : 0;
  d.scale = p.softmax_scale > 0.f ? p.softmax_scale : (float)(1.0 / std::sqrt((double)p.d));
  d.lambda = p.lambda;
  d.bf16 = p.dtype == SPARSEPR_BF16;
  return d;
}

static size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

Workspace plan_workspace(const sparsepr_params& p) {
  Workspace w{};
  const size_t n = (size_t)p.n, hkv = (size_t)p.heads_kv, hq = (size_t)p.heads_q;
  const bool semantic = p.partition_mode == SPARSEPR_PARTITION_SEMANTIC;
  w.fpk = semantic ? p.d : round_up4(p.r_k);
  w.fpq = semantic ? p.d : round_up4(p.groups_k);
  const int fpmax = w.fpk > w.fpq ? w.fpk : w.fpq;
  size_t o = 0;
  w.maxbits = o; o = align_up(o + hkv * 2 * 4);
  w.xk = o; o = align_up(o + hkv * n * w.fpk);
  w.xq = o; o = align_up(o + hkv * n * w.fpq);
  w.centroids = o; o = align_up(o + 2 * hkv * kMaxGroups * fpmax * 4);
  w.sums = o; o = align_up(o + 3 * hkv * kMaxGroups * (fpmax + 1) * 4);
  w.usum = o; if (p.heads_q != p.heads_kv) o = align_up(o + hkv * n * p.groups_k * 4);
  w.gm_hist = o; o = align_up(o + hkv * (size_t)ceil_div(p.n, kGmChunk) * kMaxGroups * 4);
  w.total_partition = o;
  w.nchunks = (int)ceil_div(p.n, probe_chunk(p.n));
  o = 0;
  w.probe_alloc = o; o = align_up(o + hkv * n * 4);
  w.partials = o; o = align_up(o + hq * w.nchunks * p.n_probe * 2 * (p.d + 2) * 4);
  w.fitbuf = o; o = align_up(o + hq * (size_t)FitBuf::per_head(p.d) * 8);
  w.total_probe = o;
  w.dense_meta = 0;
  w.dense_claim = align_up(hkv * (size_t)p.d * (size_t)vt_pad(p.n) * (p.dtype == SPARSEPR_BF16 ? 2 : 4));
  w.total_dense = align_up(w.dense_claim + 64);   // the attention's eight tile-claim counters
  // the fused write-back runs in the attention epilogue for bf16 (under GQA with the query
  // heads' corrections applied in turn); for fp32 attend writes O_gm into the workspace and
  // apply follows
  w.fused_ogm = 0;
  w.total_fused = p.dtype == SPARSEPR_BF16 ? 0 : align_up(hkv * n * (size_t)(p.heads_q / p.heads_kv) * p.d * 4);
  {
    const size_t cells = hkv * (size_t)p.groups_q * (size_t)p.groups_k;
    size_t r = 0;
    w.rt_order = r; r = align_up(r + cells * 4);
    w.rt_pos = r; r = align_up(r + cells * 4);
    w.rt_prefix = r; r = align_up(r + cells * 8);
    w.rt_cost = r; r = align_up(r + cells * 8);
    w.rt_kept = r; r = align_up(r + cells);
    w.rt_head = r; r = align_up(r + hkv * 16);
    w.total_route = p.budget_mode == SPARSEPR_BUDGET_GLOBAL ? r : 0;
  }
  w.total = w.total_partition;
  if (w.total_route > w.total) w.total = w.total_route;
  if (w.total_fused > w.total) w.total = w.total_fused;
  if (w.total_probe > w.total) w.total = w.total_probe;
  if (w.total_dense > w.total) w.total = w.total_dense;
  w.attn_order = align_up(w.total);
  w.total = align_up(w.attn_order + attn_order_bytes(p.n, p.heads_q / p.heads_kv, p.heads_kv, p.groups_q));
  return w;
}

static sparsepr_status check_params(const sparsepr_params* p) {
  if (!p) return SPARSEPR_ERR_NULL;
  if (p->dtype != SPARSEPR_BF16 && p->dtype != SPARSEPR_FP32) return SPARSEPR_ERR_DTYPE;
  if (p->n < 1 || p->n > (1 << 22)) return SPARSEPR_ERR_SHAPE;
  if (p->d != 64 && p->d != 128) return SPARSEPR_ERR_SHAPE;
  if (p->heads_q < 1 || p->heads_kv < 1 || p->heads_q % p->heads_kv != 0) return SPARSEPR_ERR_SHAPE;
  if (p->heads_q / p->heads_kv > 16) return SPARSEPR_ERR_SHAPE;
  if (p->groups_q < 1 || p->groups_q > kMaxGroups || p->groups_k < 1 || p->groups_k > kMaxGroups)
    return SPARSEPR_ERR_SHAPE;
  if (p->groups_q > p->n || p->groups_k > p->n) return SPARSEPR_ERR_SHAPE;
  if (p->r_q < 1 || p->groups_k > p->r_q) return SPARSEPR_ERR_PARAM;
  if (p->r_k < 1 || p->r_k > kMaxFeat) return SPARSEPR_ERR_PARAM;
  if (p->n_probe < 1 || p->n_probe > kMaxProbe || p->n_probe > p->n) return SPARSEPR_ERR_PARAM;
  if (p->rank < 1 || p->rank > kMaxRank || p->rank > p->n_probe || p->rank > p->d) return SPARSEPR_ERR_PARAM;
  if (!(p->lambda > 0.f) || !std::isfinite(p->lambda)) return SPARSEPR_ERR_PARAM;
  if (!(p->rho_exec <= 1.f) || !((double)p->rho_exec > (double)p->n_probe / (double)p->n)) return SPARSEPR_ERR_PARAM;
  if (p->kmeans_iters < 0 || p->kmeans_iters > 64) return SPARSEPR_ERR_PARAM;
  if (p->defer_kv_gather != 0 && p->defer_kv_gather != 1) return SPARSEPR_ERR_PARAM;
  if (p->block != 64) return SPARSEPR_ERR_PARAM;
  if (!(p->softmax_scale >= 0.f) || !std::isfinite(p->softmax_scale)) return SPARSEPR_ERR_PARAM;
  if (p->budget_mode != SPARSEPR_BUDGET_PER_HEAD && p->budget_mode != SPARSEPR_BUDGET_GLOBAL)
    return SPARSEPR_ERR_PARAM;
  if (p->cost_mode != SPARSEPR_COST_PAIRS && p->cost_mode != SPARSEPR_COST_TILES) return SPARSEPR_ERR_PARAM;
  if (p->ablation != SPARSEPR_ABLATE_NONE && p->ablation != SPARSEPR_ABLATE_HARD_DROP &&
      p->ablation != SPARSEPR_ABLATE_RIDGE_ONLY)
    return SPARSEPR_ERR_PARAM;
  if (p->probe_mode != SPARSEPR_PROBES_RADIAL && p->probe_mode != SPARSEPR_PROBES_UNIFORM &&
      p->probe_mode != SPARSEPR_PROBES_GIVEN)
    return SPARSEPR_ERR_PARAM;
  if (p->partition_mode != SPARSEPR_PARTITION_RESPONSE && p->partition_mode != SPARSEPR_PARTITION_SEMANTIC)
    return SPARSEPR_ERR_PARAM;
  return SPARSEPR_OK;
}

static bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

static sparsepr_status check_ws(const sparsepr_params* p, const void* ws, size_t bytes, size_t need_of_part) {
  (void)p;
  if (need_of_part > 0 && ws == nullptr) return SPARSEPR_ERR_NULL;
  if (bytes < need_of_part) return SPARSEPR_ERR_WORKSPACE;
  if (ws && ((uintptr_t)ws & 255u) != 0) return SPARSEPR_ERR_ALIGN;
  return SPARSEPR_OK;
}

static sparsepr_status hip_status() {
  return hipGetLastError() == hipSuccess ? SPARSEPR_OK : SPARSEPR_ERR_HIP;
}

// Route budget in pairs per head: floor(rho_ppm n^2 / 10^6) - M n with rho_ppm the
// target density rounded once to integer parts per million.
static int64_t route_budget(const sparsepr_params& p) {
  const int64_t ppm = (int64_t)std::floor((double)p.rho_exec * 1e6 + 0.5);
  const int64_t n = p.n;
  // ppm n^2 reaches 10^6 2^44 at the largest accepted n: formed in 128 bits
  const unsigned __int128 prod = (unsigned __int128)(uint64_t)ppm * (uint64_t)n * (uint64_t)n;
  return (int64_t)(prod / 1000000u) - (int64_t)p.n_probe * n;
}

// Attention arguments of the block-sparse path (group-major Q, K, transposed V, CSR).
static AttnArgs sparse_args(const Dims& dm, const sparsepr_partition_t& part, const sparsepr_route_t& route) {
  AttnArgs a{};
  a.q = part.q_gm;
  a.k = part.k_gm;
  a.v = part.v_gm;
  a.q_skv = (int64_t)dm.n * dm.g * dm.d;
  a.q_sp = (int64_t)dm.g * dm.d;
  a.q_sj = dm.d;
  a.kv_skv = (int64_t)dm.n * dm.d;
  a.v_np = (int)vt_pad(dm.n);
  a.v_skv = (int64_t)dm.d * a.v_np;
  a.qoff = part.query_offsets;
  a.koff = part.key_offsets;
  a.row_ptr = route.row_ptr;
  a.cols = route.cols;
  a.o_skv = a.q_skv;
  a.o_sp = a.q_sp;
  a.o_sj = a.q_sj;
  a.n = dm.n;
  a.g = dm.g;
  a.gq = dm.gq;
  a.gk = dm.gk;
  a.scale = dm.scale;
  return a;
}

// Attention arguments of the dense path (token order, V already transposed into vt).
static AttnArgs dense_args(const Dims& dm, const void* q, const void* k, const void* vt) {
  AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = vt;
  a.v_np = (int)vt_pad(dm.n);
  a.v_skv = (int64_t)dm.d * a.v_np;
  a.q_skv = (int64_t)dm.g * dm.n * dm.d;
  a.q_sp = dm.d;
  a.q_sj = (int64_t)dm.n * dm.d;
  a.kv_skv = (int64_t)dm.n * dm.d;
  a.o_skv = a.q_skv;
  a.o_sp = a.q_sp;
  a.o_sj = a.q_sj;
  a.n = dm.n;
  a.g = dm.g;
  a.gq = 1;
  a.gk = 1;
  a.scale = dm.scale;
  return a;
}

// Scratch of sparsepr_attend_noalloc: the attention's tile schedule (each KV head's query
// groups longest first) in a file-scope device array instead of the caller's workspace.
// Every GPU the library runs on holds its own copy until the process ends; host code uses
// the per-device address from hipGetSymbolAddress, never the array's name.
constexpr size_t kNoAllocScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

// The device address of `scratch` on the current device, looked up once per device.
static sparsepr_status scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return SPARSEPR_ERR_HIP;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return SPARSEPR_ERR_HIP;
    addr[dev] = ptr;
  }
  *out = addr[dev];
  return SPARSEPR_OK;
}

}  // namespace sp

using namespace sp;

extern "C" {

sparsepr_status sparsepr_workspace_size(const sparsepr_params* params, size_t* bytes) {
  sparsepr_status st = check_params(params);
  if (st != SPARSEPR_OK) return st;
  if (!bytes) return SPARSEPR_ERR_NULL;
  *bytes = plan_workspace(*params).total;
  return SPARSEPR_OK;
}

// Partitions made with defer_kv_gather = 1 whose K/V gathers have not been enqueued yet,
// keyed by their k_gm buffer: the entry points that read k_gm and v_gm refuse them
// (SPARSEPR_ERR_PARAM) instead of reading the previous call's rows.  Host-side and in call
// order, so a graph captured from a valid order replays without consulting it.
static std::mutex g_deferred_mu;
static std::unordered_set<const void*> g_deferred;

static void set_deferred(const void* k_gm, bool deferred) {
  std::lock_guard<std::mutex> lk(g_deferred_mu);
  if (deferred) g_deferred.insert(k_gm);
  else g_deferred.erase(k_gm);
}

static bool gathers_pending(const sparsepr_partition_t* part) {
  std::lock_guard<std::mutex> lk(g_deferred_mu);
  return part && g_deferred.count(part->k_gm) != 0;
}

sparsepr_status sparsepr_partition(const sparsepr_params* params, const void* q, const void* k, const void* v,
                                   const sparsepr_partition_t* out, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  sparsepr_status st = check_params(params);
  if (st != SPARSEPR_OK) return st;
  if (!q || !k || !v || !out) return SPARSEPR_ERR_NULL;
  const sparsepr_partition_t& o = *out;
  if (!o.responses_s || !o.responses_u || !o.exponents || !o.key_labels || !o.key_centroids_int || !o.key_perm ||
      !o.key_offsets || !o.key_centroids || !o.query_features || !o.query_labels || !o.query_centroids ||
      !o.query_perm || !o.query_offsets || !o.q_gm || !o.k_gm || !o.v_gm)
    return SPARSEPR_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o.q_gm) || !aligned16(o.k_gm) ||
      !aligned16(o.v_gm))
    return SPARSEPR_ERR_ALIGN;
  const Workspace wp = plan_workspace(*params);
  st = check_ws(params, workspace, workspace_bytes, wp.total_partition);
  if (st != SPARSEPR_OK) return st;
  (void)hipGetLastError();
  launch_partition(dims_of(*params), wp, q, k, v, o, static_cast<char*>(workspace), params->defer_kv_gather != 0,
                   (hipStream_t)stream);
  st = hip_status();
  if (st == SPARSEPR_OK) set_deferred(o.k_gm, params->defer_kv_gather != 0);
  return st;
}

sparsepr_status sparsepr_gather_kv(const sparsepr_params* params, const void* k, const void* v,
                                   const sparsepr_partition_t* part, void* stream) {
  sparsepr_status st = check_params(params);
  if (st != SPARSEPR_OK) return st;
  if (!k || !v || !part) return SPARSEPR_ERR_NULL;
  if (!part->key_perm || !part->k_gm || !part->v_gm) return SPARSEPR_ERR_NULL;
  if (!aligned16(k) || !aligned16(v) || !aligned16(part->k_gm) || !aligned16(part->v_gm)) return SPARSEPR_ERR_ALIGN;
  (void)hipGetLastError();
  launch_gather_kv(dims_of(*params), k, v, *part, (hipStream_t)stream);
  st = hip_status();
  if (st == SPARSEPR_OK) set_deferred(part->k_gm, false);
  return st;
}

sparsepr_status sparsepr_route(const sparsepr_params* params, const sparsepr_partition_t* part,
                               const sparsepr_route_t* out, void* workspace, size_t workspace_bytes, void* stream) {
  sparsepr_status st = check_params(params);
  if (st != SPARSEPR_OK) return st;
  if (!part || !out) return SPARSEPR_ERR_NULL;
  if (!part->responses_u || !part->query_labels || !part->query_offsets || !part->key_offsets)
    return SPARSEPR_ERR_NULL;
  if (!out->row_ptr || !out->cols || !out->kept_mask || !out->pairs || !out->cell_mass) return SPARSEPR_ERR_NULL;
  if (((uintptr_t)out->cell_mass & 7u) != 0) return SPARSEPR_ERR_ALIGN;
  const Workspace wp = plan_workspace(*params);
  st = check_ws(params, workspace, workspace_bytes, wp.total_route);
  if (st != SPARSEPR_OK) return st;
  (void)hipGetLastError();
  launch_route(dims_of(*params), route_budget(*params), *part, *out, wp, static_cast<char*>(workspace),
               (hipStream_t)stream);
  return hip_status();
}

sparsepr_status sparsepr_attend(const sparsepr_params* params, const sparsepr_partition_t* part,
                                const sparsepr_route_t* route, float* o_gm, float* lse, void* workspace,
                                size_t workspace_bytes, void* stream) {
  sparsepr_status st = check_params(params);
  if (st != SPARSEPR_OK) return st;
  if (!part || !route || !o_gm) return SPARSEPR_ERR_NULL;
  if (!part->q_gm || !part->k_gm || !part->v_gm || !part->query_offsets || !part->key_offsets || !route->row_ptr ||
      !route->cols)
    return SPARSEPR_ERR_NULL;
  if (!aligned16(part->q_gm) || !aligned16(part->k_gm) || !aligned16(part->v_gm) || !aligned16(o_gm))
    return SPARSEPR_ERR_ALIGN;
  if (gathers_pending(part)) return SPARSEPR_ERR_PARAM;   // sparsepr_gather_kv has not run
  const Workspace wp = plan_workspace(*params);
  st = check_ws(params, workspace, workspace_bytes, wp.total);
  if (st != SPARSEPR_OK) return st;
  const Dims dm = dims_of(*params);
  AttnArgs a = sparse_args(dm, *part, *route);
  a.o = o_gm;
  a.lse = lse;
  (void)hipGetLastError();
  if (dm.bf16) launch_tile_order(dm, a, static_cast<char*>(workspace) + wp.attn_order, (hipStream_t)stream);
  launch_attention(dm, a, false, (hipStream_t)stream);
  return hip_status();
}

sparsepr_status sparsepr_attend_noalloc(const sparsepr_params* params, const sparsepr_partition_t* part,
                                        const sparsepr_route_t* route, float* o_gm, float* lse, void* stream) {
  sparsepr_status st = check_params(params);
  if (st != SPARSEPR_OK) return st;
  if (!part || !route || !o_gm) return SPARSEPR_ERR_NULL;
  if (!part->q_gm || !part->k_gm || !part->v_gm || !part->query_offsets || !part->key_offsets || !route->row_ptr ||
      !route->cols)
    return SPARSEPR_ERR_NULL;
  if (!aligned16(part->q_gm) || !aligned16(part->k_gm) || !aligned16(part->v_gm) || !aligned16(o_gm))
    return SPARSEPR_ERR_ALIGN;
  if (gathers_pending(part)) return SPARSEPR_ERR_PARAM;   // sparsepr_gather_kv has not run
  const Dims dm = dims_of(*params);
  if (dm.bf16 && attn_order_bytes(dm.n, dm.g, dm.hkv, dm.gq) > kNoAllocScratchBytes) return SPARSEPR_ERR_WORKSPACE;
  void* scr = nullptr;
  if (dm.bf16) {
    st = scratch_address(&scr);
    if (st != SPARSEPR_OK) return st;
  }
  AttnArgs a = sparse_args(dm, *part, *route);
  a.o = o_gm;
  a.lse = lse;
  (void)hipGetLastError();
  if (dm.bf16) launch_tile_order(dm, a, static_cast<char*>(scr), (hipStream_t)stream);
  launch_attention(dm, a, false, (hipStream_t)stream);
  return hip_status();
}

sparsepr_status sparsepr_attend_apply(const sparsepr_params* params, const sparsepr_partition_t* part,
                                      const sparsepr_route_t* route, const sparsepr_fit_t* fit, void* o,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  sparsepr_status st = check_params(params);
  if (st != SPARSEPR_OK) return st;
  if (!part || !route || !fit || !o) return SPARSEPR_ERR_NULL;
  if (!part->q_gm || !part->k_gm || !part->v_gm || !part->query_offsets || !part->key_offsets ||
      !part->query_perm || !route->row_ptr || !route->cols)
    return SPARSEPR_ERR_NULL;
  if (!fit->A || !fit->B || !fit->c0 || !fit->r_eff || !fit->o_dense || !fit->probe_tokens) return SPARSEPR_ERR_NULL;
  if (!aligned16(part->q_gm) || !aligned16(part->k_gm) || !aligned16(part->v_gm) || !aligned16(o))
    return SPARSEPR_ERR_ALIGN;
  if (gathers_pending(part)) return SPARSEPR_ERR_PARAM;   // sparsepr_gather_kv has not run
  const Workspace wp = plan_workspace(*params);
  st = check_ws(params, workspace, workspace_bytes, wp.total);
  if (st != SPARSEPR_OK) return st;
  const Dims dm = dims_of(*params);
  AttnArgs a = sparse_args(dm, *part, *route);
  (void)hipGetLastError();
  if (dm.bf16) launch_tile_order(dm, a, static_cast<char*>(workspace) + wp.attn_order, (hipStream_t)stream);
  if (wp.total_fused == 0) {
    a.fitA = fit->A;
    a.fitB = fit->B;
    a.fitc0 = fit->c0;
    a.r_eff = fit->r_eff;
    a.rank = dm.rc;
    a.qperm = part->query_perm;
    a.out_tok = o;
    launch_attention(dm, a, false, (hipStream_t)stream);
    if (dm.ablation != SPARSEPR_ABLATE_HARD_DROP) launch_probe_writeback(dm, *fit, o, (hipStream_t)stream);
  } else {
    float* ogm = reinterpret_cast<float*>(static_cast<char*>(workspace) + wp.fused_ogm);
    a.o = ogm;
    launch_attention(dm, a, false, (hipStream_t)stream);
    launch_apply(dm, ogm, *part, *fit, o, (hipStream_t)stream);
  }
  return hip_status();
}

sparsepr_status sparsepr_probe_fit(const sparsepr_params* params, const void* q, const sparsepr_partition_t* part,
                                   const sparsepr_route_t* route, const sparsepr_fit_t* out, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  sparsepr_status st = check_params(params);
  if (st != SPARSEPR_OK) return st;
  if (!q || !part || !route || !out) return SPARSEPR_ERR_NULL;
  if (!part->query_features || !part->query_centroids || !part->query_perm || !part->query_offsets ||
      !part->query_labels || !part->key_offsets || !part->k_gm || !part->v_gm || !route->kept_mask)
    return SPARSEPR_ERR_NULL;
  if (!out->probe_tokens || !out->probe_groups || !out->probe_weights || !out->o_dense || !out->o_sparse ||
      !out->A || !out->B || !out->c0 || !out->r_eff || !out->eig)
    return SPARSEPR_ERR_NULL;
  if (!aligned16(q) || !aligned16(part->k_gm) || !aligned16(part->v_gm)) return SPARSEPR_ERR_ALIGN;
  if (gathers_pending(part)) return SPARSEPR_ERR_PARAM;   // sparsepr_gather_kv has not run
  const Workspace wp = plan_workspace(*params);
  st = check_ws(params, workspace, workspace_bytes, wp.total_probe);
  if (st != SPARSEPR_OK) return st;
  (void)hipGetLastError();
  launch_probe_fit(dims_of(*params), wp, q, *part, *route, *out, static_cast<char*>(workspace), (hipStream_t)stream);
  return hip_status();
}

sparsepr_status sparsepr_apply(const sparsepr_params* params, const float* o_gm, const sparsepr_partition_t* part,
                               const sparsepr_fit_t* fit, void* o, void* stream) {
  sparsepr_status st = check_params(params);
  if (st != SPARSEPR_OK) return st;
  if (!o_gm || !part || !fit || !o) return SPARSEPR_ERR_NULL;
  if (!part->query_perm || !fit->A || !fit->B || !fit->c0 || !fit->r_eff || !fit->o_dense || !fit->probe_tokens)
    return SPARSEPR_ERR_NULL;
  if (!aligned16(o_gm) || !aligned16(o)) return SPARSEPR_ERR_ALIGN;
  (void)hipGetLastError();
  launch_apply(dims_of(*params), o_gm, *part, *fit, o, (hipStream_t)stream);
  return hip_status();
}

sparsepr_status sparsepr_dense_attention(const sparsepr_params* params, const void* q, const void* k,
                                         const void* v, void* o, void* workspace, size_t workspace_bytes,
                                         void* stream) {
  sparsepr_status st = check_params(params);
  if (st != SPARSEPR_OK) return st;
  if (!q || !k || !v || !o) return SPARSEPR_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return SPARSEPR_ERR_ALIGN;
  const Workspace wp = plan_workspace(*params);
  st = check_ws(params, workspace, workspace_bytes, wp.total_dense);
  if (st != SPARSEPR_OK) return st;
  const Dims dm = dims_of(*params);
  (void)hipGetLastError();
  void* vt = static_cast<char*>(workspace) + wp.dense_meta;
  launch_transpose_v(dm, v, vt, (hipStream_t)stream);
  AttnArgs a = dense_args(dm, q, k, vt);
  a.o = o;
  if (dm.bf16)
    launch_dense_claims(dm, a, reinterpret_cast<int*>(static_cast<char*>(workspace) + wp.dense_claim),
                        (hipStream_t)stream);
  (void)hipGetLastError();
  launch_attention(dm, a, true, (hipStream_t)stream);
  return hip_status();
}

sparsepr_status sparsepr_diagnostics_workspace_size(const sparsepr_params* params, size_t* bytes) {
  sparsepr_status st = check_params(params);
  if (st != SPARSEPR_OK) return st;
  if (!bytes) return SPARSEPR_ERR_NULL;
  *bytes = plan_diagnostics(dims_of(*params)).total;
  return SPARSEPR_OK;
}

sparsepr_status sparsepr_residual_diagnostics(const sparsepr_params* params, const void* q, const void* k,
                                              const void* v, const sparsepr_partition_t* part,
                                              const sparsepr_route_t* route, double* out, void* workspace,
                                              size_t workspace_bytes, void* stream) {
  sparsepr_status st = check_params(params);
  if (st != SPARSEPR_OK) return st;
  if (!q || !k || !v || !part || !route || !out) return SPARSEPR_ERR_NULL;
  if (!part->q_gm || !part->k_gm || !part->v_gm || !part->query_offsets || !part->key_offsets ||
      !part->query_perm || !route->row_ptr || !route->cols)
    return SPARSEPR_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(part->q_gm) || !aligned16(part->k_gm) ||
      !aligned16(part->v_gm) || ((uintptr_t)out & 7u) != 0)
    return SPARSEPR_ERR_ALIGN;
  if (gathers_pending(part)) return SPARSEPR_ERR_PARAM;   // sparsepr_gather_kv has not run
  const Dims dm = dims_of(*params);
  const DiagWorkspace w = plan_diagnostics(dm);
  st = check_ws(params, workspace, workspace_bytes, w.total);
  if (st != SPARSEPR_OK) return st;
  char* ws = static_cast<char*>(workspace);
  (void)hipGetLastError();
  launch_transpose_v(dm, v, ws + w.vt, (hipStream_t)stream);
  launch_diagnostics(dm, w, dense_args(dm, q, k, ws + w.vt), sparse_args(dm, *part, *route), part->query_perm, out,
                     ws, (hipStream_t)stream);
  return hip_status();
}

sparsepr_status sparsepr_support_workspace_size(const sparsepr_params* params, int n_sets, int set_size,
                                                size_t* bytes) {
  sparsepr_status st = check_params(params);
  if (st != SPARSEPR_OK) return st;
  if (!bytes) return SPARSEPR_ERR_NULL;
  if (n_sets < 0 || set_size < 1 || set_size > kSupportMaxSet) return SPARSEPR_ERR_PARAM;
  *bytes = support_workspace_bytes(dims_of(*params), n_sets, set_size);
  return SPARSEPR_OK;
}

sparsepr_status sparsepr_support_diagnostics(const sparsepr_params* params, const void* q, const void* k,
                                             const int32_t* sets, int n_sets, int set_size, double mass,
                                             int32_t* row_support, int32_t* shared_support, void* workspace,
                                             size_t workspace_bytes, void* stream) {
  sparsepr_status st = check_params(params);
  if (st != SPARSEPR_OK) return st;
  if (n_sets < 0 || set_size < 1 || set_size > kSupportMaxSet || !(mass > 0.0 && mass <= 1.0))
    return SPARSEPR_ERR_PARAM;
  if (n_sets == 0) return SPARSEPR_OK;
  if (!q || !k || !sets || !row_support || !shared_support) return SPARSEPR_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || ((uintptr_t)sets & 3u) || ((uintptr_t)row_support & 3u) ||
      ((uintptr_t)shared_support & 3u))
    return SPARSEPR_ERR_ALIGN;
  const Dims dm = dims_of(*params);
  st = check_ws(params, workspace, workspace_bytes, support_workspace_bytes(dm, n_sets, set_size));
  if (st != SPARSEPR_OK) return st;
  (void)hipGetLastError();
  launch_support(dm, q, k, sets, n_sets, set_size, mass, row_support, shared_support, workspace,
                 (hipStream_t)stream);
  return hip_status();
}

const char* sparsepr_status_string(sparsepr_status status) {
  switch (status) {
    case SPARSEPR_OK: return "ok";
    case SPARSEPR_ERR_NULL: return "a required pointer is NULL";
    case SPARSEPR_ERR_SHAPE: return "shape out of range (n, d, heads or groups)";
    case SPARSEPR_ERR_DTYPE: return "unsupported dtype";
    case SPARSEPR_ERR_ALIGN: return "misaligned pointer";
    case SPARSEPR_ERR_WORKSPACE: return "workspace too small";
    case SPARSEPR_ERR_PARAM: return "parameter out of range";
    case SPARSEPR_ERR_HIP: return "HIP runtime or launch failure";
  }
  return "unknown status";
}

}  // extern "C"
