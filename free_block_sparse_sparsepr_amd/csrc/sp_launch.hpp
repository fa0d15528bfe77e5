// Host-side launchers of the SparsePR kernels (internal to the library).
#pragma once
#include "sp_attn.hpp"
#include "sp_common.hpp"

namespace sp {


void launch_resp_s_mfma(const Dims& dm, const void* q, const void* k, float* S, uint32_t* maxbits, hipStream_t s);
void launch_resp_u_mfma(const Dims& dm, const void* q, const float* Ck, float* U, float* Usum, uint32_t* maxbits,
                        hipStream_t s);

// V [Hkv][n][d] (token order) -> transposed layout [Hkv][d][n_pad] (see vt_pos).
void launch_transpose_v(const Dims& dm, const void* v, void* vt, hipStream_t s);
// defer_kv: leave the K and V gathers (k_gm, v_gm) to launch_gather_kv.
void launch_partition(const Dims& dm, const Workspace& wp, const void* q, const void* k, const void* v,
                      const sparsepr_partition_t& out, char* ws, bool defer_kv, hipStream_t s);
void launch_gather_kv(const Dims& dm, const void* k, const void* v, const sparsepr_partition_t& part, hipStream_t s);
void launch_route(const Dims& dm, int64_t budget, const sparsepr_partition_t& part, const sparsepr_route_t& out,
                  const Workspace& wp, char* ws, hipStream_t s);
// out_is_input_dtype: output element type equals Q's (dense baseline); otherwise fp32.
void launch_attention(const Dims& dm, AttnArgs a, bool out_is_input_dtype, hipStream_t s);
void launch_attention_mfma(const Dims& dm, AttnArgs a, bool out_is_input_dtype, hipStream_t s);
// Longest-first order of the block-sparse attention's query tiles (matrix-core path): bytes of
// its workspace region, and the kernel that fills it and points `a` at it.
size_t attn_order_bytes(int n, int g, int hkv, int gq);
void launch_tile_order(const Dims& dm, AttnArgs& a, char* region, hipStream_t s);
void launch_dense_claims(const Dims& dm, AttnArgs& a, int* claim, hipStream_t s);
void launch_probe_attn_mfma(const Dims& dm, const void* q, const sparsepr_partition_t& part,
                            const sparsepr_route_t& route, const sparsepr_fit_t& fit, int chunk, int nchunks,
                            float* partials, hipStream_t s);
void launch_probe_fit(const Dims& dm, const Workspace& wp, const void* q, const sparsepr_partition_t& part,
                      const sparsepr_route_t& route, const sparsepr_fit_t& out, char* ws, hipStream_t s);
void launch_probe_writeback(const Dims& dm, const sparsepr_fit_t& fit, void* o, hipStream_t s);
void launch_apply(const Dims& dm, const float* o_gm, const sparsepr_partition_t& part, const sparsepr_fit_t& fit,
                  void* o, hipStream_t s);
// bf16 write-back on the matrix cores (the fused epilogue's arithmetic on stored rows)
void launch_apply_mfma(const Dims& dm, const float* o_gm, const sparsepr_partition_t& part,
                       const sparsepr_fit_t& fit, void* o, hipStream_t s);

// Residual diagnostics: workspace offsets and the launch (dense and sparse AttnArgs are
// filled by the caller except for their outputs).
struct DiagWorkspace {
  size_t o_dense, o_gm, vt, part, scratch, total;
};
DiagWorkspace plan_diagnostics(const Dims& dm);
void launch_diagnostics(const Dims& dm, const DiagWorkspace& w, AttnArgs dense, AttnArgs sparse,
                        const int32_t* qperm, double* out, char* ws, hipStream_t s);

// Support diagnostics: at most kSupportMaxSet queries per set, kSupportSlots concurrent
// (head, set) items, each with its own score slot in the workspace.
constexpr int kSupportMaxSet = 16;
constexpr int kSupportSlots = 512;
size_t support_workspace_bytes(const Dims& dm, int n_sets, int set_size);
void launch_support(const Dims& dm, const void* q, const void* k, const int32_t* sets, int n_sets, int set_size,
                    double mass, int32_t* row_out, int32_t* union_out, void* ws, hipStream_t s);

}  // namespace sp
