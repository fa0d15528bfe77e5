"""ctypes binding of libsparsepr.so (include/sparsepr.h).

Argument marshalling only: torch supplies device memory and the current HIP stream;
every step of the call runs in the library's kernels.  Loading fails loudly when the
library has not been built.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsparsepr.so")

BF16, FP32 = 0, 1
ABLATE_NONE, ABLATE_HARD_DROP, ABLATE_RIDGE_ONLY = 0, 1, 2
PROBES_RADIAL, PROBES_UNIFORM, PROBES_GIVEN = 0, 1, 2
PARTITION_RESPONSE, PARTITION_SEMANTIC = 0, 1
BUDGET_PER_HEAD, BUDGET_GLOBAL = 0, 1
COST_PAIRS, COST_TILES = 0, 1
STATUS = {0: "ok", -1: "null pointer", -2: "shape", -3: "dtype", -4: "alignment",
          -5: "workspace", -6: "parameter", -7: "HIP failure"}


class Params(ctypes.Structure):
    _fields_ = [("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32), ("n", ctypes.c_int32),
                ("d", ctypes.c_int32), ("dtype", ctypes.c_int32), ("groups_q", ctypes.c_int32),
                ("groups_k", ctypes.c_int32), ("r_k", ctypes.c_int32), ("r_q", ctypes.c_int32),
                ("n_probe", ctypes.c_int32), ("rank", ctypes.c_int32), ("lam", ctypes.c_float),
                ("rho_exec", ctypes.c_float), ("block", ctypes.c_int32),
                ("kmeans_iters", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("ablation", ctypes.c_int32), ("probe_mode", ctypes.c_int32),
                ("partition_mode", ctypes.c_int32), ("budget_mode", ctypes.c_int32),
                ("cost_mode", ctypes.c_int32), ("defer_kv_gather", ctypes.c_int32)]


def _ptr_struct(name, names):
    return type(name, (ctypes.Structure,), {"_fields_": [(n, ctypes.c_void_p) for n in names]})


PARTITION_FIELDS = ["responses_s", "responses_u", "exponents", "key_labels", "key_centroids_int",
                    "key_perm", "key_offsets", "key_centroids", "query_features", "query_labels",
                    "query_centroids", "query_perm", "query_offsets", "q_gm", "k_gm", "v_gm",
                    "query_coord_sum"]
ROUTE_FIELDS = ["row_ptr", "cols", "kept_mask", "pairs", "cell_mass"]
FIT_FIELDS = ["probe_tokens", "probe_groups", "probe_weights", "o_dense", "o_sparse", "A", "B", "c0",
              "r_eff", "eig"]

PartitionT = _ptr_struct("PartitionT", PARTITION_FIELDS)
RouteT = _ptr_struct("RouteT", ROUTE_FIELDS)
FitT = _ptr_struct("FitT", FIT_FIELDS)

EXPORTS = ["sparsepr_workspace_size", "sparsepr_partition", "sparsepr_gather_kv", "sparsepr_route", "sparsepr_attend",
           "sparsepr_attend_noalloc",
           "sparsepr_probe_fit", "sparsepr_apply", "sparsepr_attend_apply", "sparsepr_dense_attention",
           "sparsepr_diagnostics_workspace_size", "sparsepr_residual_diagnostics",
           "sparsepr_support_workspace_size", "sparsepr_support_diagnostics", "sparsepr_status_string"]

_lib = None


class SparsePRError(RuntimeError):
    pass


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} not built: run `python -m free_block_sparse_sparsepr_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    sigs = {
        "sparsepr_workspace_size": [P(Params), P(ctypes.c_size_t)],
        "sparsepr_partition": [P(Params), vp, vp, vp, P(PartitionT), vp, sz, vp],
        "sparsepr_gather_kv": [P(Params), vp, vp, P(PartitionT), vp],
        "sparsepr_route": [P(Params), P(PartitionT), P(RouteT), vp, sz, vp],
        "sparsepr_attend": [P(Params), P(PartitionT), P(RouteT), vp, vp, vp, sz, vp],
        "sparsepr_attend_noalloc": [P(Params), P(PartitionT), P(RouteT), vp, vp, vp],
        "sparsepr_probe_fit": [P(Params), vp, P(PartitionT), P(RouteT), P(FitT), vp, sz, vp],
        "sparsepr_apply": [P(Params), vp, P(PartitionT), P(FitT), vp, vp],
        "sparsepr_attend_apply": [P(Params), P(PartitionT), P(RouteT), P(FitT), vp, vp, sz, vp],
        "sparsepr_dense_attention": [P(Params), vp, vp, vp, vp, vp, sz, vp],
        "sparsepr_diagnostics_workspace_size": [P(Params), P(ctypes.c_size_t)],
        "sparsepr_residual_diagnostics": [P(Params), vp, vp, vp, P(PartitionT), P(RouteT), vp, vp, sz, vp],
        "sparsepr_support_workspace_size": [P(Params), ctypes.c_int, ctypes.c_int, P(ctypes.c_size_t)],
        "sparsepr_support_diagnostics": [P(Params), vp, vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                         vp, vp, vp, sz, vp],
    }
    for name, args in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.sparsepr_status_string.argtypes = [ctypes.c_int]
    lib.sparsepr_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def check(status):
    if status != 0:
        msg = load().sparsepr_status_string(status).decode()
        raise SparsePRError(f"sparsepr status {status}: {msg}")
