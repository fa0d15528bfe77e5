"""SparsePR attention call on AMD Instinct MI355X (gfx950): hand-written HIP kernels behind
the C ABI in include/sparsepr.h, with a thin ctypes front end."""
from ._binding import EXPORTS, SparsePRError, load  # noqa: F401
from .sparsepr import Config, PipelinedSparsePR, SparsePR, config_from_workload, workspace_bytes  # noqa: F401
