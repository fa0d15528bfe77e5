"""CPU oracle of the SparsePR attention call — TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import it.
It shares no code with the GPU library (free_block_sparse_sparsepr_amd).
"""
from . import sparsepr  # noqa: F401
