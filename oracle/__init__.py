"""fp64 CPU oracle for C = A.B -- TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check and the bench's CPU-baseline leg may import this
package.  The HIP path never imports, links or calls it, and it imports nothing
from the HIP path.  See oracle.c for what is computed and why.
"""
from .oracle import (  # noqa: F401
    build, gemm, gemm_sampled, gemm_strided_batched, epilogue, ACT_NONE, ACT_RELU, ACT_GELU, normalised_error, num_threads, library_path,
)
