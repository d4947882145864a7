"""fp64 CPU oracle for scaled dot-product attention and its backward pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
package: only the test suite, the package's smoke check and the CPU-baseline leg
of the benchmark use it.  It shares no code with the HIP library.

Every function here is the plain definition of what it computes, written out in
fp64 with numpy: scores and probabilities are materialised in full and the
softmax gradient is the Jacobian-vector product of the row softmax.  None of
the GPU path's shortcuts (tiling, the rowsum(dO*O) term, atomics) appear.
"""
from .sdpa import (  # noqa: F401
    head_forward,
    head_backward,
    causal_mask,
    dense_forward,
    dense_backward,
    varlen_forward,
    varlen_backward,
    selected_key_positions,
    selected_block_lists,
    selected_forward,
    selected_backward,
    rowsum_do_o,
)
