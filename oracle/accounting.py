"""Tensor-payload accounting of exact attention -- TEST INFRASTRUCTURE.

Restates the memory-budget exercise of "FlashAttention Interview Questions: IO
Complexity, Tiling, and Numerical Stability" (cswork.org), section "Which complexity
becomes smaller, and which does not?" and its payload table: one head, one
sequence, a fixed number of bytes per stored element, tensor payloads only (no
allocator reservations).  The N-by-N score matrix is the object tiling never
stores in HBM; the N-by-d tensors (Q, K, V, output) are what remains.

Also the element counts of "FlashAttention 1, 2 & 3: Memory Tiling & Eliminating the
O(N^2) HBM Bottleneck" (learn-interview-questions, Q18), section 1.

MiB is 2**20 bytes.
"""

MIB = 1 << 20


def score_matrix_elements(N: int) -> int:
    """Elements of one N-by-N score matrix."""
    return N * N


def score_matrix_bytes(N: int, elem_bytes: int) -> int:
    return score_matrix_elements(N) * elem_bytes


def head_tensor_elements(N: int, d: int) -> int:
    """Elements of one N-by-d tensor (Q, K, V or the output)."""
    return N * d


def head_tensor_bytes(N: int, d: int, elem_bytes: int) -> int:
    return head_tensor_elements(N, d) * elem_bytes


def qkvo_bytes(N: int, d: int, elem_bytes: int) -> int:
    """Q, K, V and the output together."""
    return 4 * head_tensor_bytes(N, d, elem_bytes)
