"""fp64 CPU oracle for the batch-invariant GEMM.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package's ``smoke()`` check and the
benchmark may import this module.  It shares no code with the HIP path.

What it computes (RL-Kernel PR "MFMA batch-invariant GEMM and chunked Triton
attention" page, section 1): ``C = A B`` for bf16 operands with fp32
accumulation and one final bf16 rounding, the weight given either as
``[N, K]`` (``C = A W^T``, the layer-weight view) or as ``[K, N]``.  The method
consumes K in ascending 64-wide blocks inside fixed 1024-wide chunks and adds
the chunk partials in ascending order; in exact arithmetic that is the plain
product, which is what the oracle returns.

Two evaluations:
  ``gemm``          the plain definition, one BLAS matrix product in fp64;
  ``gemm_chunked``  the method's steps in fp64: 64-wide K blocks accumulated
                    in ascending order inside each 1024-wide chunk from zero,
                    chunk partials folded left to right.  It agrees with
                    ``gemm`` to fp64 rounding; the tests check that.
"""
from __future__ import annotations

import numpy as np

BLOCK_K = 64     # K per block (method page, section 1)
CHUNK_K = 1024   # K per chunk partial (same section)


def _operands(a, w, weight_nk: bool):
    a = np.asarray(a, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    b = w.T if weight_nk else w  # [K, N]
    assert a.ndim == 2 and b.ndim == 2 and a.shape[1] == b.shape[0]
    return a, b


def gemm(a, w, weight_nk: bool = True) -> np.ndarray:
    """C[M, N] = A[M, K] @ B[K, N] in fp64, B = W^T for an [N, K] weight."""
    a, b = _operands(a, w, weight_nk)
    return a @ b


def gemm_chunked(a, w, weight_nk: bool = True) -> np.ndarray:
    """The method's order in fp64: per 1024-wide chunk, 64-wide K blocks added
    in ascending order to a zero partial; partials folded in ascending order."""
    a, b = _operands(a, w, weight_nk)
    m, k = a.shape
    total = np.zeros((m, b.shape[1]))
    for c0 in range(0, k, CHUNK_K):
        part = np.zeros_like(total)
        for k0 in range(c0, min(c0 + CHUNK_K, k), BLOCK_K):
            k1 = min(k0 + BLOCK_K, k)
            part = part + a[:, k0:k1] @ b[k0:k1, :]
        total = total + part
    return total


def gemm_flops(m: int, n: int, k: int) -> int:
    """Algorithmic FLOP count of C = A B: 2 M N K."""
    return 2 * int(m) * int(n) * int(k)
