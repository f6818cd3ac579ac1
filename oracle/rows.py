"""Reading stored rows, and the per-request status bits of the verify contract.

TEST INFRASTRUCTURE (see the package docstring).

Status bits, as the library's contract defines them (a request carrying any of
the INVALID_FLAGS gets no output: count 0, accepted 0, every token -1):

  1  FLAG_BAD_REQUEST  draft count outside [0, k_max], a row index out of range,
                       or a context length outside [0, stride]
  2  FLAG_BAD_TOKEN    a draft token outside [0, V)
  4  FLAG_NONFINITE    a target row whose normaliser is not finite and positive
                       (sampled), a NaN in a target row (greedy), a NaN in the
                       draft row a residual is taken from, or a non-finite
                       residual mass
  8  FLAG_OVER_BUDGET  more drafts than the request's remaining budget
                       (the output is still produced and truncated)
 16  FLAG_FALLBACK     the residual had zero mass; the token was drawn from p
 32  FLAG_BAD_TREE     a tree whose root is not node 0 or where some node's
                       parent does not come before it
"""
import numpy as np

FLAG_BAD_REQUEST = 1
FLAG_BAD_TOKEN = 2
FLAG_NONFINITE = 4
FLAG_OVER_BUDGET = 8
FLAG_FALLBACK = 16
FLAG_BAD_TREE = 32
INVALID_FLAGS = FLAG_BAD_REQUEST | FLAG_BAD_TOKEN | FLAG_NONFINITE | FLAG_BAD_TREE


def widen(row, kind: str) -> np.ndarray:
    """A stored row as float64.  ``f32``: float32 values.  ``f64``: float64
    values (used by the oracle's own pins only).  ``bf16``: uint16 bit
    patterns; a bfloat16 is the upper half of a float32, so the value is the
    pattern shifted left by 16 and read as float32 (exact)."""
    if kind == "f32":
        return np.asarray(row, dtype=np.float32).astype(np.float64)
    if kind == "f64":
        return np.asarray(row, dtype=np.float64)
    if kind == "bf16":
        bits = np.asarray(row, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown row kind {kind!r}")
