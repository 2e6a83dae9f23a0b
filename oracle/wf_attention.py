"""Oracle attention: the plain definition of softmax attention, fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

WF ("Wave Forcing: Towards Speed-of-Light Streaming Video Generation")
§3.1, Eq. 4-5: a query chunk attends to the concatenation of its ordered
context, with full attention inside and across the readable chunks; chunks
the mask excludes are simply absent from the context.  The scale 1/sqrt(d)
is not on the page; it is the usual scaled-dot-product choice.
"""

import numpy as np


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
           block: int = 1024) -> np.ndarray:
    """softmax(scale q k^T) v for q [Nq, d], k [Nk, d], v [Nk, d]; fp64.

    Blocked over query rows only, to bound memory; each row is computed
    independently, so blocking changes nothing.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    out = np.empty((q.shape[0], v.shape[1]), dtype=np.float64)
    for r0 in range(0, q.shape[0], block):
        s = scale * (q[r0:r0 + block] @ k.T)
        s -= s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[r0:r0 + block] = p @ v
    return out


def attend_heads(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                 scale: float) -> np.ndarray:
    """Per-head attention: q [Nq, H, d], k/v [Nk, H, d] -> [Nq, H, d]."""
    out = np.empty(q.shape, dtype=np.float64)
    for h in range(q.shape[1]):
        out[:, h, :] = attend(q[:, h, :], k[:, h, :], v[:, h, :], scale)
    return out
