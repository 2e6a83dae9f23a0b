"""Oracle 3D rotary position embedding, fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

WF ("Wave Forcing: Towards Speed-of-Light Streaming Video Generation")
§4.1 (Eq. 8) puts RoPE inside the producer step P_{s,l} with the QKV
projection, and App. B.3 keeps the anchor's unrotated key so RoPE can be
applied again at a shifted position.  The page gives no axis split, so this
is the reading used here:

* d/2 rotation pairs, split over (frame, row, column) as
  n_t = d/2 - 2 floor(d/6), n_h = n_w = floor(d/6)  (d=128 -> 22, 21, 21).
* Pair p rotates the interleaved elements (x[2p], x[2p+1]); pairs
  [0, n_t) use the frame position, then n_h pairs the row, then n_w the
  column.  Inside an axis with n_a pairs, pair m has frequency
  theta^(-m / n_a).
* The rotation is (x0, x1) -> (x0 cos a - x1 sin a, x0 sin a + x1 cos a)
  with a = position * frequency.
* Token n of a chunk sits at frame n // (Hh Ww), row (n // Ww) % Hh,
  column n % Ww; the frame position is the chunk's first frame plus that
  frame index.
"""

import numpy as np


def axis_split(head_dim: int):
    """Number of rotation pairs given to the frame, row and column axes."""
    nh = head_dim // 6
    nt = head_dim // 2 - 2 * nh
    return nt, nh, nh


def token_positions(frame0: int, F: int, Hh: int, Ww: int):
    """(frame, row, column) of every token of a chunk, token-major order."""
    n = np.arange(F * Hh * Ww)
    f = n // (Hh * Ww)
    y = (n // Ww) % Hh
    x = n % Ww
    return frame0 + f, y, x


def angles(frame0: int, F: int, Hh: int, Ww: int, head_dim: int,
           theta: float = 10000.0) -> np.ndarray:
    """Rotation angle of every (token, pair): array [N_C, head_dim // 2]."""
    nt, nh, nw = axis_split(head_dim)
    t, y, x = token_positions(frame0, F, Hh, Ww)
    cols = []
    for pos, na in ((t, nt), (y, nh), (x, nw)):
        freq = theta ** (-np.arange(na, dtype=np.float64) / na)
        cols.append(pos[:, None].astype(np.float64) * freq[None, :])
    return np.concatenate(cols, axis=1)


def rope3d(x: np.ndarray, frame0: int, F: int, Hh: int, Ww: int,
           theta: float = 10000.0) -> np.ndarray:
    """Rotate x [N_C, H, d] (or [N_C, d]) at the chunk positions; fp64."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    a = angles(frame0, F, Hh, Ww, d, theta)          # [N_C, d/2]
    if x.ndim == 3:
        a = a[:, None, :]
    c, s = np.cos(a), np.sin(a)
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out
