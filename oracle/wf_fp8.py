"""FP8 (E4M3) K/V pages: the quantisation reading, fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

WF ("Wave Forcing: Towards Speed-of-Light Streaming Video Generation")
App. C.6, Eq. 20-21 and Tab. 8: K/V may travel in FP8, which halves the
payload (metadata excluded) at the cost of a conversion.  The page fixes
neither the FP8 format nor the scale granularity.  Readings taken here:

* Format: OCP E4M3 -- 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits,
  subnormals below 2^-6, largest finite value 448, no infinities, NaN codes
  0x7F / 0xFF.  Conversion rounds to nearest, ties to even, and keeps the
  sign of a value that rounds to zero (-0 is 0x80).
* Scales are powers of two.  A block with largest magnitude ``amax`` uses the
  smallest integer exponent e with amax <= 448 * 2^e (e = 0 for an all-zero
  block), and stores x / 2^e.
* Blocks: every 64-token tile of one head of a page, separately for the
  rotated key (after RoPE) and for the value; pages hold ceil(N / 64) * 64
  tokens, the padding tokens are zero and never attended.
* Queries: App. C.6 speaks of the K/V payload only and says nothing of the
  query.  The plainest reading that keeps q_rot's bf16 layout is to quantise
  each bf16 rotated query row (one token of one head) on its own, by the same
  block rule with one exponent per row (``fp8_query``).
* Attention over FP8 pages is the plain softmax attention of
  ``wf_attention.attend`` applied to the dequantised Q, K and V.

Parity status: pinned by ``tests/test_oracle_fp8.py`` (every code against
torch's float8_e4m3fn, closed-form exponents, rounding ties, scale
invariance).
"""

import math

import numpy as np

E4M3_MAX = 448.0
TILE = 64


def e4m3_decode(code: int) -> float:
    """Value of an E4M3 code (0..255); NaN for 0x7F / 0xFF."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return math.nan
    if exp == 0:
        return sign * math.ldexp(man / 8.0, -6)
    return sign * math.ldexp(1.0 + man / 8.0, exp - 7)


def _positive_values() -> np.ndarray:
    """The 127 non-negative finite E4M3 values, indexed by code 0..126."""
    return np.array([e4m3_decode(c) for c in range(127)], dtype=np.float64)


_POS = _positive_values()


def e4m3_encode(x) -> np.ndarray:
    """Round-to-nearest-even E4M3 codes of ``x`` (|x| <= 448 required)."""
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    if np.any(ax > E4M3_MAX) or np.any(np.isnan(x)):
        raise ValueError("e4m3_encode: value outside the finite range")
    # nearest representable magnitude; on a tie the even code wins
    hi = np.searchsorted(_POS, ax, side="left")          # first value >= ax
    hi = np.clip(hi, 0, len(_POS) - 1)
    lo = np.clip(hi - 1, 0, len(_POS) - 1)
    d_lo = ax - _POS[lo]
    d_hi = _POS[hi] - ax
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.int64)
    code = np.where(ax == _POS[hi], hi, code)
    # the sign survives rounding to zero (a negative value gives -0, 0x80)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def e4m3_values(codes) -> np.ndarray:
    """Decode an array of codes."""
    table = np.array([e4m3_decode(c) for c in range(256)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.int64)]


def pow2_exponent(amax: float) -> int:
    """Smallest integer e with amax <= 448 * 2^e (0 for amax == 0)."""
    amax = float(amax)
    if amax == 0.0:
        return 0
    e = math.ceil(math.log2(amax / E4M3_MAX))
    while amax > math.ldexp(E4M3_MAX, e):
        e += 1
    while amax <= math.ldexp(E4M3_MAX, e - 1):
        e -= 1
    return e


def quantize_block(x: np.ndarray):
    """One block: (codes, exponent) with codes = E4M3(x / 2^e)."""
    x = np.asarray(x, dtype=np.float64)
    e = pow2_exponent(np.max(np.abs(x)) if x.size else 0.0)
    return e4m3_encode(np.ldexp(x, -e)), e


def quantize_tiles(x: np.ndarray, tile: int = TILE):
    """Per-tile quantisation of one head's tokens: x [N, d] -> (codes
    [Np, d] with Np = ceil(N / tile) * tile and zero padding, exponents [Np / tile])."""
    x = np.asarray(x, dtype=np.float64)
    n, d = x.shape
    n_t = -(-n // tile)
    codes = np.zeros((n_t * tile, d), dtype=np.uint8)
    exps = np.zeros(n_t, dtype=np.int64)
    for t in range(n_t):
        blk = x[t * tile:min(n, (t + 1) * tile)]
        c, e = quantize_block(blk)
        codes[t * tile:t * tile + blk.shape[0]] = c
        exps[t] = e
    return codes, exps


def dequantize_tiles(codes: np.ndarray, exps: np.ndarray, n: int, tile: int = TILE) -> np.ndarray:
    """Inverse of ``quantize_tiles`` restricted to the first n tokens."""
    vals = e4m3_values(codes)
    scale = np.repeat(np.ldexp(1.0, np.asarray(exps, dtype=np.int64)), tile)[:vals.shape[0]]
    return (vals * scale[:, None])[:n]


def fp8_tiles(x: np.ndarray, tile: int = TILE) -> np.ndarray:
    """x [N, d] as the attention sees it after tile quantisation (fp64)."""
    codes, exps = quantize_tiles(x, tile)
    return dequantize_tiles(codes, exps, x.shape[0], tile)


def fp8_rows(x: np.ndarray) -> np.ndarray:
    """x [N, d] quantised per row (the query reading), dequantised (fp64)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    for r in range(x.shape[0]):
        c, e = quantize_block(x[r])
        out[r] = np.ldexp(e4m3_values(c), e)
    return out


def fp8_query(q_bf16: np.ndarray) -> np.ndarray:
    """The query reading: each row of q (bf16 values, [N, d]) quantised on
    its own by the block rule (one power-of-two exponent per row), then
    dequantised (fp64)."""
    return fp8_rows(q_bf16)


def bf16_round(x) -> np.ndarray:
    """Round to the nearest bfloat16 (8 significant bits), ties to even, as
    fp64 (the rotated query is stored in bf16 before it is quantised)."""
    x = np.asarray(x, dtype=np.float64)
    f32 = x.astype(np.float32)
    # fp64 -> fp32 can itself round; redo the rounding from fp64 exactly
    m, e = np.frexp(x)                       # x = m 2^e, 0.5 <= |m| < 1
    scaled = np.ldexp(m, 8)                  # 8 significant bits
    r = np.round(scaled)                     # numpy rounds half to even
    out = np.ldexp(r, e - 8)
    return np.where(np.isfinite(x), out, f32.astype(np.float64))
