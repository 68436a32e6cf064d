"""Inverse rotary position embedding followed by per-head FP8 quantisation
(oracle).

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.

The pages name one attention-side kernel next to the MoE layer, a fused
inverse rotary-embedding and per-head FP8 quantisation that had been
recompiled for every new token count until its variable-length arguments were
left unspecialised (toolboxkart.tech page, section 3 on JIT recompilation;
aib.vote page, fourth paragraph).  They give its name and that property only.
Readings, the plainest ones the name supports:

* Rotary embedding rotates pairs of a head's features by angles that grow with
  the token's position; the inverse rotates them back, by the negative angle.
  With c = cos(theta), s = sin(theta) for the pair (x1, x2):
      x1' = x1 * c + x2 * s
      x2' = x2 * c - x1 * s
* The pairs are (i, i + R/2) for i < R/2 ("half" layout, the default) or
  (2i, 2i + 1) ("interleaved"); R <= D is the number of rotated features of a
  head of D, the features from R on pass through unchanged.
* The angles come from a table the caller supplies, cos_sin[p] = (cos
  theta_p,0 .. cos theta_p,R/2-1, sin theta_p,0 .. sin theta_p,R/2-1) in
  float32, row p for position p.
* The rotation is done in float32, each product and each sum rounded on its
  own (no fused multiply-add), because the rotated value decides an integer
  FP8 code: both sides must decide in the same precision.
* Per-head quantisation: each (token, head) row of D rotated values gets its
  own scale amax / max of the format (1 when the row is zero) and the codes
  encode(v / scale), exactly the row quantiser of ``fp8.quantize_rows``.
"""

import numpy as np

from . import fp8 as _fp8


def pair_index(D, R, interleaved):
    """(first, second) feature indices of the R/2 rotated pairs of a head."""
    if R % 2 or not 0 < R <= D:
        raise ValueError("need an even rotary size 0 < R <= D")
    i = np.arange(R // 2)
    if interleaved:
        return 2 * i, 2 * i + 1
    return i, i + R // 2


def inv_rope(x, positions, cos_sin, R, interleaved=False):
    """[T, NH, D] float32 heads rotated back by their token's angles.

    x          [T, NH, D] float values (bfloat16 activations as float32)
    positions  [T] integer positions, rows of cos_sin
    cos_sin    [P, R] float32: cos of the R/2 angles, then their sin
    """
    x32 = np.asarray(x, dtype=np.float32)
    T, NH, D = x32.shape
    first, second = pair_index(D, R, interleaved)
    table = np.asarray(cos_sin, dtype=np.float32)
    rows = table[np.asarray(positions, dtype=np.int64)]          # [T, R]
    c = rows[:, None, :R // 2]                                    # [T, 1, R/2]
    s = rows[:, None, R // 2:]
    x1 = x32[:, :, first]
    x2 = x32[:, :, second]
    # float32 numpy arithmetic: every product and every sum rounds once
    y1 = (x1 * c) + (x2 * s)
    y2 = (x2 * c) - (x1 * s)
    out = x32.copy()
    out[:, :, first] = y1
    out[:, :, second] = y2
    return out


def inv_rope_fp8_quant_per_head(x, positions, cos_sin, R, interleaved=False, fmt="e4m3"):
    """(codes [T, NH, D] uint8, scales [T, NH] float32): the inverse rotary
    embedding of each head, then one FP8 scale per (token, head)."""
    y = inv_rope(x, positions, cos_sin, R, interleaved)
    T, NH, D = y.shape
    codes, scales = _fp8.quantize_rows(y.reshape(T * NH, D), fmt)
    return codes.reshape(T, NH, D), scales.reshape(T, NH)
