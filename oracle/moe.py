"""Fused Mixture-of-Experts layer forward, written as its plain definition.

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.

What the layer computes (the pages describe it in words only):

* A router picks, per token, a few experts out of E; only those experts run
  for that token (toolboxkart.tech page, "Why MoE inference needs specialized
  kernels"; kongchang.com page, "Why MoE Inference Is So Sensitive to Kernel
  Engineering": routing is dynamic and the number of tokens per expert varies).
* Tokens are grouped by expert so that each expert runs one grouped matrix
  product over its tokens (kongchang.com page, "Swap-AB": grouped and batched
  GEMMs are abundant in MoE; aib.vote page, second paragraph: top-k=8 joins the
  selected experts' intermediate dimensions).
* Each expert is a gated feed-forward network; the layer output is the
  routing-weighted sum of the chosen experts' outputs, and the fused kernel
  does scaling, the products and this aggregation in one pass without
  changing the math (aib.vote page, third paragraph).

Readings where the pages are silent (each listed with its reason in the
design notes of the repository):

* score = softmax over all E logits (float64 here); the top-K set and its
  order are decided on the raw float32 logits: larger first, equal logits ->
  lower expert id first (+0.0 and -0.0 are equal);
* renormalised weights w_k = p_{S[k]} / sum_j p_{S[j]};
* w13[e] is [2I, H]: rows [0, I) are the gate projection W1, rows [I, 2I) the
  up projection W3; w2[e] is [H, I];
* expert(x) = W2 (silu(W1 x) * (W3 x)), silu(z) = z / (1 + exp(-z));
* the routing weight multiplies the expert output after the down projection;
* FP8 mode: x is quantised per tensor (one scale for the call), weights are
  code * per-expert-tensor scale, and the intermediate a is quantised per
  tensor over all routed pairs, from its float32 value;
* output = bfloat16(round-to-nearest-even(float32(y))).
"""

from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import fp8 as _fp8


def _map(fn, items, workers):
    """map() over experts, optionally on a thread pool (numpy's table lookups
    and BLAS release the GIL).  Each expert is computed exactly as in the
    serial loop; only the wall time changes."""
    if workers and workers > 1:
        with ThreadPoolExecutor(workers) as ex:
            return list(ex.map(fn, items))
    return [fn(i) for i in items]


# --------------------------------------------------------------------------
# a1: routing
# --------------------------------------------------------------------------

def route(logits, K, renormalize=True):
    """Top-K expert ids and routing weights per token.

    logits: [T, E] float32.  Returns (ids [T, K] int32, weights [T, K] float64).

    The order is: larger logit first; equal logits -> lower expert id first.
    Comparing the float32 logits themselves (softmax is strictly increasing)
    makes the chosen set independent of how exp is rounded.
    """
    lg = np.asarray(logits, dtype=np.float32)
    T, E = lg.shape
    if not 1 <= K <= E:
        raise ValueError("need 1 <= K <= E")
    ids = np.empty((T, K), dtype=np.int32)
    w = np.empty((T, K), dtype=np.float64)
    expert = np.arange(E)
    for t in range(T):
        row = lg[t].astype(np.float64)
        # lexsort: last key is primary.  -row puts larger logits first; on
        # equal logits the expert id (ascending) decides.  -0.0 == +0.0.
        order = np.lexsort((expert, -row))
        sel = order[:K]
        ids[t] = sel
        p = np.exp(row - row.max())
        p = p / p.sum()                      # softmax over all E experts
        ws = p[sel]
        if renormalize:
            ws = ws / ws.sum()
        w[t] = ws
    return ids, w


# --------------------------------------------------------------------------
# a2: align (sort token-expert pairs by expert, pad to the block size)
# --------------------------------------------------------------------------

def align(ids, E, block_m):
    """Stable counting sort of the pairs by expert, each run padded to block_m.

    Pair i = t*K + k stands for (token t, slot k).  Experts are laid out in
    ascending id; inside an expert, pairs keep ascending i; each expert's run is
    padded with the sentinel T*K up to a multiple of block_m; experts with no
    pair take no block.

    Returns (sorted_ids int32 [num_post_pad], block_expert int32
    [num_post_pad / block_m], num_post_pad int).
    """
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    P = flat.size
    sentinel = P
    sorted_ids = []
    block_expert = []
    for e in range(E):
        members = np.nonzero(flat == e)[0]          # ascending pair ids
        if members.size == 0:
            continue
        nblk = -(-members.size // block_m)
        pad = nblk * block_m - members.size
        sorted_ids.extend(members.tolist())
        sorted_ids.extend([sentinel] * pad)
        block_expert.extend([e] * nblk)
    return (np.asarray(sorted_ids, dtype=np.int32),
            np.asarray(block_expert, dtype=np.int32),
            len(sorted_ids))


# --------------------------------------------------------------------------
# a0: activation quantisation (FP8 mode)
# --------------------------------------------------------------------------

def act_quant(x, scales="tensor", fmt="e4m3"):
    """FP8 quantisation of the activations: (codes uint8, scale).

    scales == "tensor": one scale for the whole [T, H] tensor (float32).
    scales == "row":    one scale per token row, [T] float32.
    fmt: "e4m3" or "e5m2".
    """
    x32 = np.asarray(x, dtype=np.float32)
    if scales == "row":
        return _fp8.quantize_rows(x32, fmt)
    return _fp8.quantize(x32, fmt=fmt)


def _dequant(codes, scale, scales, fmt="e4m3"):
    """codes times the tensor scale, or times each row's scale."""
    if scales == "row":
        return _fp8.decode(codes, fmt) * np.asarray(scale, dtype=np.float64)[:, None]
    return _fp8.decode(codes, fmt) * np.float64(scale)


# --------------------------------------------------------------------------
# a3..a6: the layer
# --------------------------------------------------------------------------

def silu(z):
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def _weight(wt, e, scale, fp8_mode, dtype, fmt="e4m3"):
    """Expert weight matrix in ``dtype``: code * scale (FP8) or the value.

    ``scale[e]`` is the expert tensor's scale, or an array with one scale per
    output row (per-channel scales: [2I] for w13, [H] for w2)."""
    m = np.asarray(wt[e])
    if fp8_mode:
        se = np.asarray(scale[e], dtype=np.float64)
        if se.ndim == 1:
            return (_fp8.decode(m, fmt) * se[:, None]).astype(dtype)
        return (_fp8.decode(m, fmt) * np.float64(se)).astype(dtype)
    return m.astype(dtype)


def _gate_up(xh, W13, I):
    """a = silu(x W1^T) * (x W3^T) for rows of xh; W13 = [W1; W3]."""
    g = xh @ W13[:I].T
    u = xh @ W13[I:].T
    return silu(g) * u


def moe_forward(x, logits, w13, w2, K, wdtype="float", w13_scale=None,
                w2_scale=None, renormalize=True, dtype=np.float64,
                tokens=None, return_parts=False, workers=1, act_scales="tensor",
                fp8_format="e4m3"):
    """The layer output for the tokens in ``tokens`` (all by default).

    x       [T, H] float values (the bfloat16 activations as float32).
    logits  [T, E] float32.
    w13     indexable by expert -> [2I, H]; float values, or uint8 E4M3 codes
            when wdtype == "fp8".
    w2      indexable by expert -> [H, I]; same convention.
    w13_scale, w2_scale  [E] float32 per-expert-tensor scales (FP8 only), or
            per-channel scales [E, 2I] / [E, H] (one per output row).
    act_scales  "tensor": one scale for x and one for the intermediate a over
            all routed pairs; "row": one per token row of x and one per pair
            row of a (FP8 only).
    fp8_format  "e4m3" or "e5m2": the code format of the weights, x and a
            (FP8 only).
    dtype   arithmetic precision of the products (float64 by default).
    workers experts evaluated concurrently (same arithmetic, less wall time).

    Returns out [len(tokens), H] float32 holding bfloat16 values; with
    ``return_parts`` also a dict with y (before rounding), ids, weights, the
    intermediate rows a (in ``dtype``, one row per (t, k) in a_pairs) and, in
    FP8 mode, the activation scales and the float32 rows that were quantised
    (a_f32).

    In FP8 mode the intermediate scale needs every routed pair, so gate/up runs
    for all pairs; the down projection and the combine run for ``tokens`` only.
    """
    fp8_mode = (wdtype == "fp8")
    x32 = np.asarray(x, dtype=np.float32)
    T, H = x32.shape
    ids, wts = route(logits, K, renormalize)
    if tokens is None:
        tokens = np.arange(T)
    tokens = np.asarray(tokens, dtype=np.int64)
    parts = {"ids": ids, "weights": wts}

    fmt = fp8_format
    if fp8_mode:
        qx, s_x = act_quant(x32, act_scales, fmt)
        xh = _dequant(qx, s_x, act_scales, fmt).astype(dtype)
        parts["s_x"] = s_x
    else:
        xh = x32.astype(dtype)

    # a per-tensor intermediate scale needs every routed pair; per-pair
    # scales do not
    need_all = fp8_mode and act_scales == "tensor"
    want = np.zeros(T, dtype=bool)
    want[tokens] = True

    # gate/up + SiLU-and-mul per expert over its routed pairs
    experts = np.unique(ids)

    def gate_up_of(e):
        tk = np.argwhere(ids == e)           # rows (t, k), ascending t
        if not need_all:
            tk = tk[want[tk[:, 0]]]
        if tk.size == 0:
            return tk, None
        W13 = _weight(w13, e, w13_scale, fp8_mode, dtype, fmt)
        I = W13.shape[0] // 2
        return tk, _gate_up(xh[tk[:, 0]], W13, I)

    a = {}                                   # (t, k) -> intermediate row
    for tk, ae in _map(gate_up_of, experts, workers):
        for r, (t, k) in enumerate(tk):
            a[(int(t), int(k))] = ae[r]

    if a:
        keys = sorted(a)
        parts["a_pairs"] = keys              # (t, k) of each row of a / a_f32 / s_a
        parts["a"] = np.stack([a[kk] for kk in keys])   # before any quantisation
    if fp8_mode and a:
        amat = parts["a"].astype(np.float32)
        qa, s_a = act_quant(amat, act_scales, fmt)
        ah = _dequant(qa, s_a, act_scales, fmt)
        for r, kk in enumerate(keys):
            a[kk] = ah[r].astype(dtype)
        parts["s_a"] = s_a
        parts["a_f32"] = amat                # the values that were quantised

    # down projection and routing-weighted combine
    def down_of(e):
        tk = [(int(t), int(k)) for t, k in np.argwhere(ids == e)
              if want[int(t)]]
        if not tk:
            return tk, None
        W2 = _weight(w2, e, w2_scale, fp8_mode, dtype, fmt)
        A = np.stack([a[p] for p in tk]).astype(dtype)
        return tk, A @ W2.T

    y = np.zeros((tokens.size, H), dtype=np.float64)
    row_of = {int(t): r for r, t in enumerate(tokens)}
    for tk, d in _map(down_of, experts, workers):   # experts in ascending id
        for r, (t, k) in enumerate(tk):
            y[row_of[t]] += wts[t, k] * d[r]

    out = _fp8.bf16_round(y.astype(np.float32))
    if return_parts:
        parts["y"] = y
        return out, parts
    return out


def moe_dense(x, logits, w13, w2, K, wdtype="float", w13_scale=None,
              w2_scale=None, renormalize=True, dtype=np.float64, act_scales="tensor",
              fp8_format="e4m3"):
    """The same layer written as "run every expert on every token, mask".

    y_t = sum_e M[t, e] * expert_e(x_t), with M[t, e] the routing weight of e
    for t (0 when e is not among t's top-K).  In FP8 mode the intermediate
    scale is taken over the routed (t, e) entries only, as the layer defines
    it.  Returns y (float64, before the bfloat16 rounding).
    """
    fp8_mode = (wdtype == "fp8")
    x32 = np.asarray(x, dtype=np.float32)
    T, H = x32.shape
    E = np.asarray(logits).shape[1]
    ids, wts = route(logits, K, renormalize)
    M = np.zeros((T, E))
    routed = np.zeros((T, E), dtype=bool)
    for t in range(T):
        for k in range(K):
            M[t, ids[t, k]] = wts[t, k]
            routed[t, ids[t, k]] = True
    fmt = fp8_format
    if fp8_mode:
        qx, s_x = act_quant(x32, act_scales, fmt)
        xh = _dequant(qx, s_x, act_scales, fmt).astype(dtype)
    else:
        xh = x32.astype(dtype)
    A = []
    for e in range(E):
        W13 = _weight(w13, e, w13_scale, fp8_mode, dtype, fmt)
        I = W13.shape[0] // 2
        A.append(_gate_up(xh, W13, I))       # [T, I] for every token
    A = np.stack(A, axis=1)                  # [T, E, I]
    if fp8_mode and act_scales == "row":
        # every (token, expert) row on its own scale; unrouted rows are masked
        flat = A.reshape(T * E, -1).astype(np.float32)
        q, s_rows = _fp8.quantize_rows(flat, fmt)
        A = (_fp8.decode(q, fmt) * s_rows.astype(np.float64)[:, None]).reshape(A.shape)
    elif fp8_mode:
        amax_src = A[routed].astype(np.float32)
        s_a = _fp8.per_tensor_scale(amax_src, fmt)
        q, _ = _fp8.quantize(A.astype(np.float32), scale=s_a, fmt=fmt)
        A = _fp8.decode(q, fmt) * np.float64(s_a)
    y = np.zeros((T, H))
    for e in range(E):
        W2 = _weight(w2, e, w2_scale, fp8_mode, dtype, fmt)
        y += M[:, e:e + 1] * (A[:, e, :].astype(dtype) @ W2.T)
    return y
