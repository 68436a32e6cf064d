"""ctypes binding of libmoemi.so (C ABI in include/moe.h).

Argument marshalling only: torch provides device memory and the current
stream; every step of the layer runs in the library's HIP kernels.  There is no
fallback: if the library is missing or fails to load, every call raises.
"""

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoemi.so")

MOE_BF16 = 0
MOE_FP8_E4M3 = 1
MOE_FP8_E5M2 = 2
_FP8_WDTYPE = {"e4m3": MOE_FP8_E4M3, "e5m2": MOE_FP8_E5M2}

MOE_SCALES_TENSOR = 0
MOE_SCALES_ROW = 1

STATUS = {0: "MOE_OK", 1: "MOE_ERR_NULL", 2: "MOE_ERR_SHAPE", 3: "MOE_ERR_UNSUPPORTED",
          4: "MOE_ERR_WORKSPACE", 5: "MOE_ERR_HIP"}


class MoEError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)}")


class FusedArgs(ctypes.Structure):
    _fields_ = [
        ("wdtype", ctypes.c_int),
        ("fp8_scales", ctypes.c_int),
        ("T", ctypes.c_int64),
        ("H", ctypes.c_int32),
        ("I", ctypes.c_int32),
        ("E", ctypes.c_int32),
        ("K", ctypes.c_int32),
        ("renormalize", ctypes.c_int32),
        ("x", ctypes.c_void_p),
        ("router_logits", ctypes.c_void_p),
        ("w13", ctypes.c_void_p),
        ("w2", ctypes.c_void_p),
        ("w13_scale", ctypes.c_void_p),
        ("w2_scale", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("topk_ids_out", ctypes.c_void_p),
        ("topk_weights_out", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
    ]


NO_SECTION = ctypes.c_size_t(-1).value


class FusedLayout(ctypes.Structure):
    """moe_fused_layout: byte offsets of a call's intermediate results inside
    its workspace (NO_SECTION where the call has no such result)."""
    _fields_ = [
        ("total", ctypes.c_size_t),
        ("block_m", ctypes.c_int32),
        ("tiled", ctypes.c_int32),
        ("tile_block_m", ctypes.c_int32),
        ("tile_threshold", ctypes.c_int32),
        ("capacity", ctypes.c_int64),
        ("tile_capacity", ctypes.c_int64),
        ("topk_ids", ctypes.c_size_t),
        ("topk_weights", ctypes.c_size_t),
        ("sorted_ids", ctypes.c_size_t),
        ("block_expert", ctypes.c_size_t),
        ("num_post_pad", ctypes.c_size_t),
        ("tile_sorted_ids", ctypes.c_size_t),
        ("tile_block_expert", ctypes.c_size_t),
        ("tile_num_post_pad", ctypes.c_size_t),
        ("x_amax", ctypes.c_size_t),
        ("x_codes", ctypes.c_size_t),
        ("x_scales", ctypes.c_size_t),
        ("a", ctypes.c_size_t),
        ("a_amax", ctypes.c_size_t),
        ("a_codes", ctypes.c_size_t),
        ("a_scales", ctypes.c_size_t),
    ]


_lib = None

_SIGS = {
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_route_topk": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                      ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p]),
    "moe_align_capacity": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_int32]),
    "moe_align_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int32,
                                                    ctypes.c_int32, ctypes.c_int32]),
    "moe_align": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                 ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                 ctypes.c_void_p]),
    "moe_act_quant_workspace_bytes": (ctypes.c_size_t, []),
    "moe_act_quant_fp8": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                         ctypes.c_void_p]),
    "moe_act_quant_fp8_rows": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                              ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_void_p]),
    "moe_fused_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(FusedArgs)]),
    "moe_fused_block_m": (ctypes.c_int32, [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_int32, ctypes.c_int]),
    "moe_fused_workspace_layout": (ctypes.c_int, [ctypes.POINTER(FusedArgs),
                                                  ctypes.POINTER(FusedLayout)]),
    "moe_fused_forward": (ctypes.c_int, [ctypes.POINTER(FusedArgs), ctypes.c_void_p]),
    "moe_fused_forward_timed": (ctypes.c_int, [ctypes.POINTER(FusedArgs), ctypes.c_void_p,
                                               ctypes.c_void_p]),
    "moe_fused_forward_noalloc": (ctypes.c_int, [ctypes.POINTER(FusedArgs), ctypes.c_void_p]),
    "moe_inv_rope_fp8_quant_per_head": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
        ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
}

# Stage boundaries of moe_fused_forward_timed (moe_stage in include/moe.h).
STAGES = ("route", "act_quant", "align", "gate_up", "inter_quant", "down", "combine")


def lib():
    """The loaded library; raises if it is not built (no fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m moe_layer_05_amd.build`; "
                "this package has no non-HIP fallback")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status, what):
    if status != 0:
        raise MoEError(status, what)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t, dtype, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


# ------------------------------------------------------------------ a1

def route_topk(logits, K, renormalize=True, stream=None):
    """(topk_ids [T, K] int32, topk_weights [T, K] float32) of [T, E] logits."""
    T, E = logits.shape
    lp = _dev(logits, torch.float32, "logits")
    ids = torch.empty(T, K, dtype=torch.int32, device=logits.device)
    w = torch.empty(T, K, dtype=torch.float32, device=logits.device)
    _check(lib().moe_route_topk(lp, T, E, K, int(bool(renormalize)), _ptr(ids), _ptr(w),
                                _stream(stream)), "moe_route_topk")
    return ids, w


# ------------------------------------------------------------------ a2

def align_capacity(T, K, E, block_m):
    return int(lib().moe_align_capacity(T, K, E, block_m))


def align(topk_ids, E, block_m, stream=None):
    """(sorted_ids, block_expert, num_post_pad [1] int32) of [T, K] ids.
    Only sorted_ids[:num_post_pad] and block_expert[:num_post_pad // block_m]
    are defined."""
    T, K = topk_ids.shape
    ip = _dev(topk_ids, torch.int32, "topk_ids")
    L = lib()
    cap = int(L.moe_align_capacity(T, K, E, block_m))
    if cap == 0 and T > 0:
        raise MoEError(3, "moe_align_capacity")
    dev = topk_ids.device
    sorted_ids = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    block_expert = torch.empty(max(cap // max(block_m, 1), 1), dtype=torch.int32, device=dev)
    npp = torch.zeros(1, dtype=torch.int32, device=dev)
    wsb = int(L.moe_align_workspace_bytes(T, K, E, block_m))
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    _check(L.moe_align(ip, T, K, E, block_m, _ptr(sorted_ids), _ptr(block_expert), _ptr(npp),
                       _ptr(ws), wsb, _stream(stream)), "moe_align")
    return sorted_ids, block_expert, npp


# ------------------------------------------------------------------ a0

def act_quant_fp8(x, stream=None):
    """(codes uint8 shaped like x, scale [1] float32) of bfloat16 x."""
    xp = _dev(x, torch.bfloat16, "x")
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    scale = torch.empty(1, dtype=torch.float32, device=x.device)
    L = lib()
    wsb = int(L.moe_act_quant_workspace_bytes())
    ws = torch.empty(wsb, dtype=torch.uint8, device=x.device)
    _check(L.moe_act_quant_fp8(xp, x.numel(), _ptr(codes), _ptr(scale), _ptr(ws), wsb,
                               _stream(stream)), "moe_act_quant_fp8")
    return codes, scale


def act_quant_fp8_rows(x, fmt="e4m3", stream=None):
    """(codes uint8 [R, C], scales [R] float32) of bfloat16 x [R, C], one
    scale per row; fmt "e4m3" or "e5m2"."""
    if x.dim() != 2:
        raise ValueError("x must be [rows, cols]")
    xp = _dev(x, torch.bfloat16, "x")
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    scales = torch.empty(x.shape[0], dtype=torch.float32, device=x.device)
    _check(lib().moe_act_quant_fp8_rows(xp, x.shape[0], x.shape[1], _FP8_WDTYPE[fmt],
                                        _ptr(codes), _ptr(scales), _stream(stream)),
           "moe_act_quant_fp8_rows")
    return codes, scales


# ------------------------------------------------------------------ attention side

def inv_rope_fp8_quant_per_head(x, positions, cos_sin, R, interleaved=False, fmt="e4m3",
                                codes=None, scales=None, stream=None):
    """(codes uint8 [T, NH, D], scales float32 [T, NH]): the inverse rotary
    embedding of bfloat16 heads x [T, NH, D] (token rows may be strided, the
    heads of a token contiguous) at int64 ``positions`` [T] with the float32
    table ``cos_sin`` [max_pos, R], then one FP8 scale per (token, head)."""
    if x.dim() != 3:
        raise ValueError("x must be [T, NH, D]")
    T, NH, D = x.shape
    if not x.is_cuda or x.dtype != torch.bfloat16:
        raise TypeError("x must be a bfloat16 CUDA (HIP) tensor")
    if x.stride(2) != 1 or x.stride(1) != D:
        raise ValueError("the heads of a token must be contiguous")
    pp = _dev(positions, torch.int64, "positions")
    cp = _dev(cos_sin, torch.float32, "cos_sin")
    if tuple(positions.shape) != (T,):
        raise ValueError(f"positions must be [{T}]")
    if cos_sin.dim() != 2 or cos_sin.shape[1] != R:
        raise ValueError(f"cos_sin must be [max_pos, {R}]")
    if codes is None:
        codes = torch.empty(T, NH, D, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(T, NH, dtype=torch.float32, device=x.device)
    _dev(codes, torch.uint8, "codes")
    _dev(scales, torch.float32, "scales")
    if tuple(codes.shape) != (T, NH, D) or tuple(scales.shape) != (T, NH):
        raise ValueError("codes must be [T, NH, D] and scales [T, NH]")
    stride = x.stride(0) if T > 1 else NH * D
    _check(lib().moe_inv_rope_fp8_quant_per_head(
        ctypes.c_void_p(x.data_ptr()), stride, pp, cp, cos_sin.shape[0], T, NH, D, R,
        int(bool(interleaved)), _FP8_WDTYPE[fmt], _ptr(codes), _ptr(scales), _stream(stream)),
        "moe_inv_rope_fp8_quant_per_head")
    return codes, scales


# ------------------------------------------------------------------ a0..a6

def fused_block_m(T, H, I, E, K, fp8):
    return int(lib().moe_fused_block_m(T, H, I, E, K, MOE_FP8_E4M3 if fp8 else MOE_BF16))


class WorkspacePool:
    """Workspaces of one layer, one per (device, stream) key, so calls
    enqueued on different streams never share scratch memory.  At most
    ``max_entries`` are kept: taking a workspace for a new key when the pool is
    full drops the least recently used one (a dropped buffer returns to
    torch's caching allocator, which reuses its memory only for work ordered
    after the calls already enqueued on that buffer's stream).  ``alloc(nbytes,
    key, ctx)`` makes a buffer with ``numel()`` bytes; ``ctx`` is passed through
    from ``get``."""

    def __init__(self, alloc, max_entries=4):
        if max_entries < 1:
            raise ValueError("max_entries must be >= 1")
        self.alloc = alloc
        self.max_entries = max_entries
        self._bufs = {}                              # key -> buffer, oldest use first

    def get(self, key, nbytes, ctx=None):
        buf = self._bufs.pop(key, None)
        if buf is None or buf.numel() < nbytes:
            buf = None                               # drop a too-small buffer first
            while len(self._bufs) >= self.max_entries:
                self._bufs.pop(next(iter(self._bufs)))
            buf = self.alloc(max(nbytes, 256), key, ctx)
        self._bufs[key] = buf                        # most recently used last
        return buf

    def release(self, key=None):
        """Drop the workspace of ``key``, or every workspace."""
        if key is None:
            self._bufs.clear()
        else:
            self._bufs.pop(key, None)

    def __len__(self):
        return len(self._bufs)

    def keys(self):
        return list(self._bufs)


class FusedMoE:
    """The fused layer forward bound to fixed weights.

    w13 [E, 2I, H] and w2 [E, H, I] are bfloat16, or uint8 E4M3 codes with
    w13_scale / w2_scale float32: [E] (one scale per expert tensor, and per
    tensor activation scales) or [E, 2I] / [E, H] (one per weight row, and
    per row activation scales); ``fp8_format`` says whether the codes are
    E4M3 or E5M2.  The workspace is a torch buffer grown on demand and reused
    across calls on the same stream (the library allocates nothing); calls on
    different streams get separate workspaces, so they may overlap.  At most
    ``max_workspaces`` are kept (least recently used dropped first);
    ``release_workspaces()`` drops them all."""

    def __init__(self, w13, w2, K, w13_scale=None, w2_scale=None, renormalize=True,
                 fp8_format="e4m3", max_workspaces=4):
        self.fp8 = w13.dtype == torch.uint8
        if fp8_format not in _FP8_WDTYPE:
            raise ValueError(f"fp8_format must be one of {sorted(_FP8_WDTYPE)}")
        self.wdtype = _FP8_WDTYPE[fp8_format] if self.fp8 else MOE_BF16
        self.E, twoI, self.H = w13.shape
        self.I = twoI // 2
        self.K = K
        self.renormalize = renormalize
        self.w13 = w13
        self.w2 = w2
        want = torch.uint8 if self.fp8 else torch.bfloat16
        _dev(w13, want, "w13")
        _dev(w2, want, "w2")
        if tuple(w2.shape) != (self.E, self.H, self.I):
            raise ValueError("w2 must be [E, H, I]")
        self.rows = False
        if self.fp8:
            _dev(w13_scale, torch.float32, "w13_scale")
            _dev(w2_scale, torch.float32, "w2_scale")
            self.rows = w13_scale.dim() == 2
            want13 = (self.E, 2 * self.I) if self.rows else (self.E,)
            want2 = (self.E, self.H) if self.rows else (self.E,)
            if tuple(w13_scale.shape) != want13 or tuple(w2_scale.shape) != want2:
                raise ValueError(f"scales must be {want13} and {want2}")
        self.w13_scale = w13_scale
        self.w2_scale = w2_scale
        self._ws = WorkspacePool(self._alloc_ws, max_workspaces)

    def args(self, x, logits, out, ids=None, wts=None):
        # the library trusts these shapes: a wrong width would be read out of bounds
        if x.dim() != 2 or x.shape[1] != self.H:
            raise ValueError(f"x must be [T, {self.H}], got {tuple(x.shape)}")
        T = x.shape[0]
        if tuple(logits.shape) != (T, self.E):
            raise ValueError(f"logits must be [{T}, {self.E}], got {tuple(logits.shape)}")
        if tuple(out.shape) != (T, self.H):
            raise ValueError(f"out must be [{T}, {self.H}], got {tuple(out.shape)}")
        for name, t, dt in (("topk_ids", ids, torch.int32), ("topk_weights", wts, torch.float32)):
            if t is not None:
                _dev(t, dt, name)
                if tuple(t.shape) != (T, self.K):
                    raise ValueError(f"{name} must be [{T}, {self.K}]")
        a = FusedArgs()
        a.wdtype = self.wdtype
        a.fp8_scales = MOE_SCALES_ROW if self.rows else MOE_SCALES_TENSOR
        a.T = x.shape[0]
        a.H, a.I, a.E, a.K = self.H, self.I, self.E, self.K
        a.renormalize = int(bool(self.renormalize))
        a.x = _dev(x, torch.bfloat16, "x").value
        a.router_logits = _dev(logits, torch.float32, "logits").value
        a.w13 = self.w13.data_ptr()
        a.w2 = self.w2.data_ptr()
        a.w13_scale = self.w13_scale.data_ptr() if self.fp8 else None
        a.w2_scale = self.w2_scale.data_ptr() if self.fp8 else None
        a.out = _dev(out, torch.bfloat16, "out").value
        a.topk_ids_out = ids.data_ptr() if ids is not None else None
        a.topk_weights_out = wts.data_ptr() if wts is not None else None
        return a

    def _shape_args(self, T):
        a = FusedArgs()
        a.wdtype = self.wdtype
        a.fp8_scales = MOE_SCALES_ROW if self.rows else MOE_SCALES_TENSOR
        a.T, a.H, a.I, a.E, a.K = T, self.H, self.I, self.E, self.K
        a.renormalize = int(bool(self.renormalize))
        return a

    def workspace_bytes(self, T):
        return int(lib().moe_fused_workspace_bytes(ctypes.byref(self._shape_args(T))))

    def workspace_layout(self, T):
        """FusedLayout of a call with T tokens (offsets into its workspace)."""
        out = FusedLayout()
        _check(lib().moe_fused_workspace_layout(ctypes.byref(self._shape_args(T)),
                                                ctypes.byref(out)),
               "moe_fused_workspace_layout")
        return out

    @staticmethod
    def _alloc_ws(nbytes, key, st):
        with torch.cuda.stream(st):
            return torch.empty(nbytes, dtype=torch.uint8, device=key[0])

    def workspace(self, T, device, stream=None):
        """The workspace for calls on ``stream`` (default: the current one),
        grown to T tokens if needed."""
        need = self.workspace_bytes(T)
        st = stream if stream is not None else torch.cuda.current_stream(device)
        return self._ws.get((str(device), st.cuda_stream), need, st)

    def release_workspaces(self):
        """Drop every workspace this layer holds (the next call allocates)."""
        self._ws.release()

    def __call__(self, x, logits, out=None, return_topk=False, stream=None, events=None):
        """out [T, H] bfloat16 of x [T, H] bfloat16 and logits [T, E] float32.

        ``events``: optional list of len(STAGES) + 1 entries, each a
        torch.cuda.Event created with enable_timing=True or None; the library
        records the events at the stage boundaries on the stream
        (moe_fused_forward_timed) and skips the None entries."""
        T = x.shape[0]
        if out is None:
            out = torch.empty(T, self.H, dtype=torch.bfloat16, device=x.device)
        ids = wts = None
        if return_topk:
            ids = torch.empty(T, self.K, dtype=torch.int32, device=x.device)
            wts = torch.empty(T, self.K, dtype=torch.float32, device=x.device)
        a = self.args(x, logits, out, ids, wts)
        ws = self.workspace(T, x.device, stream)
        a.workspace = ws.data_ptr()
        a.workspace_bytes = ws.numel()
        if events is None:
            _check(lib().moe_fused_forward(ctypes.byref(a), _stream(stream)), "moe_fused_forward")
        else:
            if len(events) != len(STAGES) + 1:
                raise ValueError(f"need {len(STAGES) + 1} events")
            st = stream if stream is not None else torch.cuda.current_stream()
            for ev in events:
                if ev is not None and ev.cuda_event == 0:
                    ev.record(st)           # torch creates the event on its first record
            arr = (ctypes.c_void_p * len(events))(
                *[ev.cuda_event if ev is not None else None for ev in events])
            _check(lib().moe_fused_forward_timed(ctypes.byref(a), _stream(stream), arr),
                   "moe_fused_forward_timed")
        return (out, ids, wts) if return_topk else out


NOALLOC_SCRATCH_BYTES = 64 << 20           # MOE_NOALLOC_SCRATCH_BYTES


def fused_forward_noalloc(layer, x, logits, out, ids=None, wts=None, stream=None):
    """moe_fused_forward_noalloc: the layer ``layer`` (a FusedMoE) on x and
    logits into the caller's ``out`` (and optional ids / wts), with the
    library's own scratch buffer as workspace; nothing is allocated."""
    a = layer.args(x, logits, out, ids, wts)
    _check(lib().moe_fused_forward_noalloc(ctypes.byref(a), _stream(stream)),
           "moe_fused_forward_noalloc")
    return out


def fused_forward(x, logits, w13, w2, K, w13_scale=None, w2_scale=None, renormalize=True,
                  return_topk=False, stream=None, fp8_format="e4m3"):
    """One-shot fused forward (allocates its workspace through torch)."""
    m = FusedMoE(w13, w2, K, w13_scale, w2_scale, renormalize, fp8_format)
    return m(x, logits, return_topk=return_topk, stream=stream)
