"""The C ABI on the CPU: the library loads, exports every function that
include/moe.h declares, and its host-side checks reject bad arguments before
any HIP call (so they run without a GPU).  No compute call is made here."""

import ctypes
import os
import re
import shutil
import subprocess

import pytest

from moe_layer_05_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

OK, NULL, SHAPE, UNSUP, WS = 0, 1, 2, 3, 4


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("libmoemi.so is not built (run __graft_entry__.build())")
    return binding.lib()


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", src)))


def test_header_functions_exported(L):
    names = _declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    # the binding declares a signature for each of them
    assert set(names) == set(binding._SIGS)


def test_struct_layout_matches_c():
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    prog = r'''
#include <stdio.h>
#include <stddef.h>
#include "moe.h"
int main(void) {
  printf("%zu", sizeof(moe_fused_args));
#define F(n) printf(" %zu", offsetof(moe_fused_args, n));
  F(wdtype) F(fp8_scales) F(T) F(H) F(I) F(E) F(K) F(renormalize) F(x) F(router_logits) F(w13) F(w2)
  F(w13_scale) F(w2_scale) F(out) F(topk_ids_out) F(topk_weights_out) F(workspace)
  F(workspace_bytes)
  return 0;
}
'''
    import tempfile
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "l.c")
        open(c, "w").write(prog)
        exe = os.path.join(d, "l")
        r = subprocess.run([gcc, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                            f"-I{os.path.join(ROOT, 'include')}", c, "-o", exe],
                           capture_output=True, text=True)
        if r.returncode:
            pytest.skip("cannot compile against hip_runtime_api.h: " + r.stderr[:200])
        vals = [int(v) for v in subprocess.check_output([exe], text=True).split()]
    F = binding.FusedArgs
    want = [ctypes.sizeof(F)] + [getattr(F, n).offset for n, _ in F._fields_]
    assert vals == want


def test_layout_struct_matches_c():
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    F = binding.FusedLayout
    names = [n for n, _ in F._fields_]
    prog = ('#include <stdio.h>\n#include <stddef.h>\n#include "moe.h"\n'
            'int main(void) {\n  printf("%zu %zu", sizeof(moe_fused_layout), (size_t)MOE_NO_SECTION);\n'
            + "".join(f'  printf(" %zu", offsetof(moe_fused_layout, {n}));\n' for n in names)
            + "  return 0;\n}\n")
    import tempfile
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "l.c")
        open(c, "w").write(prog)
        exe = os.path.join(d, "l")
        r = subprocess.run([gcc, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                            f"-I{os.path.join(ROOT, 'include')}", c, "-o", exe],
                           capture_output=True, text=True)
        if r.returncode:
            pytest.skip("cannot compile against hip_runtime_api.h: " + r.stderr[:200])
        vals = [int(v) for v in subprocess.check_output([exe], text=True).split()]
    want = [ctypes.sizeof(F), binding.NO_SECTION] + [getattr(F, n).offset for n in names]
    assert vals == want


def test_status_strings(L):
    for s in range(6):
        assert L.moe_status_string(s).decode().startswith(binding.STATUS[s])


def test_route_topk_validation(L):
    p = ctypes.c_void_p(16)
    assert L.moe_route_topk(p, 4, 8, 9, 1, p, p, None) == SHAPE      # K > E
    assert L.moe_route_topk(p, -1, 8, 2, 1, p, p, None) == SHAPE
    assert L.moe_route_topk(p, 4, 2048, 2, 1, p, p, None) == UNSUP   # E > 1024
    assert L.moe_route_topk(p, 4, 128, 65, 1, p, p, None) == UNSUP  # K > 64
    assert L.moe_route_topk(None, 4, 8, 2, 1, p, p, None) == NULL
    assert L.moe_route_topk(None, 0, 8, 2, 1, None, None, None) == OK  # T = 0


def test_align_capacity_and_validation(L):
    for T, K, E, bm in [(64, 8, 256, 64), (1, 8, 256, 16), (4096, 8, 256, 128), (3, 2, 8, 16)]:
        P = T * K
        assert L.moe_align_capacity(T, K, E, bm) == (P // bm + min(E, P)) * bm
    assert L.moe_align_capacity(4, 2, 8, 48) == 0
    p = ctypes.c_void_p(256)
    big = 1 << 30
    assert L.moe_align(p, 4, 2, 8, 48, p, p, p, p, big, None) == UNSUP
    assert L.moe_align(p, 4, 3, 2, 16, p, p, p, p, big, None) == SHAPE
    assert L.moe_align(p, 4, 2, 8, 16, p, p, None, p, big, None) == NULL
    assert L.moe_align(p, 4, 2, 8, 16, p, p, p, p, 0, None) == WS
    assert L.moe_align(None, 0, 2, 8, 16, None, None, p, None, 0, None) == OK


def test_act_quant_validation(L):
    p = ctypes.c_void_p(256)
    assert L.moe_act_quant_workspace_bytes() >= 4
    assert L.moe_act_quant_fp8(p, 12, p, p, p, 256, None) == UNSUP            # n % 8
    assert L.moe_act_quant_fp8(ctypes.c_void_p(258), 16, p, p, p, 256, None) == UNSUP
    assert L.moe_act_quant_fp8(p, 16, p, None, p, 256, None) == NULL
    assert L.moe_act_quant_fp8(p, 16, p, p, p, 1, None) == WS
    assert L.moe_act_quant_fp8(p, -8, p, p, p, 256, None) == SHAPE


def test_act_quant_rows_validation(L):
    p = ctypes.c_void_p(256)
    E4, E5 = binding.MOE_FP8_E4M3, binding.MOE_FP8_E5M2
    assert L.moe_act_quant_fp8_rows(p, 4, 12, E4, p, p, None) == UNSUP         # cols % 8
    assert L.moe_act_quant_fp8_rows(ctypes.c_void_p(258), 4, 16, E5, p, p, None) == UNSUP
    assert L.moe_act_quant_fp8_rows(p, 4, 16, binding.MOE_BF16, p, p, None) == UNSUP
    assert L.moe_act_quant_fp8_rows(p, 4, 16, 9, p, p, None) == UNSUP          # no such format
    assert L.moe_act_quant_fp8_rows(p, 4, 16, E4, p, None, None) == NULL
    assert L.moe_act_quant_fp8_rows(p, -1, 16, E4, p, p, None) == SHAPE
    assert L.moe_act_quant_fp8_rows(None, 0, 16, E5, None, None, None) == OK  # no rows


def _args(**kw):
    a = binding.FusedArgs()
    a.wdtype, a.T, a.H, a.I, a.E, a.K, a.renormalize = 1, 8, 256, 64, 16, 4, 1
    for f in ("x", "router_logits", "w13", "w2", "w13_scale", "w2_scale", "out", "workspace"):
        setattr(a, f, 4096)
    a.workspace_bytes = 1 << 40
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _fwd(L, **kw):
    a = _args(**kw)
    return L.moe_fused_forward(ctypes.byref(a), None)


def test_fused_validation(L):
    assert L.moe_fused_forward(None, None) == NULL
    assert _fwd(L, K=17) == SHAPE
    assert _fwd(L, T=-1) == SHAPE
    assert _fwd(L, H=0) == SHAPE
    assert _fwd(L, H=264) == UNSUP          # H % 16
    assert _fwd(L, I=40) == UNSUP           # I % 16
    assert _fwd(L, E=2048, K=4) == UNSUP
    assert _fwd(L, wdtype=7) == UNSUP
    assert _fwd(L, wdtype=2, workspace_bytes=16) == WS        # E5M2 is a weight type
    assert _fwd(L, wdtype=2, w2_scale=None) == NULL           # and needs scales
    assert _fwd(L, x=None) == NULL
    assert _fwd(L, w13_scale=None) == NULL          # fp8 needs scales
    assert _fwd(L, out=4097) == UNSUP               # misaligned
    assert _fwd(L, workspace_bytes=16) == WS
    assert _fwd(L, fp8_scales=2) == UNSUP           # unknown scale mode
    assert _fwd(L, fp8_scales=1, w2_scale=4100) == UNSUP   # row scales: 16-byte aligned
    assert _fwd(L, wdtype=0, fp8_scales=9, w13_scale=None, w2_scale=None,
                workspace_bytes=16) == WS           # bf16 ignores the scale mode
    assert _fwd(L, T=0, x=None, out=None) == OK     # empty batch: no-op


def test_fused_block_m_and_workspace(L):
    # a block holds one expert's tokens; its size follows the expected tokens
    # per expert (T*K/E), so an expert's weights stream once per call
    bm = [L.moe_fused_block_m(T, 7168, 2048, 256, 8, 1) for T in (1, 8, 16, 17, 32, 64, 4096)]
    assert all(b in (16, 32, 64, 128, 256) for b in bm)
    assert bm[:3] == [16, 16, 16]                    # T <= 16: one 16-token block
    assert bm[5] == 16                               # 2 tokens per expert on average
    assert L.moe_fused_block_m(32, 4096, 14336, 8, 2, 0) == 16     # 8 per expert
    assert L.moe_fused_block_m(64, 4096, 14336, 8, 2, 0) == 32     # 16 per expert
    assert L.moe_fused_block_m(256, 4096, 192, 128, 8, 1) == 32    # 16 per expert
    assert L.moe_fused_block_m(4096, 7168, 2048, 256, 8, 1) == 64  # 128 per expert
    a = _args()
    n1 = L.moe_fused_workspace_bytes(ctypes.byref(a))
    assert n1 > 8 * 4 * (256 * 4)                    # at least the pair outputs
    a.T = 16
    assert L.moe_fused_workspace_bytes(ctypes.byref(a)) > n1
    a.fp8_scales = 1                                 # per-row scales of x and a
    assert L.moe_fused_workspace_bytes(ctypes.byref(a)) >= \
        L.moe_fused_workspace_bytes(ctypes.byref(_args(T=16))) + (16 + 16 * 4) * 4
    a.fp8_scales = 5
    assert L.moe_fused_workspace_bytes(ctypes.byref(a)) == 0
    a.fp8_scales = 0
    a.K = 99
    assert L.moe_fused_workspace_bytes(ctypes.byref(a)) == 0


def _layout(L, **kw):
    a = _args(**kw)
    out = binding.FusedLayout()
    st = L.moe_fused_workspace_layout(ctypes.byref(a), ctypes.byref(out))
    return st, out


def _sections(lay):
    return {n: getattr(lay, n) for n in ("topk_ids", "topk_weights", "sorted_ids",
                                         "block_expert", "num_post_pad", "tile_sorted_ids",
                                         "tile_block_expert", "tile_num_post_pad", "x_amax",
                                         "x_codes", "x_scales", "a", "a_amax", "a_codes",
                                         "a_scales")}


def test_workspace_layout_query(L):
    """The layout query agrees with the size query and with the block size,
    marks the sections a call does not have, and its sections lie inside the
    workspace without overlapping (sizes from the documented shapes)."""
    NO = binding.NO_SECTION
    assert L.moe_fused_workspace_layout(None, None) == NULL
    assert _layout(L, K=17)[0] == SHAPE
    for kw in (dict(), dict(fp8_scales=1), dict(wdtype=0), dict(wdtype=2),
               dict(T=4096, H=7168, I=2048, E=256, K=8),
               dict(T=4096, H=7168, I=2048, E=256, K=8, wdtype=0),
               dict(T=1, H=4096, I=14336, E=8, K=2, wdtype=0)):
        st, lay = _layout(L, **kw)
        assert st == OK, kw
        a = _args(**kw)
        assert lay.total == L.moe_fused_workspace_bytes(ctypes.byref(a))
        assert lay.block_m == L.moe_fused_block_m(a.T, a.H, a.I, a.E, a.K, a.wdtype) or lay.tiled
        fp8 = a.wdtype != 0
        rows = fp8 and a.fp8_scales == 1
        sec = _sections(lay)
        assert (sec["x_codes"] != NO) == fp8 and (sec["a_codes"] != NO) == fp8
        assert (sec["x_amax"] != NO) == (fp8 and not rows)
        assert (sec["a_amax"] != NO) == (fp8 and not rows)
        assert (sec["x_scales"] != NO) == rows and (sec["a_scales"] != NO) == rows
        assert (sec["tile_sorted_ids"] != NO) == bool(lay.tiled)
        P = a.T * a.K
        size = {"topk_ids": 4 * P, "topk_weights": 4 * P, "sorted_ids": 4 * lay.capacity,
                "block_expert": 4 * lay.capacity // lay.block_m, "num_post_pad": 4,
                "tile_sorted_ids": 4 * lay.tile_capacity,
                "tile_block_expert": 4 * lay.tile_capacity // max(lay.tile_block_m, 1),
                "tile_num_post_pad": 4, "x_amax": 4, "x_codes": a.T * a.H,
                "x_scales": 4 * a.T, "a": P * a.I * (4 if fp8 else 2), "a_amax": 4,
                "a_codes": P * a.I, "a_scales": 4 * P}
        spans = sorted((off, off + size[n], n) for n, off in sec.items() if off != NO)
        for (o0, e0, n0), (o1, _, n1) in zip(spans, spans[1:]):
            assert e0 <= o1, (n0, n1)
        assert spans[-1][1] <= lay.total
        if lay.tiled:
            assert lay.tile_block_m == 256 and lay.tile_threshold == 16 and lay.block_m == 16


def test_workspace_bytes_bound_the_down_parts(L):
    """The partial-row buffer is sized for the most parts any shape choice
    could split the down product into, so the size does not depend on the
    device: a one-token call whose I spans 129 chunks (16 parts)."""
    a = _args(T=1, H=256, I=16400, E=2, K=1, wdtype=0)
    n = L.moe_fused_workspace_bytes(ctypes.byref(a))
    assert n >= 16 * 1 * 256 * 4


class _Buf:
    def __init__(self, n):
        self.n = n

    def numel(self):
        return self.n


def test_workspace_pool_policy():
    """Per-stream workspaces: reused per key, grown when too small, at most
    max_entries kept (least recently used dropped), release drops them."""
    made = []

    def alloc(n, key, ctx):
        made.append((key, n, ctx))
        return _Buf(n)

    pool = binding.WorkspacePool(alloc, max_entries=2)
    a = pool.get("s1", 1000, "ctx1")
    assert a.numel() == 1000 and made[-1] == ("s1", 1000, "ctx1")
    assert pool.get("s1", 500) is a and len(made) == 1          # reused: large enough
    b = pool.get("s1", 4000)
    assert b is not a and b.numel() == 4000 and len(pool) == 1  # grown in place of a
    pool.get("s2", 10)
    assert pool.get("s2", 10).numel() == 256                    # minimum size
    pool.get("s1", 10)                                          # s1 most recent now
    pool.get("s3", 10)                                          # evicts s2
    assert pool.keys() == ["s1", "s3"] and len(pool) == 2
    pool.release("s1")
    assert pool.keys() == ["s3"]
    pool.release()
    assert len(pool) == 0
    with pytest.raises(ValueError):
        binding.WorkspacePool(alloc, max_entries=0)


def test_noalloc_validation(L):
    """The no-allocation entry point checks everything on the host first: a
    call whose workspace exceeds the scratch buffer is refused, as are bad
    arguments, without touching a device (none is present here)."""
    big = _args(T=4096, H=7168, I=2048, E=256, K=8, workspace=None, workspace_bytes=0)
    assert L.moe_fused_workspace_bytes(ctypes.byref(big)) > binding.NOALLOC_SCRATCH_BYTES
    assert L.moe_fused_forward_noalloc(ctypes.byref(big), None) == WS
    assert L.moe_fused_forward_noalloc(None, None) == NULL
    assert L.moe_fused_forward_noalloc(ctypes.byref(_args(K=17)), None) == SHAPE
    assert L.moe_fused_forward_noalloc(ctypes.byref(_args(x=None)), None) == NULL
    assert L.moe_fused_forward_noalloc(ctypes.byref(_args(out=4097)), None) == UNSUP
    assert L.moe_fused_forward_noalloc(ctypes.byref(_args(T=0, x=None, out=None)), None) == OK


def test_inv_rope_validation(L):
    p = ctypes.c_void_p(256)
    E4, E5 = binding.MOE_FP8_E4M3, binding.MOE_FP8_E5M2
    f = L.moe_inv_rope_fp8_quant_per_head
    assert f(p, 512, p, p, 100, 4, 4, 128, 130, 0, E4, p, p, None) == SHAPE     # R > D
    assert f(p, 512, p, p, 100, 4, 4, 128, 63, 0, E4, p, p, None) == SHAPE      # odd R
    assert f(p, 512, p, p, 100, 4, 4, 128, 24, 0, E4, p, p, None) == UNSUP      # half: R % 16
    assert f(p, 512, p, p, 100, 4, 4, 128, 20, 1, E5, p, p, None) == UNSUP      # R % 8
    assert f(p, 4 * 520, p, p, 100, 4, 4, 520, 16, 0, E4, p, p, None) == UNSUP  # D > 512
    assert f(p, 512, p, p, 100, 4, 4, 124, 16, 0, E4, p, p, None) == UNSUP     # D % 8
    assert f(p, 256, p, p, 100, 4, 4, 128, 128, 0, E4, p, p, None) == UNSUP    # stride < NH*D
    assert f(p, 512, p, p, 100, 4, 4, 128, 128, 0, binding.MOE_BF16, p, p, None) == UNSUP
    assert f(p, 512, None, p, 100, 4, 4, 128, 128, 0, E4, p, p, None) == NULL
    assert f(ctypes.c_void_p(258), 512, p, p, 100, 4, 4, 128, 128, 0, E4, p, p, None) == UNSUP
    assert f(p, 512, p, p, 0, 4, 4, 128, 128, 0, E4, p, p, None) == SHAPE       # empty table
    assert f(None, 512, None, None, 100, 0, 4, 128, 128, 0, E4, None, None, None) == OK
