"""Host-side checks of the C ABI (CPU only; no kernel is launched).

* the shared library loads and exports every function include/moe_w4a16.h declares;
* the Python binding's prototypes agree with the header (argument counts and order of
  pointer / integer kinds) -- a signature-drift contract like the AST contract tests the
  b12x PR 137 page describes;
* size queries and argument validation return the documented status codes.
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_w4a16.h")

moe = pytest.importorskip("fp4_weight_grouped_moe_amd")


def _declarations():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    decls = {}
    for m in re.finditer(r"^(?:int|int64_t|const char\*)\s+(moe_\w+)\s*\(([^;]*?)\)\s*;", src, flags=re.M | re.S):
        args = [a.strip() for a in m.group(2).replace("\n", " ").split(",")]
        args = [] if args == ["void"] else args
        decls[m.group(1)] = args
    return decls


def test_header_declares_the_expected_entry_points():
    decls = _declarations()
    assert set(decls) == set(moe.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(moe.LIB_PATH)
    for name in _declarations():
        assert hasattr(lib, name), name


def _kind(c_arg: str) -> str:
    c_arg = c_arg.strip()
    if "*" in c_arg or c_arg.startswith("hipStream_t"):
        return "ptr"
    if c_arg.startswith(("int64_t", "size_t")):
        return "i64"
    return "i32"


def _ctype_kind(t) -> str:
    if t in (ctypes.c_int64, ctypes.c_size_t):
        return "i64"
    if t in (ctypes.c_int, ctypes.c_int32):
        return "i32"
    return "ptr"


def test_binding_prototypes_match_header():
    decls = _declarations()
    lib = moe.lib()
    for name, args in decls.items():
        fn = getattr(lib, name)
        got = [_ctype_kind(t) for t in fn.argtypes]
        want = [_kind(a) for a in args]
        assert got == want, (name, got, want)


def test_token_capacity():
    f = moe.moe_route_pack_token_capacity
    assert [f(m) for m in (0, 1, 2, 3, 4, 5, 300, 511, 512, 513, 2048)] == [1, 1, 2, 4, 4, 8, 512, 512, 512, 1024, 2048]
    assert f(-1) == -1


def test_route_pack_workspace_size_matches_capacity_formula():
    from oracle.route_pack import capacities
    for cap, k, E, B in [(1, 8, 128, 16), (512, 4, 64, 16), (2048, 8, 256, 16), (4, 2, 8, 128), (8, 3, 3, 32)]:
        n = moe.moe_route_pack_workspace_size(cap, k, E, B)
        cr, cb = capacities(cap, k, E, B)
        # counts, offsets, sorted, blocks, live, route_slot and the fused-layer tables fit
        assert n >= 4 * (E + (E + 1) + cr + cb + 4 + cap * k)
        assert n % 256 == 0


@pytest.mark.parametrize("args,code", [
    ((3, 2, 8, 16), moe.MOE_ERR_INVALID_ARG),      # capacity not a power of two
    ((4, 0, 8, 16), moe.MOE_ERR_INVALID_ARG),      # topk 0
    ((4, 65, 8, 16), moe.MOE_ERR_INVALID_ARG),     # topk too large
    ((4, 2, 0, 16), moe.MOE_ERR_INVALID_ARG),      # no experts
    ((4, 2, 4096, 16), moe.MOE_ERR_INVALID_ARG),   # beyond the LDS histogram bound
    ((4, 2, 8, 17), moe.MOE_ERR_INVALID_ARG),      # block_m not supported
])
def test_route_pack_size_rejects(args, code):
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_route_pack_workspace_size(*args)
    assert ei.value.code == code
    assert moe.moe_last_error()


@pytest.mark.parametrize("dims,code", [
    (("nvfp4", "silu_swiglu", 8, 255, 128), moe.MOE_ERR_UNSUPPORTED),   # odd hidden
    (("nvfp4", "silu_swiglu", 8, 260, 128), moe.MOE_ERR_UNSUPPORTED),   # hidden not a multiple of 8
    (("nvfp4", "relu2", 8, 256, 127), moe.MOE_ERR_UNSUPPORTED),         # odd inter
    ((3, "relu2", 8, 256, 128), moe.MOE_ERR_UNSUPPORTED),               # unknown format
    (("mxfp4", 7, 8, 256, 128), moe.MOE_ERR_UNSUPPORTED),               # unknown activation
    (("mxfp4", "relu2", 0, 256, 128), moe.MOE_ERR_INVALID_ARG),         # no experts
])
def test_prepared_size_rejects(dims, code):
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_w4a16_prepared_size(moe.make_dims(*dims))
    assert ei.value.code == code


def test_prepared_size_counts_every_region():
    d = moe.make_dims("nvfp4", "silu_swiglu", 128, 4096, 1536)
    n = moe.moe_w4a16_prepared_size(d)
    # E * (2I*H + H*I) / 2 nibble bytes and one scale byte per 16 weights, plus two fp32 globals per expert
    nib = 128 * (2 * 1536 * 4096 + 4096 * 1536) // 2
    assert n >= nib + nib // 8 + 2 * 4 * 128
    assert n <= (nib + nib // 8) * 1.01 + 4096
    d2 = moe.make_dims("mxfp4", "silu_swiglu", 64, 3072, 1400)     # I = 1400 pads to 1408
    assert moe.moe_w4a16_prepared_size(d2) >= 64 * (2 * 1408 * 3072 + 3072 * 1408) // 2


def test_fused_validation_precedes_device_access():
    d = moe.make_dims("mxfp4", "silu_swiglu", 8, 256, 128)
    psz = moe.moe_w4a16_prepared_size(d)
    wsz = moe.moe_w4a16_workspace_size(d, 4, 2)
    fake = 1 << 20          # an aligned address that is never dereferenced: every case fails validation first

    def call(**kw):
        a = dict(prepared=fake, prepared_bytes=psz, x=fake, m=4, topk_ids=fake, topk_weights=fake, topk=2,
                 expert_map=None, num_global_experts=8, token_capacity=4, workspace=fake, workspace_bytes=wsz,
                 out=fake, stream=0)
        a.update(kw)
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_w4a16_fused(d, **a)
        return ei.value.code

    assert call(workspace_bytes=wsz - 1) == moe.MOE_ERR_WORKSPACE
    assert call(prepared_bytes=psz - 1) == moe.MOE_ERR_WORKSPACE
    assert call(m=5) == moe.MOE_ERR_INVALID_ARG                    # m above the capacity
    assert call(token_capacity=6) == moe.MOE_ERR_INVALID_ARG
    assert call(x=0) == moe.MOE_ERR_INVALID_ARG
    assert call(x=fake + 2) == moe.MOE_ERR_INVALID_ARG             # misaligned activations
    assert call(workspace=fake + 64) == moe.MOE_ERR_INVALID_ARG    # workspace not 256-byte aligned
    assert call(num_global_experts=0) == moe.MOE_ERR_INVALID_ARG
    prev = moe.moe_w4a16_set_path("decode")
    try:
        wsz32 = moe.moe_w4a16_workspace_size(d, 32, 2)
        assert call(m=17, token_capacity=32, workspace_bytes=wsz32) == moe.MOE_ERR_UNSUPPORTED
    finally:
        moe.moe_w4a16_set_path(prev)


def test_path_and_threshold_setters():
    prev = moe.moe_w4a16_set_path(2)
    assert moe.moe_w4a16_set_path(prev) == 2
    with pytest.raises(moe.MoeError):
        moe.moe_w4a16_set_path(3)
    old = moe.moe_w4a16_set_decode_max_m(4)
    assert moe.moe_w4a16_set_decode_max_m(old) == 4
    with pytest.raises(moe.MoeError):
        moe.moe_w4a16_set_decode_max_m(17)
    old = moe.moe_w4a16_set_grid_limit(3)
    assert moe.moe_w4a16_set_grid_limit(old) == 3
    with pytest.raises(moe.MoeError):
        moe.moe_w4a16_set_grid_limit(-1)


def test_one_hip_runtime_in_process():
    """The library must bind to the HIP runtime torch loaded, never a second copy."""
    import subprocess
    import sys
    code = ("import fp4_weight_grouped_moe_amd, torch\n"
            "libs = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}\n"
            "print(len(libs))\n")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip() == "1", out.stdout


def test_binding_rejects_mismatched_tensors_before_any_call():
    """int64 ids (what torch.topk returns), transposed views, wrong widths and host tensors are
    refused by the binding with MOE_ERR_INVALID_ARG instead of being read as wrong data."""
    torch = pytest.importorskip("torch")
    d = moe.make_dims("mxfp4", "silu_swiglu", 8, 256, 128)
    m, k = 4, 2
    good = dict(x=torch.zeros((m, 256), dtype=torch.bfloat16), topk_ids=torch.zeros((m, k), dtype=torch.int32),
                topk_weights=torch.zeros((m, k), dtype=torch.float32), out=torch.zeros((m, 256), dtype=torch.bfloat16))

    def code(**kw):
        a = dict(good)
        a.update(kw)
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_w4a16_fused(d, 1 << 20, 1 << 30, a["x"], m, a["topk_ids"], a["topk_weights"], k, None, 8, 4,
                                1 << 20, 1 << 30, a["out"], stream=0)
        return ei.value.code, str(ei.value)

    c, msg = code(topk_ids=torch.zeros((m, k), dtype=torch.int64))
    assert c == moe.MOE_ERR_INVALID_ARG and "topk_ids" in msg and "int32" in msg
    c, msg = code(x=torch.zeros((256, m), dtype=torch.bfloat16).t())
    assert c == moe.MOE_ERR_INVALID_ARG and "x" in msg
    c, msg = code(topk_weights=torch.zeros((m, k + 1), dtype=torch.float32))
    assert c == moe.MOE_ERR_INVALID_ARG and "topk_weights" in msg
    c, msg = code(out=torch.zeros((m, 256), dtype=torch.float32))
    assert c == moe.MOE_ERR_INVALID_ARG and "out" in msg
    c, msg = code()                                              # host tensors of the right kinds
    assert c == moe.MOE_ERR_INVALID_ARG and "cpu" in msg


def test_profiled_twin_validates_its_event_arguments():
    d = moe.make_dims("mxfp4", "silu_swiglu", 8, 256, 128)
    lib = moe.lib()
    ids = (ctypes.c_int32 * 5)()
    n = ctypes.c_int(7)
    ev = (ctypes.c_void_p * 5)()
    rc = lib.moe_w4a16_fused_profiled(ctypes.byref(d), 1 << 20, 1 << 30, 1 << 20, 4, 1 << 20, 1 << 20, 2, None, 8, 4,
                                      1 << 20, 1 << 30, 1 << 20, None, ev, 5, ids, ctypes.byref(n))
    assert rc == moe.MOE_ERR_INVALID_ARG
    ev6 = (ctypes.c_void_p * 6)()
    rc = lib.moe_w4a16_fused_profiled(ctypes.byref(d), 1 << 20, 1 << 30, 1 << 20, 4, 1 << 20, 1 << 20, 2, None, 8, 4,
                                      1 << 20, 1 << 30, 1 << 20, None, ev6, 6, None, ctypes.byref(n))
    assert rc == moe.MOE_ERR_INVALID_ARG
