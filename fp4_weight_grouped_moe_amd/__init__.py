"""Python binding of libmoe_w4a16.so, the MI355X (gfx950) fused W4A16 MoE layer.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels. Functions carry the C names of include/moe_w4a16.h and take torch
tensors (device memory) or raw integer device pointers; torch supplies memory
and the current HIP stream. If the library has not been built this module
raises on import -- there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_w4a16.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_HIP = -4

MOE_FMT_NVFP4_E4M3_K16 = 1
MOE_FMT_MXFP4_E8M0_K32 = 2
MOE_ACT_SILU_SWIGLU = 1
MOE_ACT_RELU2 = 2
MOE_DECODE_MAX_M = 16
MOE_STATIC_WORKSPACE_BYTES = 64 << 20

FMT = {"nvfp4": MOE_FMT_NVFP4_E4M3_K16, "mxfp4": MOE_FMT_MXFP4_E8M0_K32}
ACT = {"silu_swiglu": MOE_ACT_SILU_SWIGLU, "relu2": MOE_ACT_RELU2}
PATH = {"auto": 0, "decode": 1, "gemm": 2}


class MoeError(RuntimeError):
    def __init__(self, code: int, where: str, msg: str):
        super().__init__(f"{where} failed with status {code}: {msg}")
        self.code = code


class moe_w4a16_dims(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("act", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32)]


class moe_w4a16_source_layout(ctypes.Structure):
    _fields_ = [("w13_up_first", ctypes.c_int32), ("global_scale_reciprocal", ctypes.c_int32),
                ("scale_per_row", ctypes.c_int32), ("w13_interleaved", ctypes.c_int32)]


class moe_route_pack_view(ctypes.Structure):
    _fields_ = [("expert_counts", ctypes.c_void_p), ("expert_offsets", ctypes.c_void_p),
                ("sorted_route_ids", ctypes.c_void_p), ("block_expert", ctypes.c_void_p),
                ("live", ctypes.c_void_p), ("route_slot", ctypes.c_void_p),
                ("token_capacity", ctypes.c_int64), ("cap_routes", ctypes.c_int64),
                ("cap_blocks", ctypes.c_int64), ("block_m", ctypes.c_int32), ("num_experts", ctypes.c_int32)]


def _load():
    # torch wheels bundle their own libamdhip64 with the same soname as ROCm's. Loading
    # torch first makes this library bind to that runtime; the other order would put two
    # HIP runtimes in the process, and torch's streams and pointers would not be valid in
    # the one the kernels launch on.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
                          "(hipcc, gfx950). There is no CPU fallback.")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    PSZ = ctypes.POINTER(ctypes.c_size_t)
    PD = ctypes.POINTER(moe_w4a16_dims)
    sig = {
        "moe_route_pack_token_capacity": (I64, [I64]),
        "moe_route_pack_workspace_size": (I32, [I64, I32, I32, I32, PSZ]),
        "moe_route_pack": (I32, [P, I64, I32, P, I32, I32, I32, I64, P, SZ, ctypes.POINTER(moe_route_pack_view), P]),
        "moe_w4a16_prepared_size": (I32, [PD, PSZ]),
        "moe_w4a16_prepare": (I32, [PD, P, P, P, P, P, P, P, SZ, P]),
        "moe_w4a16_workspace_size": (I32, [PD, I64, I32, PSZ]),
        "moe_w4a16_fused": (I32, [PD, P, SZ, P, I64, P, P, I32, P, I32, I64, P, SZ, P, P]),
        "moe_w4a8_fused": (I32, [PD, P, SZ, P, I64, P, P, I32, P, I32, I64, P, SZ, P, P]),
        "moe_w4a16_fused_device_m": (I32, [PD, P, SZ, P, P, P, P, I32, P, I32, I64, P, SZ, P, P]),
        "moe_w4a16_fused_atomic_bf16": (I32, [PD, P, SZ, P, I64, P, P, I32, P, I32, I64, P, SZ, P, P]),
        "moe_w4a16_fused_static_workspace": (I32, [PD, P, SZ, P, I64, P, P, I32, P, I32, I64, P, P]),
        "moe_w4a16_fused_profiled": (I32, [PD, P, SZ, P, I64, P, P, I32, P, I32, I64, P, SZ, P, P, P, I32,
                                           ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int)]),
        "moe_last_error": (ctypes.c_char_p, []),
        "moe_w4a16_set_path": (I32, [I32]),
        "moe_w4a16_set_decode_max_m": (I32, [I32]),
        "moe_w4a16_set_grid_limit": (I32, [I32]),
        "moe_router_topk": (I32, [P, I64, I32, I32, I32, I32, P, P, P]),
        "moe_w4a16_prepare_layout": (I32, [PD, ctypes.POINTER(moe_w4a16_source_layout), P, P, P, P, P, P, P, SZ, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()
EXPORTED = ("moe_route_pack_token_capacity", "moe_route_pack_workspace_size", "moe_route_pack",
            "moe_w4a16_prepared_size", "moe_w4a16_prepare", "moe_w4a16_workspace_size", "moe_w4a16_fused",
            "moe_w4a8_fused", "moe_w4a16_fused_atomic_bf16", "moe_w4a16_fused_static_workspace",
            "moe_w4a16_fused_device_m",
            "moe_w4a16_fused_profiled", "moe_last_error", "moe_w4a16_set_path", "moe_w4a16_set_decode_max_m",
            "moe_w4a16_set_grid_limit",
            "moe_router_topk", "moe_w4a16_prepare_layout")


def lib():
    return _lib


def _ptr(t) -> int:
    if t is None:
        return 0
    if isinstance(t, int):
        return t
    return int(t.data_ptr())


def _stream(stream) -> int:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def _check(rc: int, where: str) -> int:
    if rc < 0:
        raise MoeError(rc, where, moe_last_error())
    return rc


def _require(t, name: str, dtype, rows, cols, device, where: str) -> None:
    """Raise MoeError (MOE_ERR_INVALID_ARG) unless torch tensor ``t`` has this dtype, is contiguous
    and holds at least ``rows`` rows of ``cols`` elements ([rows, cols], or [rows] when cols is
    None); _require_device then checks that every tensor sits on the same GPU. Raw integer pointers and None pass
    unchecked: they are the caller's responsibility. No arithmetic: a mismatch here (int64 ids,
    a transposed view, a host tensor) would otherwise be read as wrong data without an error."""
    if t is None or isinstance(t, int):
        return
    if t.dtype != dtype:
        raise MoeError(MOE_ERR_INVALID_ARG, where, f"{name} must be {dtype}, got {t.dtype}")
    shape = tuple(t.shape)
    ok = (len(shape) == 1 and shape[0] >= rows) if cols is None else (len(shape) == 2 and shape[0] >= rows
                                                                       and shape[1] == cols)
    if not ok:
        want = f"[>= {rows}]" if cols is None else f"[>= {rows}, {cols}]"
        raise MoeError(MOE_ERR_INVALID_ARG, where, f"{name} must have shape {want}, got {list(shape)}")
    if not t.is_contiguous():
        raise MoeError(MOE_ERR_INVALID_ARG, where, f"{name} must be contiguous")


def _require_device(t, name: str, device, where: str) -> None:
    if t is None or isinstance(t, int):
        return
    if t.device.type != "cuda" or (device is not None and t.device != device):
        raise MoeError(MOE_ERR_INVALID_ARG, where, f"{name} is on {t.device}, expected {device or 'a GPU'}")


def _check_fused_args(dims, x, m, topk_ids, topk_weights, topk, expert_map, num_global_experts, out, where) -> None:
    import torch
    args = (("x", x, torch.bfloat16, m, dims.hidden), ("topk_ids", topk_ids, torch.int32, m, topk),
            ("topk_weights", topk_weights, torch.float32, m, topk),
            ("expert_map", expert_map, torch.int32, num_global_experts, None),
            ("out", out, torch.bfloat16, m, dims.hidden))
    for name, t, dtype, rows, cols in args:
        _require(t, name, dtype, rows, cols, None, where)
    device = next((t.device for _, t, *_ in args if t is not None and not isinstance(t, int)), None)
    for name, t, *_ in args:
        _require_device(t, name, device, where)


def make_dims(fmt, act, num_experts: int, hidden: int, inter: int) -> moe_w4a16_dims:
    f = FMT.get(fmt, fmt)
    a = ACT.get(act, act)
    return moe_w4a16_dims(int(f), int(a), int(num_experts), int(hidden), int(inter))


def moe_last_error() -> str:
    s = _lib.moe_last_error()
    return s.decode() if s else ""


def moe_route_pack_token_capacity(m: int) -> int:
    return int(_lib.moe_route_pack_token_capacity(int(m)))


def moe_route_pack_workspace_size(token_capacity: int, topk: int, num_local_experts: int, block_m: int) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib.moe_route_pack_workspace_size(token_capacity, topk, num_local_experts, block_m, ctypes.byref(n)),
           "moe_route_pack_workspace_size")
    return n.value


def moe_route_pack(topk_ids, m: int, topk: int, expert_map, num_global_experts: int, num_local_experts: int,
                   block_m: int, token_capacity: int, workspace, workspace_bytes: int, stream=None) -> moe_route_pack_view:
    view = moe_route_pack_view()
    _check(_lib.moe_route_pack(_ptr(topk_ids), m, topk, _ptr(expert_map), num_global_experts, num_local_experts,
                               block_m, token_capacity, _ptr(workspace), workspace_bytes, ctypes.byref(view),
                               _stream(stream)), "moe_route_pack")
    return view


def moe_w4a16_prepared_size(dims: moe_w4a16_dims) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib.moe_w4a16_prepared_size(ctypes.byref(dims), ctypes.byref(n)), "moe_w4a16_prepared_size")
    return n.value


def moe_w4a16_prepare(dims: moe_w4a16_dims, w13, s13, g13, w2, s2, g2, prepared, prepared_bytes: int,
                      stream=None) -> None:
    _check(_lib.moe_w4a16_prepare(ctypes.byref(dims), _ptr(w13), _ptr(s13), _ptr(g13), _ptr(w2), _ptr(s2),
                                  _ptr(g2), _ptr(prepared), prepared_bytes, _stream(stream)), "moe_w4a16_prepare")


def moe_w4a16_workspace_size(dims: moe_w4a16_dims, token_capacity: int, topk: int) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib.moe_w4a16_workspace_size(ctypes.byref(dims), token_capacity, topk, ctypes.byref(n)),
           "moe_w4a16_workspace_size")
    return n.value


def moe_w4a16_fused(dims: moe_w4a16_dims, prepared, prepared_bytes: int, x, m: int, topk_ids, topk_weights,
                    topk: int, expert_map, num_global_experts: int, token_capacity: int, workspace,
                    workspace_bytes: int, out, stream=None) -> None:
    _check_fused_args(dims, x, m, topk_ids, topk_weights, topk, expert_map, num_global_experts, out, "moe_w4a16_fused")
    _check(_lib.moe_w4a16_fused(ctypes.byref(dims), _ptr(prepared), prepared_bytes, _ptr(x), m, _ptr(topk_ids),
                                _ptr(topk_weights), topk, _ptr(expert_map), num_global_experts, token_capacity,
                                _ptr(workspace), workspace_bytes, _ptr(out), _stream(stream)), "moe_w4a16_fused")


def moe_w4a16_fused_device_m(dims: moe_w4a16_dims, prepared, prepared_bytes: int, x, m_device, topk_ids,
                             topk_weights, topk: int, expert_map, num_global_experts: int, token_capacity: int,
                             workspace, workspace_bytes: int, out, stream=None) -> None:
    """The fused layer with m read from the device int32 ``m_device`` when the call runs; x,
    topk_ids, topk_weights and out hold token_capacity rows (rows at or past m of out become 0)."""
    import torch
    _check_fused_args(dims, x, token_capacity, topk_ids, topk_weights, topk, expert_map, num_global_experts, out,
                      "moe_w4a16_fused_device_m")
    _require(m_device, "m_device", torch.int32, 1, None, None, "moe_w4a16_fused_device_m")
    _check(_lib.moe_w4a16_fused_device_m(ctypes.byref(dims), _ptr(prepared), prepared_bytes, _ptr(x), _ptr(m_device),
                                         _ptr(topk_ids), _ptr(topk_weights), topk, _ptr(expert_map),
                                         num_global_experts, token_capacity, _ptr(workspace), workspace_bytes,
                                         _ptr(out), _stream(stream)), "moe_w4a16_fused_device_m")


def moe_w4a8_fused(dims: moe_w4a16_dims, prepared, prepared_bytes: int, x, m: int, topk_ids, topk_weights,
                   topk: int, expert_map, num_global_experts: int, token_capacity: int, workspace,
                   workspace_bytes: int, out, stream=None) -> None:
    _check_fused_args(dims, x, m, topk_ids, topk_weights, topk, expert_map, num_global_experts, out, "moe_w4a8_fused")
    _check(_lib.moe_w4a8_fused(ctypes.byref(dims), _ptr(prepared), prepared_bytes, _ptr(x), m, _ptr(topk_ids),
                               _ptr(topk_weights), topk, _ptr(expert_map), num_global_experts, token_capacity,
                               _ptr(workspace), workspace_bytes, _ptr(out), _stream(stream)), "moe_w4a8_fused")


def moe_w4a16_fused_atomic_bf16(dims: moe_w4a16_dims, prepared, prepared_bytes: int, x, m: int, topk_ids,
                                topk_weights, topk: int, expert_map, num_global_experts: int, token_capacity: int,
                                workspace, workspace_bytes: int, out, stream=None) -> None:
    _check_fused_args(dims, x, m, topk_ids, topk_weights, topk, expert_map, num_global_experts, out, "moe_w4a16_fused_atomic_bf16")
    _check(_lib.moe_w4a16_fused_atomic_bf16(ctypes.byref(dims), _ptr(prepared), prepared_bytes, _ptr(x), m,
                                            _ptr(topk_ids), _ptr(topk_weights), topk, _ptr(expert_map),
                                            num_global_experts, token_capacity, _ptr(workspace), workspace_bytes,
                                            _ptr(out), _stream(stream)), "moe_w4a16_fused_atomic_bf16")


def moe_w4a16_fused_static_workspace(dims: moe_w4a16_dims, prepared, prepared_bytes: int, x, m: int, topk_ids,
                                     topk_weights, topk: int, expert_map, num_global_experts: int,
                                     token_capacity: int, out, stream=None) -> None:
    """moe_w4a16_fused with the library's own device workspace (no caller workspace, no allocation)."""
    _check_fused_args(dims, x, m, topk_ids, topk_weights, topk, expert_map, num_global_experts, out,
                      "moe_w4a16_fused_static_workspace")
    _check(_lib.moe_w4a16_fused_static_workspace(ctypes.byref(dims), _ptr(prepared), prepared_bytes, _ptr(x), m,
                                                 _ptr(topk_ids), _ptr(topk_weights), topk, _ptr(expert_map),
                                                 num_global_experts, token_capacity, _ptr(out), _stream(stream)),
           "moe_w4a16_fused_static_workspace")


KERNEL_NAMES = ("route_pack", "fc1", "requant", "fc2", "combine")    # moe_kernel_id order


def moe_w4a16_fused_profiled(dims: moe_w4a16_dims, prepared, prepared_bytes: int, x, m: int, topk_ids, topk_weights,
                             topk: int, expert_map, num_global_experts: int, token_capacity: int, workspace,
                             workspace_bytes: int, out, events, stream=None):
    """``events``: six or more HIP event handles (ints) or torch.cuda.Event(enable_timing=True).
    Returns the names of the kernels launched, in order; event j + 1 follows kernel j."""
    _check_fused_args(dims, x, m, topk_ids, topk_weights, topk, expert_map, num_global_experts, out,
                      "moe_w4a16_fused_profiled")
    arr = (ctypes.c_void_p * len(events))(*[e if isinstance(e, int) else int(e.cuda_event) for e in events])
    ids = (ctypes.c_int32 * 5)()
    n = ctypes.c_int(0)
    _check(_lib.moe_w4a16_fused_profiled(ctypes.byref(dims), _ptr(prepared), prepared_bytes, _ptr(x), m,
                                         _ptr(topk_ids), _ptr(topk_weights), topk, _ptr(expert_map),
                                         num_global_experts, token_capacity, _ptr(workspace), workspace_bytes,
                                         _ptr(out), _stream(stream), arr, len(events), ids, ctypes.byref(n)),
           "moe_w4a16_fused_profiled")
    return [KERNEL_NAMES[ids[i]] for i in range(n.value)]


def moe_w4a16_prepare_layout(dims: moe_w4a16_dims, layout: moe_w4a16_source_layout, w13, s13, g13, w2, s2, g2,
                             prepared, prepared_bytes: int, stream=None) -> None:
    _check(_lib.moe_w4a16_prepare_layout(ctypes.byref(dims), ctypes.byref(layout) if layout is not None else None,
                                         _ptr(w13), _ptr(s13), _ptr(g13), _ptr(w2), _ptr(s2), _ptr(g2),
                                         _ptr(prepared), prepared_bytes, _stream(stream)), "moe_w4a16_prepare_layout")


ROUTER_SCORING = {"softmax": 0, "sigmoid": 1}


def moe_router_topk(logits, m: int, num_experts: int, topk: int, scoring, renormalize: bool, topk_ids,
                    topk_weights, stream=None) -> None:
    """Top-k experts and weights of fp32 logits [m, num_experts] (device tensors)."""
    _check(_lib.moe_router_topk(_ptr(logits), m, num_experts, topk, ROUTER_SCORING.get(scoring, scoring),
                                1 if renormalize else 0, _ptr(topk_ids), _ptr(topk_weights), _stream(stream)),
           "moe_router_topk")


def moe_w4a16_set_path(path) -> int:
    return _check(_lib.moe_w4a16_set_path(PATH.get(path, path)), "moe_w4a16_set_path")


def moe_w4a16_set_decode_max_m(max_m: int) -> int:
    return _check(_lib.moe_w4a16_set_decode_max_m(int(max_m)), "moe_w4a16_set_decode_max_m")


def moe_w4a16_set_grid_limit(max_cus: int) -> int:
    return _check(_lib.moe_w4a16_set_grid_limit(int(max_cus)), "moe_w4a16_set_grid_limit")


class MoeLayer:
    """Owns the prepared weights and a workspace for one layer shape (torch device memory)."""

    def __init__(self, fmt, act, num_experts, hidden, inter, topk, token_capacity, device="cuda"):
        import torch
        self.dims = make_dims(fmt, act, num_experts, hidden, inter)
        self.topk = int(topk)
        self.token_capacity = int(token_capacity)
        self.prepared_bytes = moe_w4a16_prepared_size(self.dims)
        self.workspace_bytes = moe_w4a16_workspace_size(self.dims, self.token_capacity, self.topk)
        # 256-byte alignment: torch's caching allocator hands out 512-byte aligned blocks.
        self.prepared = torch.empty(self.prepared_bytes, dtype=torch.uint8, device=device)
        self.workspace = torch.empty(self.workspace_bytes, dtype=torch.uint8, device=device)

    def prepare(self, w13, s13, g13, w2, s2, g2, stream=None):
        moe_w4a16_prepare(self.dims, w13, s13, g13, w2, s2, g2, self.prepared, self.prepared_bytes, stream)

    def __call__(self, x, topk_ids, topk_weights, expert_map=None, num_global_experts=None, out=None, stream=None,
                 w4a8=False, atomic_bf16=False):
        """``w4a8``: the W4A8 variant (moe_w4a8_fused; MXFP4 weights only). ``atomic_bf16``: the
        opt-in approximate packed-bf16 atomic top-k combine (moe_w4a16_fused_atomic_bf16)."""
        if w4a8 and atomic_bf16:
            raise ValueError("w4a8 and atomic_bf16 are separate variants")
        import torch
        m = int(x.shape[0])
        if out is None:
            out = torch.empty((m, self.dims.hidden), dtype=torch.bfloat16, device=x.device)
        ng = num_global_experts if num_global_experts is not None else (
            int(expert_map.numel()) if expert_map is not None else self.dims.num_experts)
        fn = moe_w4a8_fused if w4a8 else (moe_w4a16_fused_atomic_bf16 if atomic_bf16 else moe_w4a16_fused)
        fn(self.dims, self.prepared, self.prepared_bytes, x, m, topk_ids, topk_weights, self.topk,
           expert_map, ng, self.token_capacity, self.workspace, self.workspace_bytes, out, stream)
        return out
