"""ctypes binding of libmoe.so (include/moe.h): same names, argument marshalling only.

Every function takes torch tensors (device memory) or None for NULL, passes
their data pointers and the current HIP stream to the C ABI, and raises
MoeError on a non-OK status.  All computation happens in the library's
kernels; there is no fallback path.
"""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_HIP = -4
MOE_BF16 = 0
MOE_FP8_E4M3_BLOCK128 = 1
MOE_MXFP8 = 2

# Every function include/moe.h declares, with (restype, argtypes).
_P = ctypes.c_void_p
_SZ = ctypes.c_size_t


class MoeShape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("I", ctypes.c_int32), ("n_shared", ctypes.c_int32),
                ("wdtype", ctypes.c_int32), ("e_first", ctypes.c_int32), ("e_local", ctypes.c_int32)]


_SP = ctypes.POINTER(MoeShape)
SIGNATURES = {
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_abi_version": (ctypes.c_int, []),
    "moe_forward_workspace_bytes": (_SZ, [_SP]),
    "moe_workspace_bytes": (_SZ, [_SP]),
    "moe_ffn_workspace_bytes": (_SZ, [_SP]),
    "moe_route_workspace_bytes": (_SZ, [_SP]),
    "moe_route": (ctypes.c_int, [_SP, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_route_from_logits": (ctypes.c_int, [_SP, _P, _P, _P, _P]),
    "moe_permute_workspace_bytes": (_SZ, [_SP]),
    "moe_permute": (ctypes.c_int, [_SP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_grouped_ffn": (ctypes.c_int, [_SP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_combine": (ctypes.c_int, [_SP, _P, _P, _P, _P, _P, _P]),
    "moe_forward": (ctypes.c_int, [_SP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_forward_noalloc": (ctypes.c_int, [_SP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_profile_start": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int]),
    "moe_profile_count": (ctypes.c_int, []),
    "moe_profile_read": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(ctypes.c_float),
                                        ctypes.POINTER(ctypes.c_char_p)]),
    "moe_profile_stop": (ctypes.c_int, []),
}

_lib = None


class MoeError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"libmoe error {code}: {msg}")
        self.code = code


def lib() -> ctypes.CDLL:
    """Load libmoe.so from the package directory (fails loudly if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() "
                               "(hipcc --offload-arch=gfx950) first")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def make_shape(T, H, E, k, I, n_shared=0, wdtype=MOE_BF16, e_first=0, e_local=0) -> MoeShape:
    if isinstance(wdtype, str):
        wdtype = {"bf16": MOE_BF16, "fp8": MOE_FP8_E4M3_BLOCK128, "mxfp8": MOE_MXFP8}[wdtype]
    return MoeShape(T, H, E, k, I, n_shared, wdtype, e_first, e_local)


def shape_of(cfg) -> MoeShape:
    return make_shape(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.n_shared, cfg.wdtype,
                      getattr(cfg, "e_first", 0), getattr(cfg, "e_local", 0))


def _nbytes(t) -> int:
    return t.numel() * t.element_size() if t is not None else 0


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("libmoe needs contiguous tensors")
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(rc, fn):
    if rc != MOE_OK:
        raise MoeError(rc, f"{fn}: {lib().moe_last_error().decode()}")


def moe_last_error() -> str:
    return lib().moe_last_error().decode()


def moe_abi_version() -> int:
    return lib().moe_abi_version()


def moe_forward_workspace_bytes(shape: MoeShape) -> int:
    return lib().moe_forward_workspace_bytes(ctypes.byref(shape))


def moe_workspace_bytes(shape: MoeShape) -> int:
    return lib().moe_workspace_bytes(ctypes.byref(shape))


def moe_ffn_workspace_bytes(shape: MoeShape) -> int:
    return lib().moe_ffn_workspace_bytes(ctypes.byref(shape))


def moe_route_workspace_bytes(shape: MoeShape) -> int:
    return lib().moe_route_workspace_bytes(ctypes.byref(shape))


def moe_route(shape, x, w_router, router_bias, logits, topk_idx, topk_w, workspace=None,
              stream=None):
    _check(lib().moe_route(ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(router_bias),
                           _ptr(logits), _ptr(topk_idx), _ptr(topk_w), _ptr(workspace),
                           _nbytes(workspace), _stream(stream)), "moe_route")


def moe_route_from_logits(shape, logits, topk_idx, topk_w, stream=None):
    _check(lib().moe_route_from_logits(ctypes.byref(shape), _ptr(logits), _ptr(topk_idx),
                                       _ptr(topk_w), _stream(stream)), "moe_route_from_logits")


def moe_permute_workspace_bytes(shape: MoeShape) -> int:
    return lib().moe_permute_workspace_bytes(ctypes.byref(shape))


def moe_permute(shape, topk_idx, x, counts, offsets, dest, src_row, x_perm, x_perm_scale,
                workspace=None, stream=None):
    _check(lib().moe_permute(ctypes.byref(shape), _ptr(topk_idx), _ptr(x), _ptr(counts),
                             _ptr(offsets), _ptr(dest), _ptr(src_row), _ptr(x_perm),
                             _ptr(x_perm_scale), _ptr(workspace), _nbytes(workspace),
                             _stream(stream)), "moe_permute")


def moe_grouped_ffn(shape, offsets, x_perm, x_perm_scale, w_gate, w_up, w_down, s_gate, s_up,
                    s_down, y_perm, workspace, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().moe_grouped_ffn(ctypes.byref(shape), _ptr(offsets), _ptr(x_perm),
                                 _ptr(x_perm_scale), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                                 _ptr(s_gate), _ptr(s_up), _ptr(s_down), _ptr(y_perm),
                                 _ptr(workspace), ws_bytes, _stream(stream)), "moe_grouped_ffn")


def moe_combine(shape, y_perm, dest, topk_w, offsets, out, stream=None):
    _check(lib().moe_combine(ctypes.byref(shape), _ptr(y_perm), _ptr(dest), _ptr(topk_w),
                             _ptr(offsets), _ptr(out), _stream(stream)), "moe_combine")


def moe_forward(shape, x, w_router, router_bias, w_gate, w_up, w_down, s_gate, s_up, s_down,
                out, topk_idx_out, topk_w_out, workspace, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().moe_forward(ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(router_bias),
                             _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(s_gate), _ptr(s_up),
                             _ptr(s_down), _ptr(out), _ptr(topk_idx_out), _ptr(topk_w_out),
                             _ptr(workspace), ws_bytes, _stream(stream)), "moe_forward")


NOALLOC_SCRATCH_BYTES = 64 << 20   # MOE_NOALLOC_SCRATCH_BYTES


def moe_forward_noalloc(shape, x, w_router, router_bias, w_gate, w_up, w_down, s_gate, s_up,
                        s_down, out, topk_idx_out, topk_w_out, stream=None):
    _check(lib().moe_forward_noalloc(ctypes.byref(shape), _ptr(x), _ptr(w_router),
                                     _ptr(router_bias), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                                     _ptr(s_gate), _ptr(s_up), _ptr(s_down), _ptr(out),
                                     _ptr(topk_idx_out), _ptr(topk_w_out), _stream(stream)),
           "moe_forward_noalloc")


def moe_profile_start(mode: int, which: int = 0, capacity: int = 64) -> None:
    rc = lib().moe_profile_start(mode, which, capacity)
    if rc != MOE_OK:
        raise MoeError(rc, "moe_profile_start failed")


def moe_profile_count() -> int:
    return lib().moe_profile_count()


def moe_profile_read(i: int):
    """(milliseconds, kernel name) of recorded event pair i (waits for it)."""
    ms = ctypes.c_float()
    name = ctypes.c_char_p()
    rc = lib().moe_profile_read(i, ctypes.byref(ms), ctypes.byref(name))
    if rc != MOE_OK:
        raise MoeError(rc, f"moe_profile_read({i}) failed")
    return ms.value, name.value.decode()


def moe_profile_stop() -> None:
    lib().moe_profile_stop()
