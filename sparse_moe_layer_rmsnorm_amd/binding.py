"""ctypes binding of libmoe.so (include/moe.h), with the same names.

Argument marshalling only: every step of the layer runs in the HIP kernels
behind the C ABI.  PyTorch provides device memory and the stream.  Loading
fails loudly when the library has not been built; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re
from ctypes import POINTER, c_char_p, c_double, c_float, c_int, c_int32, c_int64, c_size_t, c_void_p
from typing import Dict, Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "moe.h")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_SHAPE, MOE_ERR_DTYPE, MOE_ERR_WORKSPACE, MOE_ERR_STATE, MOE_ERR_HIP = range(7)
MOE_F32, MOE_BF16 = 0, 1
MOE_QB_TRAIN, MOE_QB_FROZEN = 0, 1
MOE_BALANCE_QB, MOE_BALANCE_SIGN = 0, 1
MOE_EXPERTS_BF16, MOE_EXPERTS_MXFP8, MOE_EXPERTS_MXFP4 = 0, 1, 2
_EXPERT_FORMATS = {"bf16": MOE_EXPERTS_BF16, "mxfp8": MOE_EXPERTS_MXFP8, "mxfp4": MOE_EXPERTS_MXFP4}
KERNELS = ["rmsnorm", "gemm_h", "topk", "hist", "scan", "scatter", "expert_up", "expert_down", "combine",
           "gemm_out", "qb_update", "qb_bias", "gemm_rz", "sign_bias", "bwd_gemm", "bwd_expert", "bwd_wgrad",
           "bwd_eltwise", "bwd_transpose", "mx_quant"]
MOE_NUM_KERNELS = len(KERNELS)


class moe_config(ctypes.Structure):
    _fields_ = [("d", c_int32), ("l", c_int32), ("E", c_int32), ("k", c_int32), ("f", c_int32), ("f_s", c_int32),
                ("n_shared", c_int32), ("dtype", c_int), ("rms_eps", c_float), ("qb_bins", c_int32),
                ("qb_lo", c_float), ("qb_hi", c_float), ("qb_mode", c_int), ("max_tokens", c_int64),
                ("routed_scale", c_float), ("balancer", c_int), ("sign_gamma", c_float), ("experts", c_int),
                ("keep_preact", c_int32)]


class moe_weights(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("gamma", "W_r", "logit_offset", "W_sg", "W_su", "W_sd", "W_dn", "W_g",
                                        "W_u", "W_d", "W_up")]


class moe_route_out(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("logits", "topk_idx", "gates", "counts", "offsets", "perm_src", "inv")]


class moe_grads(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("gamma", "W_r", "W_sg", "W_su", "W_sd", "W_dn", "W_g", "W_u", "W_d", "W_up")]


class moe_state_layout(ctypes.Structure):
    _fields_ = [(n, c_size_t) for n in ("bias", "count", "q", "hist", "hist_slices", "load", "mx", "total")]


class moe_ws_layout(ctypes.Structure):
    _fields_ = [(n, c_size_t) for n in ("h", "logits", "idx", "gates", "bitmap", "cbase", "sbase", "counts",
                                        "offsets", "tile_offsets", "perm_src", "inv", "tile_info", "G", "z", "X",
                                        "H", "Y", "y_lat", "z8", "zs", "Xs", "H8", "Hs", "P", "Q", "A", "U",
                                        "total")]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libmoe.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m sparse_moe_layer_rmsnorm_amd.build` "
                               "(there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        cfgp = POINTER(moe_config)
        sig = {
            "moe_state_bytes": (c_size_t, [cfgp]),
            "moe_state_layout_of": (c_int, [cfgp, POINTER(moe_state_layout)]),
            "moe_workspace_bytes": (c_size_t, [cfgp, c_int64]),
            "moe_workspace_layout": (c_int, [cfgp, c_int64, POINTER(moe_ws_layout)]),
            "moe_init": (c_int, [cfgp, POINTER(moe_weights), c_void_p, c_void_p, POINTER(c_void_p)]),
            "moe_route": (c_int, [c_void_p, c_void_p, c_void_p, c_int64, POINTER(moe_route_out), c_void_p, c_size_t,
                                  c_void_p]),
            "moe_forward": (c_int, [c_void_p, c_void_p, c_int64, c_void_p, POINTER(moe_route_out), c_void_p,
                                    c_size_t, c_void_p]),
            "moe_forward_noalloc": (c_int, [c_void_p, c_void_p, c_int64, c_void_p, POINTER(moe_route_out),
                                            c_void_p]),
            "moe_backward_workspace_bytes": (c_size_t, [cfgp, c_int64]),
            "moe_backward": (c_int, [c_void_p, c_void_p, c_void_p, c_int64, POINTER(moe_route_out), c_void_p,
                                     c_size_t, c_void_p, POINTER(moe_grads), c_void_p, c_size_t, c_void_p]),
            "qb_update": (c_int, [c_void_p, c_void_p]),
            "moe_requantize_experts": (c_int, [c_void_p, c_void_p]),
            "moe_get_bias": (c_int, [c_void_p, c_void_p, c_void_p]),
            "moe_fast_score_error": (c_int, [c_void_p, c_void_p]),
            "moe_set_bias": (c_int, [c_void_p, c_void_p, c_void_p]),
            "moe_set_qb_mode": (c_int, [c_void_p, c_int]),
            "moe_destroy": (None, [c_void_p]),
            "moe_status_string": (c_char_p, [c_int]),
            "moe_last_error": (c_char_p, []),
            "moe_kernel_name": (c_char_p, [c_int]),
            "moe_profile_begin": (c_int, [c_void_p, c_int, ctypes.c_uint32]),
            "moe_profile_end": (c_int, [c_void_p, POINTER(c_double), POINTER(c_int64), c_int]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def header_functions() -> list:
    """Names of the functions include/moe.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:moe|qb)_\w+)\s*\(", text)))


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        L = lib()
        msg = L.moe_last_error().decode()
        super().__init__(f"{where}: {L.moe_status_string(status).decode()}: {msg}")
        self.status = status


def check(status: int, where: str) -> None:
    if status != MOE_OK:
        raise MoeError(status, where)


# ---------------------------------------------------------------- wrappers --
# Same names as the C functions; plain integers stand for device pointers and
# the stream (a hipStream_t handle, e.g. torch.cuda.current_stream().cuda_stream).

def moe_state_bytes(cfg: moe_config) -> int:
    return lib().moe_state_bytes(ctypes.byref(cfg))


def moe_workspace_bytes(cfg: moe_config, T: int) -> int:
    return lib().moe_workspace_bytes(ctypes.byref(cfg), T)


def moe_state_layout_of(cfg: moe_config) -> moe_state_layout:
    out = moe_state_layout()
    check(lib().moe_state_layout_of(ctypes.byref(cfg), ctypes.byref(out)), "moe_state_layout_of")
    return out


def moe_workspace_layout(cfg: moe_config, T: int) -> moe_ws_layout:
    out = moe_ws_layout()
    check(lib().moe_workspace_layout(ctypes.byref(cfg), T, ctypes.byref(out)), "moe_workspace_layout")
    return out


def moe_init(cfg: moe_config, w: moe_weights, state: int, stream: int) -> int:
    ctx = c_void_p()
    check(lib().moe_init(ctypes.byref(cfg), ctypes.byref(w), state, stream, ctypes.byref(ctx)), "moe_init")
    return ctx.value


def moe_route(ctx: int, x: Optional[int], logits: Optional[int], T: int, r: Optional[moe_route_out], ws: int,
              ws_bytes: int, stream: int) -> None:
    check(lib().moe_route(ctx, x, logits, T, ctypes.byref(r) if r is not None else None, ws, ws_bytes, stream),
          "moe_route")


def moe_forward(ctx: int, x: int, T: int, out: int, r: Optional[moe_route_out], ws: int, ws_bytes: int,
                stream: int) -> None:
    check(lib().moe_forward(ctx, x, T, out, ctypes.byref(r) if r is not None else None, ws, ws_bytes, stream),
          "moe_forward")


MOE_NOALLOC_SCRATCH_BYTES = 160 << 20
MOE_FAST_SCORE_ERR = 2.0 ** -20  # bound on |fast - exact| router score that the routing kernels rely on


def moe_forward_noalloc(ctx: int, x: int, T: int, out: int, r: Optional[moe_route_out], stream: int) -> None:
    check(lib().moe_forward_noalloc(ctx, x, T, out, ctypes.byref(r) if r is not None else None, stream),
          "moe_forward_noalloc")


def moe_backward_workspace_bytes(cfg: moe_config, T: int) -> int:
    return lib().moe_backward_workspace_bytes(ctypes.byref(cfg), T)


def moe_backward(ctx: int, x: int, dout: int, T: int, r: Optional[moe_route_out], fwd_ws: int, fwd_ws_bytes: int,
                 dx: int, g: moe_grads, ws: int, ws_bytes: int, stream: int) -> None:
    check(lib().moe_backward(ctx, x, dout, T, ctypes.byref(r) if r is not None else None, fwd_ws, fwd_ws_bytes, dx,
                             ctypes.byref(g), ws, ws_bytes, stream), "moe_backward")


def moe_requantize_experts(ctx: int, stream: int) -> None:
    check(lib().moe_requantize_experts(ctx, stream), "moe_requantize_experts")


def qb_update(ctx: int, stream: int) -> None:
    check(lib().qb_update(ctx, stream), "qb_update")


def moe_fast_score_error(err: int, stream: int) -> None:
    check(lib().moe_fast_score_error(err, stream), "moe_fast_score_error")


def moe_get_bias(ctx: int, dst: int, stream: int) -> None:
    check(lib().moe_get_bias(ctx, dst, stream), "moe_get_bias")


def moe_set_bias(ctx: int, src: int, stream: int) -> None:
    check(lib().moe_set_bias(ctx, src, stream), "moe_set_bias")


def moe_set_qb_mode(ctx: int, mode: int) -> None:
    check(lib().moe_set_qb_mode(ctx, mode), "moe_set_qb_mode")


def moe_destroy(ctx: int) -> None:
    lib().moe_destroy(ctx)


def moe_profile_begin(ctx: int, max_launches: int, kernels=None) -> None:
    """Time the launches of the named kernels (all when None)."""
    mask = 0 if not kernels else sum(1 << KERNELS.index(k) for k in kernels)
    check(lib().moe_profile_begin(ctx, max_launches, mask), "moe_profile_begin")


def moe_profile_end(ctx: int) -> Dict[str, tuple]:
    """{kernel name: (total ms, launches)} for the launches since begin."""
    ms = (c_double * MOE_NUM_KERNELS)()
    n = (c_int64 * MOE_NUM_KERNELS)()
    check(lib().moe_profile_end(ctx, ms, n, MOE_NUM_KERNELS), "moe_profile_end")
    return {KERNELS[i]: (ms[i], n[i]) for i in range(MOE_NUM_KERNELS)}


def make_config(d: int, l: int, E: int, k: int, f: int, f_s: int, *, n_shared: int = 1, dtype: str = "bf16",
                rms_eps: float = 1e-6, qb_bins: int = 256, qb_lo: float = 0.0, qb_hi: float = 1.0,
                frozen: bool = False, max_tokens: int = 1, routed_scale: float = 1.0, balancer: str = "qb",
                sign_gamma: float = 1e-2, experts: str = "bf16", keep_preact: bool = False) -> moe_config:
    """f_s is the hidden width of each of the n_shared shared experts."""
    return moe_config(d=d, l=l, E=E, k=k, f=f, f_s=f_s, n_shared=n_shared,
                      dtype=MOE_BF16 if dtype == "bf16" else MOE_F32, rms_eps=rms_eps, qb_bins=qb_bins,
                      qb_lo=qb_lo, qb_hi=qb_hi, qb_mode=MOE_QB_FROZEN if frozen else MOE_QB_TRAIN,
                      max_tokens=max_tokens, routed_scale=routed_scale,
                      balancer=MOE_BALANCE_SIGN if balancer == "sign" else MOE_BALANCE_QB, sign_gamma=sign_gamma,
                      experts=_EXPERT_FORMATS[experts],
                      keep_preact=1 if keep_preact else 0)
