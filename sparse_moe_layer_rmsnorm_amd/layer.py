"""PyTorch-side holder of one layer: device buffers (weights, QB state,
workspace) allocated with torch, and the C context.  Every computation runs in
libmoe.so through the C ABI; this class only allocates and marshals."""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np
import torch

from . import binding as B

_WEIGHT_NAMES = ("W_r", "W_sg", "W_su", "W_sd", "W_dn", "W_g", "W_u", "W_d", "W_up")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _sync(stream) -> None:
    """Wait for the stream a call was enqueued on (torch stream, raw handle or None)."""
    if stream is None:
        torch.cuda.current_stream().synchronize()
    elif hasattr(stream, "synchronize"):
        stream.synchronize()
    else:
        torch.cuda.ExternalStream(int(stream)).synchronize()


class MoeLayer:
    """One Stable LatentMoE layer on a GPU.

    ``weights`` maps the names of ``moe_weights`` to numpy arrays (or torch
    tensors) holding values of the storage dtype; ``logit_offset`` is the
    optional per-expert router offset.  ``f_s`` is the hidden width of each
    of the ``n_shared`` shared experts, whose weights are stacked along the
    hidden axis (W_sg, W_su [n_shared*f_s, d], W_sd [d, n_shared*f_s]).
    """

    def __init__(self, *, d: int, l: int, E: int, k: int, f: int, f_s: int, dtype: str, weights: Dict,
                 max_tokens: int, qb_bins: int = 256, rms_eps: float = 1e-6, frozen: bool = False,
                 routed_scale: float = 1.0, logit_offset=None, device: str = "cuda", stream=None,
                 balancer: str = "qb", sign_gamma: float = 1e-2, experts: str = "bf16", keep_preact: bool = False,
                 n_shared: int = 1, qb_lo: float = 0.0, qb_hi: float = 1.0):
        self.dtype = dtype
        self.tdtype = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.device = torch.device(device)
        self.cfg = B.make_config(d, l, E, k, f, f_s, n_shared=n_shared, dtype=dtype, rms_eps=rms_eps,
                                 qb_bins=qb_bins, qb_lo=qb_lo, qb_hi=qb_hi, frozen=frozen, max_tokens=max_tokens,
                                 routed_scale=routed_scale, balancer=balancer, sign_gamma=sign_gamma,
                                 experts=experts, keep_preact=keep_preact)
        f_s = n_shared * f_s                              # hidden width of the whole shared path
        self.dims = dict(d=d, l=l, E=E, k=k, f=f, f_s=f_s, B=qb_bins)
        self.w: Dict[str, torch.Tensor] = {}
        for name in _WEIGHT_NAMES:
            if name in ("W_sg", "W_su", "W_sd") and f_s == 0:
                continue
            self.w[name] = self._dev(weights[name], self.tdtype)
        self.w["gamma"] = self._dev(weights["gamma"], torch.float32)
        if logit_offset is not None:
            self.w["logit_offset"] = self._dev(logit_offset, torch.float32)
        self.state = torch.zeros(B.moe_state_bytes(self.cfg), dtype=torch.uint8, device=self.device)
        self.sl = B.moe_state_layout_of(self.cfg)
        mw = B.moe_weights(**{n: _ptr(self.w.get(n)) for n in ("gamma", "W_r", "logit_offset", "W_sg", "W_su",
                                                                "W_sd", "W_dn", "W_g", "W_u", "W_d", "W_up")})
        self.ctx = B.moe_init(self.cfg, mw, self.state.data_ptr(), _stream(stream))
        self._ws: Optional[torch.Tensor] = None

    def _dev(self, a, dt) -> torch.Tensor:
        t = a if isinstance(a, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(a))
        return t.to(self.device).to(dt).contiguous()

    # ------------------------------------------------------------ buffers --
    def workspace(self, T: int) -> torch.Tensor:
        need = B.moe_workspace_bytes(self.cfg, T)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.device)
        return self._ws

    def ws_views(self, T: int) -> Dict[str, torch.Tensor]:
        """Views of the intermediates of the last call with T tokens."""
        L = B.moe_workspace_layout(self.cfg, T)
        ws = self.workspace(T)
        dm = self.dims
        es = self.tdtype
        keep = int(self.cfg.keep_preact)

        def view(off, n, dt, shape):
            nbytes = n * torch.tensor([], dtype=dt).element_size()
            return ws[off:off + nbytes].view(dt).view(*shape)

        return {
            "h": view(L.h, T * dm["d"], es, (T, dm["d"])),
            "logits": view(L.logits, T * dm["E"], torch.float32, (T, dm["E"])),
            "G": view(L.G, T * dm["f_s"], es, (T, dm["f_s"])),
            "z": view(L.z, T * dm["l"], es, (T, dm["l"])),
            # H: empty when the experts ran fused (the hidden never left the chip)
            "H": view(L.H, T * dm["k"] * dm["f"] if L.Y > L.H else 0, es, (-1, dm["f"])),
            "Y": view(L.Y, T * dm["k"] * dm["l"], es, (T * dm["k"], dm["l"])),
            "y_lat": view(L.y_lat, T * dm["l"], es, (T, dm["l"])),
            "tile_offsets": view(L.tile_offsets, dm["E"] + 1, torch.int32, (dm["E"] + 1,)),
            # block-scaled experts only (empty otherwise): E4M3 bytes and E8M0 scales of z and H
            "z8": view(L.z8, L.zs - L.z8, torch.uint8, (-1,)),
            "zs": view(L.zs, L.Xs - L.zs, torch.uint8, (-1,)),
            "H8": view(L.H8, L.Hs - L.H8, torch.uint8, (-1,)),
            "Hs": view(L.Hs, L.P - L.Hs, torch.uint8, (-1,)),
            # keep_preact only (empty otherwise): the GLU pre-activations
            "P": view(L.P, keep * T * dm["f_s"], es, (-1, dm["f_s"]) if keep else (0,)),
            "Q": view(L.Q, keep * T * dm["f_s"], es, (-1, dm["f_s"]) if keep else (0,)),
            "A": view(L.A, keep * T * dm["k"] * dm["f"], es, (-1, dm["f"]) if keep else (0,)),
            "U": view(L.U, keep * T * dm["k"] * dm["f"], es, (-1, dm["f"]) if keep else (0,)),
        }

    def state_views(self) -> Dict[str, torch.Tensor]:
        E, nb, S = self.dims["E"], self.dims["B"], self.sl.hist_slices
        s = self.state
        return {
            "bias": s[self.sl.bias:self.sl.bias + 4 * E].view(torch.float32),
            "count": s[self.sl.count:self.sl.count + 8].view(torch.int64),
            "q": s[self.sl.q:self.sl.q + 8 * E].view(torch.float64),
            "hist_slices": s[self.sl.hist:self.sl.hist + 4 * S * E * nb].view(torch.int32).view(S, E, nb),
            "hist": s[self.sl.hist:self.sl.hist + 4 * S * E * nb].view(torch.int32).view(S, E, nb).sum(0),
            "load": s[self.sl.load:self.sl.load + 4 * E].view(torch.int32),
        }

    def route_buffers(self, T: int) -> Dict[str, torch.Tensor]:
        dm = self.dims
        z = lambda *s, dt=torch.int32: torch.empty(*s, dtype=dt, device=self.device)  # noqa: E731
        return {"logits": z(T, dm["E"], dt=torch.float32), "topk_idx": z(T, dm["k"]),
                "gates": z(T, dm["k"], dt=torch.float32), "counts": z(dm["E"]), "offsets": z(dm["E"] + 1),
                "perm_src": z(T * dm["k"]), "inv": z(T, dm["k"])}

    @staticmethod
    def _route_struct(r: Optional[Dict[str, torch.Tensor]]) -> Optional[B.moe_route_out]:
        if r is None:
            return None
        return B.moe_route_out(**{n: _ptr(r.get(n)) for n in ("logits", "topk_idx", "gates", "counts", "offsets",
                                                               "perm_src", "inv")})

    # -------------------------------------------------------------- calls --
    def forward(self, x: torch.Tensor, out: Optional[torch.Tensor] = None,
                route: Optional[Dict[str, torch.Tensor]] = None, stream=None) -> torch.Tensor:
        T = x.shape[0]
        if out is None:
            out = torch.empty(T, self.dims["d"], dtype=self.tdtype, device=self.device)
        ws = self.workspace(T)
        B.moe_forward(self.ctx, x.data_ptr(), T, out.data_ptr(), self._route_struct(route), ws.data_ptr(),
                      ws.numel(), _stream(stream))
        return out

    def route(self, T: int, x: Optional[torch.Tensor] = None, logits: Optional[torch.Tensor] = None,
              route: Optional[Dict[str, torch.Tensor]] = None, stream=None) -> Dict[str, torch.Tensor]:
        if route is None:
            route = self.route_buffers(T)
        ws = self.workspace(T)
        B.moe_route(self.ctx, _ptr(x), _ptr(logits), T, self._route_struct(route), ws.data_ptr(), ws.numel(),
                    _stream(stream))
        return route

    def backward(self, x: torch.Tensor, dout: torch.Tensor, route: Optional[Dict[str, torch.Tensor]] = None,
                 grads: Optional[Dict[str, torch.Tensor]] = None, stream=None):
        """Gradients for the last forward(x, route=route): returns (dx, grads),
        grads fp32 tensors keyed like the weights (plus "gamma")."""
        T = x.shape[0]
        dm = self.dims
        if grads is None:
            shapes = {"gamma": (dm["d"],), "W_r": (dm["E"], dm["d"]), "W_sg": (dm["f_s"], dm["d"]),
                      "W_su": (dm["f_s"], dm["d"]), "W_sd": (dm["d"], dm["f_s"]), "W_dn": (dm["l"], dm["d"]),
                      "W_g": (dm["E"], dm["f"], dm["l"]), "W_u": (dm["E"], dm["f"], dm["l"]),
                      "W_d": (dm["E"], dm["l"], dm["f"]), "W_up": (dm["d"], dm["l"])}
            grads = {n: torch.empty(*sh, dtype=torch.float32, device=self.device) for n, sh in shapes.items()
                     if not (n in ("W_sg", "W_su", "W_sd") and dm["f_s"] == 0)}
        dx = torch.empty_like(x)
        fws = self.workspace(T)
        need = B.moe_backward_workspace_bytes(self.cfg, T)
        if getattr(self, "_bws", None) is None or self._bws.numel() < need:
            self._bws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.device)
        g = B.moe_grads(**{n: _ptr(grads.get(n)) for n in ("gamma", "W_r", "W_sg", "W_su", "W_sd", "W_dn", "W_g",
                                                            "W_u", "W_d", "W_up")})
        B.moe_backward(self.ctx, x.data_ptr(), dout.data_ptr(), T, self._route_struct(route), fws.data_ptr(),
                       fws.numel(), dx.data_ptr(), g, self._bws.data_ptr(), self._bws.numel(), _stream(stream))
        return dx, grads

    def qb_update(self, stream=None) -> None:
        B.qb_update(self.ctx, _stream(stream))

    def get_bias(self, stream=None) -> torch.Tensor:
        out = torch.empty(self.dims["E"], dtype=torch.float32, device=self.device)
        B.moe_get_bias(self.ctx, out.data_ptr(), _stream(stream))
        return out

    def set_bias(self, b, stream=None) -> None:
        t = self._dev(b, torch.float32)                  # written on the current stream
        torch.cuda.current_stream().synchronize()         # ... and complete before another stream reads it
        B.moe_set_bias(self.ctx, t.data_ptr(), _stream(stream))
        _sync(stream)                                     # the copy has read t before t is freed

    def set_qb_mode(self, frozen: bool) -> None:
        B.moe_set_qb_mode(self.ctx, B.MOE_QB_FROZEN if frozen else B.MOE_QB_TRAIN)

    def close(self) -> None:
        if getattr(self, "ctx", None):
            B.moe_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def layer_from_shape(shape, weights: Dict, *, max_tokens: Optional[int] = None, frozen: Optional[bool] = None,
                     logit_offset=None, device: str = "cuda", balancer: str = "qb",
                     sign_gamma: float = 1e-2, experts: str = "bf16", keep_preact: bool = False,
                     n_shared: int = 1, qb_lo: float = 0.0, qb_hi: float = 1.0) -> MoeLayer:
    """MoeLayer for a workloads.LayerShape (shape.f_s: the whole shared hidden,
    split over n_shared experts of shape.f_s / n_shared each)."""
    assert shape.f_s % max(n_shared, 1) == 0
    return MoeLayer(d=shape.d, l=shape.l, E=shape.E, k=shape.k, f=shape.f,
                    f_s=shape.f_s // n_shared if n_shared > 0 else 0, n_shared=n_shared, dtype=shape.dtype,
                    weights=weights, max_tokens=max_tokens or shape.T, qb_bins=shape.B, rms_eps=shape.rms_eps,
                    frozen=shape.qb_frozen if frozen is None else frozen, logit_offset=logit_offset,
                    device=device, balancer=balancer, sign_gamma=sign_gamma, experts=experts,
                    keep_preact=keep_preact, qb_lo=qb_lo, qb_hi=qb_hi)
