"""Device-side set-up of one MoE layer: descriptor, packed weights, streams.

Plumbing only: torch allocates device memory and streams, the HIP library
(through :mod:`.binding`) packs the weights and runs every step of the layer.
Weights are drawn per expert by :mod:`.inputs`, uploaded in batches and
packed on the device, so the host never holds more than one batch.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as B
from . import inputs as I

_DT = {"f32": (B.MOE_F32, B.MOE_F32, B.MOE_F32),
       "bf16": (B.MOE_BF16, B.MOE_BF16, B.MOE_BF16),
       "mxfp8": (B.MOE_BF16, B.MOE_MXFP8, B.MOE_BF16),
       # W4A8: MXFP4 routed experts, MX-fp8 shared expert and activations
       "w4a8": (B.MOE_BF16, B.MOE_MXFP4, B.MOE_BF16),
       # static per-tensor FP8 W8A8
       "fp8": (B.MOE_BF16, B.MOE_FP8, B.MOE_BF16)}


def desc_for(w: I.Workload) -> B.MoeDesc:
    a, e, o = _DT[w.dtype]
    return B.MoeDesc(hidden=w.H, num_experts=w.E, top_k=w.k, inter=w.I, shared_inter=w.Is,
                     router_scaling_factor=w.rho, route_norm=int(w.route_norm), act_dtype=a,
                     expert_dtype=e, out_dtype=o, fp8_x_scale=w.fp8_x_scale,
                     fp8_h_scale=w.fp8_h_scale, fp8_sh_h_scale=w.fp8_sh_h_scale)


def torch_dtype(moe_dtype: int):
    return torch.float32 if moe_dtype == B.MOE_F32 else torch.bfloat16


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    """numpy -> device tensor; uint16 arrays are bf16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.to(device)


class DeviceLayer:
    """Packed weights and router of one workload on one GPU."""

    def __init__(self, w: I.Workload, device: int = 0, batch: int = 16, side_stream=True,
                 expert_fn=None, shared_fn=None, router=None):
        self.w = w
        self.dev = torch.device("cuda", device)
        self.desc = desc_for(w)
        d = self.desc
        u8 = torch.uint8
        nb = lambda shared, which: B.moe_packed_bytes(d, shared, which)
        self.gate_up = torch.empty(nb(0, B.MOE_PACK_GATE_UP), dtype=u8, device=self.dev)
        self.down = torch.empty(nb(0, B.MOE_PACK_DOWN), dtype=u8, device=self.dev)
        mx = w.dtype in ("mxfp8", "w4a8", "fp8")     # scale arrays
        self.gate_up_s = torch.empty(nb(0, B.MOE_PACK_GATE_UP_SCALE), dtype=u8, device=self.dev) if mx else None
        self.down_s = torch.empty(nb(0, B.MOE_PACK_DOWN_SCALE), dtype=u8, device=self.dev) if mx else None
        self.sh_gate_up = torch.empty(nb(1, B.MOE_PACK_GATE_UP), dtype=u8, device=self.dev)
        self.sh_down = torch.empty(nb(1, B.MOE_PACK_DOWN), dtype=u8, device=self.dev)
        self.sh_gate_up_s = torch.empty(nb(1, B.MOE_PACK_GATE_UP_SCALE), dtype=u8, device=self.dev) if mx else None
        self.sh_down_s = torch.empty(nb(1, B.MOE_PACK_DOWN_SCALE), dtype=u8, device=self.dev) if mx else None

        expert_fn = expert_fn or (lambda e: I.expert_stored(w, e))
        shared_fn = shared_fn or (lambda: I.shared_stored(w))
        if router is None:
            router = (I.router_weight(w), I.router_bias(w))
        self.router_w = to_device(router[0], self.dev)
        self.router_b = None if router[1] is None else to_device(router[1], self.dev)
        src_dt = B.MOE_BF16 if w.dtype == "bf16" else B.MOE_F32
        self._pack_routed(expert_fn, batch, src_dt)
        if w.Is > 0:
            g, u, dn = (to_device(a, self.dev) for a in shared_fn())
            B.moe_pack_experts(d, 1, src_dt, g, u, dn, self.sh_gate_up, self.sh_down,
                               self.sh_gate_up_s, self.sh_down_s)
        torch.cuda.synchronize(self.dev)

        self.weights = B.MoeWeights(
            router_w=self.router_w.data_ptr(),
            router_bias=None if self.router_b is None else self.router_b.data_ptr(),
            gate_up=self.gate_up.data_ptr(), down=self.down.data_ptr(),
            gate_up_scale=None if self.gate_up_s is None else self.gate_up_s.data_ptr(),
            down_scale=None if self.down_s is None else self.down_s.data_ptr(),
            sh_gate_up=self.sh_gate_up.data_ptr() if w.Is else None,
            sh_down=self.sh_down.data_ptr() if w.Is else None,
            sh_gate_up_scale=None if self.sh_gate_up_s is None else self.sh_gate_up_s.data_ptr(),
            sh_down_scale=None if self.sh_down_s is None else self.sh_down_s.data_ptr())
        self.side = torch.cuda.Stream(device=self.dev) if side_stream else None
        self.ctx = B.moe_ctx_create(device, self.side)
        self._ws = {}

    def _pack_routed(self, expert_fn, batch, src_dt):
        from concurrent.futures import ThreadPoolExecutor
        w, d = self.w, self.desc
        per_gu = self.gate_up.numel() // w.E
        per_dn = self.down.numel() // w.E
        per_gus = 0 if self.gate_up_s is None else self.gate_up_s.numel() // w.E
        per_dns = 0 if self.down_s is None else self.down_s.numel() // w.E
        with ThreadPoolExecutor(max_workers=16) as ex:
            for e0 in range(0, w.E, batch):
                e1 = min(w.E, e0 + batch)
                parts = list(ex.map(expert_fn, range(e0, e1)))
                g = to_device(np.stack([p[0] for p in parts]), self.dev)
                u = to_device(np.stack([p[1] for p in parts]), self.dev)
                dn = to_device(np.stack([p[2] for p in parts]), self.dev)
                sub = B.MoeDesc.from_buffer_copy(d)
                sub.num_experts = e1 - e0
                sub.top_k = min(sub.top_k, sub.num_experts)
                gs = None if self.gate_up_s is None else self.gate_up_s[e0 * per_gus:]
                ds = None if self.down_s is None else self.down_s[e0 * per_dns:]
                B.moe_pack_experts(sub, 0, src_dt, g, u, dn, self.gate_up[e0 * per_gu:],
                                   self.down[e0 * per_dn:], gs, ds)
                torch.cuda.synchronize(self.dev)

    def workspace(self, T: int, which: int = B.MOE_WS_LAYER):
        key = (T, which)
        if key not in self._ws:
            n = B.moe_workspace_bytes(self.desc, T, which)
            self._ws[key] = torch.empty(max(n, 256), dtype=torch.uint8, device=self.dev)
        return self._ws[key]

    def out_dtype(self):
        return torch_dtype(self.desc.out_dtype)

    def forward(self, x: torch.Tensor, out: torch.Tensor = None, stream=None) -> torch.Tensor:
        T = x.shape[0]
        if out is None:
            out = torch.empty((T, self.w.H), dtype=self.out_dtype(), device=self.dev)
        ws = self.workspace(T)
        s = stream if stream is not None else torch.cuda.current_stream(self.dev)
        B.moe_layer_forward(self.ctx, self.desc, self.weights, x, T, out, ws, ws.numel(), s)
        return out

    def capture(self, x: torch.Tensor, out: torch.Tensor):
        """Record one forward of the layer (x -> out, this layer's workspace)
        as a HIP graph and return it; ``graph.replay()`` runs the same kernels
        again on whatever x holds then.  The side stream joins the capture at
        the input-ready event and leaves it at the shared-done event, as in an
        eager call, so the graph keeps the two-stream schedule.  Nothing in
        the forward path allocates, clears memory or synchronizes, which is
        what capture requires."""
        T = x.shape[0]
        ws = self.workspace(T)
        torch.cuda.synchronize(self.dev)
        g = torch.cuda.CUDAGraph()
        cs = torch.cuda.Stream(device=self.dev)
        with torch.cuda.graph(g, stream=cs):
            B.moe_layer_forward(self.ctx, self.desc, self.weights, x, T, out, ws, ws.numel(), cs)
        torch.cuda.synchronize(self.dev)
        return g

    def close(self):
        if self.ctx:
            torch.cuda.synchronize(self.dev)
            B.moe_ctx_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
