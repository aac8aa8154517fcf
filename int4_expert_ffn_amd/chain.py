"""Host-side schedule of a prerouted decode stack: L MoE layers resident on one GPU.

Per token t and layer l (all calls asynchronous on one stream, routing never leaves the device):
  * layer 0, and every layer at the first token, runs its own router + softmax top-K;
    any other layer uses the set and weights the head of layer l-1 predicted at token t-1
    (the prediction is the routing: "La otra mitad del muro de la memoria: Servir MoEs de 35B
    desde SSD ...", section "Ideas clave");
  * the head of layer l (l < L-1) reads the layer input with the K-hot routing of layer l at
    tokens t and t-1 and predicts layer l+1's routing for token t+1 (section "Arquitectura del
    cabezal Prerouter");
  * the expert FFN with the fused weighted combine + residual produces the next layer's input.
Layer inputs are consumed through an RMS norm: the weightless one fused into every call
(MOE_INPUT_RMSNORM), or, for a stack whose layers carry norm gains, moe_rmsnorm before the
layer's calls (the persistent kernel applies the gain inside); the residual is the un-normalised
float16 hidden state.

Routing buffers rotate over three token slots, so the head writing token t+1's routing never
overwrites what token t still reads (slot t%3) or the previous-token vector (slot (t-1)%3).

Two ways to run a token: `token()` issues the per-layer C-ABI calls (5 launches per layer);
`step()` issues one moe_decode_step launch, the persistent kernel that runs the same schedule
with all layers in one kernel.  Both share the routing state, so they can be mixed token by token.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional

import torch

from . import _lib as L


@dataclass
class LayerWeights:
    experts: L.Experts
    router: torch.Tensor                      # [E][d] float16
    head: Optional[L.PrerouterWeights] = None  # predicts the next layer; None on the last layer
    norm_gain: Optional[torch.Tensor] = None   # [d] float16 gain of the input norm (all layers or none)


class DecodeStack:
    def __init__(self, layers: List[LayerWeights], K: int, device, renorm: bool = True):
        ex0 = layers[0].experts
        gained = [lw.norm_gain is not None for lw in layers]
        if any(gained) and not all(gained):
            raise ValueError("norm gains must be given for every layer or for none")
        self.gained = all(gained)
        self.layers = layers
        self.L = len(layers)
        self.E, self.d, self.K = ex0.E, ex0.d, K
        self.device = torch.device(device)
        self.topk_flags = L.MOE_TOPK_RENORM if renorm else 0
        dev = self.device
        E, d = self.E, self.d
        self.route_idx = torch.zeros((3, self.L, K), dtype=torch.int32, device=dev)
        self.route_w = torch.zeros((3, self.L, K), dtype=torch.float32, device=dev)
        self.logits = torch.zeros((self.L, E), dtype=torch.float32, device=dev)
        self.head_logits = torch.zeros((self.L, E), dtype=torch.float32, device=dev)
        self.h = torch.zeros((self.L + 1, d), dtype=torch.float16, device=dev)   # per-layer inputs/outputs
        self.xn = torch.zeros(d, dtype=torch.float16, device=dev)                # gained normalised input
        ffn_ws = max(L.moe_expert_ffn_workspace_size(1, K, lw.experts) for lw in layers)
        H = max([lw.head.H for lw in layers if lw.head is not None] or [8])
        head_ws = L.moe_prerouter_workspace_size(1, E, H)
        self.ffn_ws = torch.empty(ffn_ws, dtype=torch.uint8, device=dev)
        self.head_ws = torch.empty(head_ws, dtype=torch.uint8, device=dev)
        self._step = None

    # ------------------------------------------------------------------ persistent whole-token kernel
    def _step_state(self):
        """Device array of layer descriptors, the stack descriptor and the zeroed step workspace."""
        if self._step is None:
            L_ = self.L
            arr = (L.moe_decode_layer * L_)()
            H = 0
            for l, lw in enumerate(self.layers):
                arr[l].experts = lw.experts.desc
                arr[l].router = lw.router.data_ptr()
                if lw.head is not None and l + 1 < L_:
                    arr[l].head = lw.head.desc
                    H = lw.head.H
                if lw.norm_gain is not None:
                    arr[l].norm_gain = lw.norm_gain.data_ptr()
            raw = bytes(arr)
            desc = torch.frombuffer(bytearray(raw), dtype=torch.uint8).to(self.device)
            ex0 = self.layers[0].experts
            st = L.moe_decode_stack(L_, self.E, self.K, self.d, ex0.I, ex0.bits, ex0.group, H, desc.data_ptr(),
                                    self.route_idx.data_ptr(), self.route_w.data_ptr(), 1 if self.gained else 0)
            ws = torch.zeros(L.moe_decode_workspace_size(st), dtype=torch.uint8, device=self.device)
            self._step = (desc, st, ws)
        return self._step

    def step(self, t: int, h_in: torch.Tensor, h_out: Optional[torch.Tensor] = None,
             h_layers: Optional[torch.Tensor] = None, given_routing: bool = False,
             stamps: Optional[torch.Tensor] = None):
        """Enqueue token t as one persistent-kernel launch reading h_in [d] and writing h_out
        (default: self.h[L]); h_layers [L+1][d] float16, if given, receives every layer's input and
        the output.  given_routing: the expert FFN steps alone, every layer routed by what the
        caller wrote into route_idx / route_w slot t % 3 (see set_routing).  stamps: an int64
        tensor [G][L][16] (G = grid()) that receives the kernel's phase stamps.  Returns h_out."""
        desc, st, ws = self._step_state()
        out = self.h[self.L] if h_out is None else h_out
        flags = self.topk_flags | (L.MOE_DECODE_GIVEN_ROUTING if given_routing else 0)
        if stamps is None:
            L.moe_decode_step(st, t, flags, h_in, out, ws, h_layers=h_layers)
        else:
            L.moe_decode_step_stamped(st, t, flags, h_in, out, stamps, ws, h_layers=h_layers)
        return out

    def grid(self) -> int:
        """Workgroups of one persistent-kernel launch of this stack (0: not supported)."""
        return L.moe_decode_step_grid(self._step_state()[1])

    def set_routing(self, t: int, idx: torch.Tensor, w: torch.Tensor):
        """Write every layer's experts idx [L][K] (int32, distinct per layer, in [0, E)) and weights
        w [L][K] (float32) into the routing slot of token t (asynchronous, on the current stream)."""
        if tuple(idx.shape) != (self.L, self.K) or tuple(w.shape) != (self.L, self.K):
            raise ValueError(f"routing must be [{self.L}][{self.K}]")
        i64 = idx.to(torch.int64)
        if bool(((i64 < 0) | (i64 >= self.E)).any()):
            raise ValueError("expert index outside [0, E)")
        self.route_idx[t % 3].copy_(idx.to(torch.int32))
        self.route_w[t % 3].copy_(w.to(torch.float32))

    def step_error_word(self) -> int:
        """Nonzero if a wait inside a persistent-kernel step exceeded its bound (read after sync)."""
        _, _, ws = self._step_state()
        return int(ws[4:8].view(torch.int32).item())

    def token(self, t: int, h_in: Optional[torch.Tensor] = None, record_routing: bool = False):
        """Enqueue token t.  h_in [d] float16 is copied into the stack input unless None (then the
        caller has already written self.h[0]).  Returns the output view self.h[L]."""
        if h_in is not None:
            self.h[0].copy_(h_in)
        s, sp, sn = t % 3, (t - 1) % 3, (t + 1) % 3
        for l, lw in enumerate(self.layers):
            h = self.h[l]
            if lw.norm_gain is not None:      # x = g * h / rms(h), then the calls take x as it is
                L.moe_rmsnorm(1, self.d, h, lw.norm_gain, self.xn)
                x, RMS = self.xn, 0
            else:                             # the calls normalise h themselves
                x, RMS = h, L.MOE_INPUT_RMSNORM
            idx, w = self.route_idx[s, l], self.route_w[s, l]
            # a layer routes itself unless the head of the layer before predicted it one token ago
            if l == 0 or t == 0 or self.layers[l - 1].head is None:
                L.moe_route_topk(1, self.d, self.E, self.K, self.topk_flags | RMS, x, lw.router,
                                 self.logits[l], idx, w)
            if lw.head is not None and l + 1 < self.L:
                L.moe_prerouter(1, self.d, self.E, self.K, RMS, x, idx, self.route_idx[sp, l] if t > 0 else None,
                                lw.head, self.head_logits[l], self.head_ws)
                L.moe_route_topk(1, self.d, self.E, self.K, self.topk_flags, None, None, self.head_logits[l],
                                 self.route_idx[sn, l + 1], self.route_w[sn, l + 1])
            L.moe_expert_ffn_q4(1, self.K, RMS, x, idx, lw.experts, None, None, w, h, self.h[l + 1],
                                self.ffn_ws)
        return self.h[self.L]
