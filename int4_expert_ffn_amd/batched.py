"""Host-side schedule of the batched MoE layer: T tokens per call.

  router + softmax top-K -> routed experts (tokens sorted by expert, grouped MFMA GEMMs)
  shared expert with its unmerged LoRA ("La otra mitad del muro de la memoria ...", section
      "Ejecucion del adaptador no fusionado": y = W_int4 x + (alpha/r) B A x)
  combine: y = r + sum_k w_k o_k + shared

By default the shared expert runs inside the routed experts' call (moe_expert_ffn_q4_shared): its
T rows join the (token, slot) pairs as one more expert of the sort, so one grouped GEMM launch per
projection covers both and the combine adds its output.  separate=True keeps the earlier schedule:
the shared expert as its own moe_expert_ffn_q4 call, on a second stream beside the router, top-K and
routed experts (two_streams) or after them, then moe_combine.  Every step is a C-ABI call into
libmoe.so; this module only allocates the buffers and orders the calls.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _lib as L


class BatchedLayer:
    def __init__(self, experts: L.Experts, router: torch.Tensor, T: int, K: int, device,
                 shared: Optional[L.Experts] = None, lora3: Optional[L.Lora3] = None, renorm: bool = True,
                 two_streams: bool = True, separate: bool = False):
        dev = torch.device(device)
        self.ex, self.router, self.shared, self.lora3 = experts, router, shared, lora3
        self.T, self.K, self.E, self.d = T, K, experts.E, experts.d
        self.flags = L.MOE_TOPK_RENORM if renorm else 0
        self.logits = torch.empty((T, self.E), dtype=torch.float32, device=dev)
        self.idx = torch.empty((T, K), dtype=torch.int32, device=dev)
        self.w = torch.empty((T, K), dtype=torch.float32, device=dev)
        self.o = torch.empty((T, K, self.d), dtype=torch.float32, device=dev)
        self.merged = shared is not None and not separate and T >= 32
        nws = (L.moe_expert_ffn_shared_workspace_size(T, K, experts) if self.merged
               else L.moe_expert_ffn_workspace_size(T, K, experts))
        self.ws = torch.empty(nws, dtype=torch.uint8, device=dev)
        if shared is not None and not self.merged:
            self.sho = torch.empty((T, 1, self.d), dtype=torch.float32, device=dev)
            self.zeros = torch.zeros((T, 1), dtype=torch.int32, device=dev)
            self.ws_sh = torch.empty(L.moe_expert_ffn_workspace_size(T, 1, shared), dtype=torch.uint8, device=dev)
        self.side = torch.cuda.Stream(device=dev) if (two_streams and shared is not None and not self.merged) else None

    def _shared(self, h):
        L.moe_expert_ffn_q4(self.T, 1, 0, h, self.zeros, self.shared, self.lora3, self.sho, None, None, None,
                            self.ws_sh)

    def __call__(self, h: torch.Tensor, y: torch.Tensor) -> torch.Tensor:
        """Enqueue the layer for h [T][d] float16 into y [T][d] float16 (the residual is h)."""
        if self.merged:
            L.moe_route_topk(self.T, self.d, self.E, self.K, self.flags, h, self.router, self.logits, self.idx,
                             self.w)
            L.moe_expert_ffn_q4_shared(self.T, self.K, 0, h, self.idx, self.ex, self.shared, self.lora3, self.w, h, y,
                                       self.ws)
            return y
        cs = torch.cuda.current_stream(h.device)
        if self.side is not None:
            self.side.wait_stream(cs)
            with torch.cuda.stream(self.side):
                self._shared(h)
        elif self.shared is not None:
            self._shared(h)
        L.moe_route_topk(self.T, self.d, self.E, self.K, self.flags, h, self.router, self.logits, self.idx, self.w)
        L.moe_expert_ffn_q4(self.T, self.K, 0, h, self.idx, self.ex, None, self.o, None, None, None, self.ws)
        if self.side is not None:
            cs.wait_stream(self.side)
        L.moe_combine(self.T, self.K, self.d, self.o, self.w, h,
                      None if self.shared is None else self.sho.view(self.T, self.d), y)
        return y
