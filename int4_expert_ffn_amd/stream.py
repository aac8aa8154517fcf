"""Host-side schedule of a prerouted decode stack whose experts live in a slower tier (pinned host
memory) and stream into one HBM pool per layer.

The pages' storage tier is an SSD under a laptop's unified memory ("Arquitecturas nativas para
device: MoE de grano fino y pre-attention router", sections "El pre-attention router: predecir y
prefetchar" and "Las matemáticas que importan"; "La otra mitad del muro de la memoria ...", section
"Ideas clave").  On one MI355X the analogue is host memory read over the host link, roughly two
orders of magnitude below HBM.  Per token t and layer l, with the routing of the resident schedule
(`chain.DecodeStack.token`):

  * prefetch mode: the head of layer l-1 predicts layer l's experts for token t+1 during token t;
    right after that prediction, moe_stream_in(l, t+1) runs on a copy stream (placement in the
    pool, copy of the missing experts; layers take turns on a few copy streams so that the host
    link stays busy), so the copy overlaps the rest of token t on the compute stream.  The token
    ends when every stream is done (the copy streams join the compute stream),
    which keeps a token a self-contained unit that a HIP graph can hold.  A self-routed layer
    (layer 0, every layer at the first token) knows its experts only when it routes, and streams
    them in on the compute stream.
  * reactive mode: every layer streams its experts in on the compute stream just before its
    expert FFN (load on demand: the baseline the prerouter is measured against).

The expert FFN then runs on the pool with the slots moe_stream_in returned.  The same kernels read
the same bytes as the resident stack, so outputs are identical bit for bit.

Reuse safety: a pool of at least 2K slots never hands a slot used at token t to token t+1's copy,
so the copy for t+1 may run beside token t's expert FFN on the same layer.
"""
from __future__ import annotations

from typing import List

import torch

from . import _lib as L
from .chain import DecodeStack, LayerWeights


class StreamedStack(DecodeStack):
    def __init__(self, layers: List[LayerWeights], K: int, device, n_slots: int, prefetch: bool = True,
                 renorm: bool = True, copy_streams: int = 2, fork_every: int = 8):
        if n_slots < 2 * K:
            raise ValueError("a streamed pool needs at least 2K slots (a slot of token t is kept through t+1)")
        if any(lw.norm_gain is not None for lw in layers):
            raise ValueError("streamed stacks take the weightless input norm")
        super().__init__(layers, K, device, renorm)
        dev = self.device
        self.prefetch = prefetch
        self.n_slots = n_slots
        self.pools = [L.Pool(lw.experts, n_slots, dev) for lw in layers]
        self.idx_slot = torch.full((3, self.L, K), -1, dtype=torch.int32, device=dev)
        self.counters = torch.zeros((self.L, 2), dtype=torch.int32, device=dev)      # hits, misses
        self._nb = (L.moe_stream_workspace_size(K) + 255) // 256 * 256
        self.plan_ws = torch.empty((self.L, self._nb), dtype=torch.uint8, device=dev)   # one plan per layer
        # layers take turns on a few copy streams, so one layer's placement and launch overlap another
        # layer's copy and the host link stays busy
        self.copy_streams = [torch.cuda.Stream(device=dev) for _ in range(max(1, copy_streams))]
        self.kick = [torch.cuda.Event() for _ in range(self.L)]      # predictions so far ready
        self.fork_every = max(1, fork_every)
        self._ffn_ws = torch.empty(max(L.moe_expert_ffn_workspace_size(1, K, p.experts) for p in self.pools),
                                   dtype=torch.uint8, device=dev)

    def reset(self):
        """Empty every pool and clear the counters (on the current stream)."""
        for p in self.pools:
            p.reset()
        self.counters.zero_()

    def _stream_in(self, l: int, t: int, stream=None):
        s = t % 3
        L.moe_stream_in(self.K, self.route_idx[s, l], self.layers[l].experts, self.pools[l], self.idx_slot[s, l],
                        self.counters[l], self.plan_ws[l], stream=stream)

    def _prefetch(self, ls: List[int], t: int, n: int):
        """Stream the predicted experts of layers `ls` for token t in on copy stream n % count, after
        the compute stream's work so far (the predictions, and any stream-in of those layers already
        enqueued).  One fork and one moe_stream_in_many call serve several layers: each cross-stream
        dependency, and each launch, costs more than the placement of a few experts."""
        cs = torch.cuda.current_stream(self.device)
        st = self.copy_streams[n % len(self.copy_streams)]
        self.kick[n].record(cs)
        st.wait_event(self.kick[n])
        s = t % 3
        for i in range(0, len(ls), L.MOE_POOL_MAX_JOBS):   # the layers' plans are consecutive in plan_ws
            part = ls[i:i + L.MOE_POOL_MAX_JOBS]
            if part == list(range(part[0], part[0] + len(part))):
                jobs = [(self.route_idx[s, l], self.layers[l].experts, self.pools[l], self.idx_slot[s, l],
                         self.counters[l]) for l in part]
                L.moe_stream_in_many(self.K, jobs, self.plan_ws[part[0]:part[0] + len(part)], stream=st)
            else:
                for l in part:
                    self._stream_in(l, t, stream=st)

    def token(self, t: int, h_in=None, record_routing: bool = False):
        if h_in is not None:
            self.h[0].copy_(h_in)
        s, sp, sn = t % 3, (t - 1) % 3, (t + 1) % 3
        cs = torch.cuda.current_stream(self.device)
        RMS = L.MOE_INPUT_RMSNORM
        pending, forks = [], 0     # layers predicted for token t+1 whose stream-in is not issued yet
        for l, lw in enumerate(self.layers):
            x = self.h[l]
            idx, w = self.route_idx[s, l], self.route_w[s, l]
            self_routed = l == 0 or t == 0 or self.layers[l - 1].head is None
            if self_routed:
                L.moe_route_topk(1, self.d, self.E, self.K, self.topk_flags | RMS, x, lw.router, self.logits[l], idx, w)
            if self_routed or not self.prefetch:
                self._stream_in(l, t)
            if lw.head is not None and l + 1 < self.L:
                L.moe_prerouter(1, self.d, self.E, self.K, RMS, x, idx, self.route_idx[sp, l] if t > 0 else None,
                                lw.head, self.head_logits[l], self.head_ws)
                L.moe_route_topk(1, self.d, self.E, self.K, self.topk_flags, None, None, self.head_logits[l],
                                 self.route_idx[sn, l + 1], self.route_w[sn, l + 1])
                if self.prefetch:
                    pending.append(l + 1)
                    # at the first token every layer streams its own experts in on the compute stream;
                    # the copies for the next token wait for the token's end there
                    if t > 0 and len(pending) >= self.fork_every:
                        self._prefetch(pending, t + 1, forks)
                        pending, forks = [], forks + 1
            L.moe_expert_ffn_q4(1, self.K, RMS, x, self.idx_slot[s, l], self.pools[l].experts, None, None, w, x,
                                self.h[l + 1], self._ffn_ws)
        if pending:
            self._prefetch(pending, t + 1, forks)
            forks += 1
        for i in range(min(forks, len(self.copy_streams))):    # next token's experts are in place at the end
            cs.wait_stream(self.copy_streams[i])
        return self.h[self.L]

    def hits_misses(self):
        """(hits, misses) summed over layers since the last reset (synchronises)."""
        c = self.counters.sum(dim=0).tolist()
        return int(c[0]), int(c[1])
