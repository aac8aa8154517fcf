"""Helpers of the GPU parity tests: device-resident layers made by the seeded generator, the same
tensors regenerated on the CPU for the oracle, gap-filtered tokens, and the tolerance rule."""
from __future__ import annotations

import sys

import numpy as np
import torch

import moe_synth as S
import oracle as O

# Output tolerance of float16-in / float32-accumulate results, per token row:
#   max |y - y_ref| <= TOL * max |y_ref|
TOL = 2e-3
# Minimum adjacent gap among the K+1 largest oracle logits for a token used in index parity.
GAP = 1e-4


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def assert_rows_close(got, ref, tol=TOL, what=""):
    got = np.asarray(got, dtype=np.float64).reshape(-1, np.shape(ref)[-1])
    ref = np.asarray(ref, dtype=np.float64).reshape(got.shape)
    for t in range(ref.shape[0]):
        err = np.max(np.abs(got[t] - ref[t]))
        scale = np.max(np.abs(ref[t]))
        assert np.isfinite(got[t]).all(), f"{what} row {t}: non-finite output"
        assert err <= tol * scale, f"{what} row {t}: max err {err:.3e} > {tol} * {scale:.3e}"


def device_layer(syn: S.Synth, layer: int, dev):
    """All E experts of one layer on the device, wrapped for the C ABI."""
    import int4_expert_ffn_amd as M
    mats = S.fill_experts(syn, layer, dev)
    c = syn.cfg
    return M.Experts(mats["gate"], mats["up"], mats["down"], c.bits, c.group)


def cpu_expert(syn: S.Synth, layer: int, e: int):
    """(gate, up, down) packed triples of expert e, generated on the CPU (oracle side)."""
    out = []
    for m in S.MATS:
        q, s, b = syn.expert_mat(layer, [e], m, "cpu")
        out.append((q[0].numpy(), s[0].numpy(), b[0].numpy()))
    return tuple(out)


class ExpertCache:
    def __init__(self, syn, layer):
        self.syn, self.layer, self.c = syn, layer, {}

    def __call__(self, e):
        e = int(e)
        if e not in self.c:
            self.c[e] = cpu_expert(self.syn, self.layer, e)
        return self.c[e]


def gap_tokens(syn: S.Synth, router_np, T, K, rmsnorm=False, first_stream=1000):
    """T float16 hidden vectors whose oracle router logits have every adjacent gap among the top
    K+1 at least GAP (redrawing with the next stream number otherwise)."""
    rows, redraws, s = [], 0, first_stream
    while len(rows) < T:
        h = syn.hidden(s, 1)[0]
        s += 1
        x = O.rmsnorm(h.numpy()) if rmsnorm else O.f64(h.numpy())
        lg = O.router_logits(router_np, x)
        if O.topk_gaps(lg, K).min() >= GAP:
            rows.append(h)
        else:
            redraws += 1
    return torch.stack(rows), redraws
