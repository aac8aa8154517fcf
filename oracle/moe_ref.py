"""Plain float64 reference of the decode-time fine-grained MoE layer.

TEST INFRASTRUCTURE ONLY: imported by the tests, the package smoke check and the
benchmark's CPU-baseline leg, never by the library.  Every weight is
dequantised explicitly into a float64 matrix and every product is a float64
matmul; no blocking, fusion or reordering beyond the definitions below.

Pages cited (by title and section):
  [DEVICE] "Arquitecturas nativas para device: MoE de grano fino y pre-attention router"
  [EDGE0]  "La otra mitad del muro de la memoria: Servir MoEs de 35B desde SSD con
           prediccion de enrutamiento entrenada" (reading guide of the Edge0 paper)
  [METAL]  "Inferencia de LLM MoE en MacBook Pro: Streaming de Expertos desde SSD con Metal"

Readings taken where the pages leave a step open (all listed with reasons in the
design notes): codes are little-endian inside uint32 words, lowest bits = lowest
column; the group of a column is column // group along the input dimension;
SwiGLU applies SiLU to the gate branch; GELU is the exact erf form; top-K ranks
by logit, ties to the lower expert index, and the K weights are a softmax
renormalised over the K selected logits (or, without renormalisation, the
full-softmax probabilities of the selected experts); the two routing vectors of
the prerouter are binary K-hot vectors of the head's own layer at tokens t and
t-1 (zero at t = 0), concatenated after the hidden state.

Parity pins: see tests/test_oracle_pins.py.  The pages print no worked example of
the prerouted chain; its semantics (which routing vectors feed the head, where
the prediction lands, the first-token bootstrap, self-routing after a layer
without a head) are pinned by a stack worked by hand from the readings above
(tests/golden/prerouted_chain_hand.txt).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Callable, List, Optional, Sequence

import numpy as np

RMS_EPS = 1e-6


def f64(a) -> np.ndarray:
    """Widen a float16/float32/int array (numpy or CPU torch tensor) to float64 exactly."""
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    return np.asarray(a).astype(np.float64)


def _u32(a) -> np.ndarray:
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    a = np.asarray(a)
    return a.view(np.uint32) if a.dtype == np.int32 else a.astype(np.uint32)


# ----------------------------------------------------------------------------------------
# quantised weights  [METAL, "Arquitectura del Sistema" and the Metal dequant listing:
# a weight is its integer code times a scale plus a bias, for 4-bit and 2-bit codes]
# ----------------------------------------------------------------------------------------
def codes(qwords, bits: int) -> np.ndarray:
    """[rows][words] uint32 words -> [rows][cols] integer codes.

    Column j of a row is held in word j // (32/bits), at bit offset bits * (j mod 32/bits);
    the lowest bits of a word hold the lowest column."""
    w = _u32(qwords)
    per = 32 // bits
    cols = w.shape[-1] * per
    j = np.arange(cols)
    return (w[..., j // per].astype(np.int64) >> (bits * (j % per))) & ((1 << bits) - 1)


def dequant(qwords, scales, biases, bits: int, group: int) -> np.ndarray:
    """W[o][i] = q[o][i] * scale[o][i // group] + bias[o][i // group], in float64."""
    q = codes(qwords, bits).astype(np.float64)
    gi = np.arange(q.shape[-1]) // group
    return q * f64(scales)[..., gi] + f64(biases)[..., gi]


# ----------------------------------------------------------------------------------------
# elementwise pieces
# ----------------------------------------------------------------------------------------
def rmsnorm(h, gain=None, eps: float = RMS_EPS) -> np.ndarray:
    """RMS normalisation g * h / sqrt(mean(h^2) + eps) over the last axis  [METAL, "Arquitectura del
    Sistema": RMS normalisation is one of the GPU kernels; EDGE0, "Arquitectura del cabezal
    Prerouter": the head reads the normalised hidden state].  gain None: the weightless form
    (g = 1), the glue between chained layers."""
    h = f64(h)
    x = h / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)
    return x if gain is None else x * f64(gain)


def silu(v) -> np.ndarray:
    v = f64(v)
    return v / (1.0 + np.exp(-v))


def gelu_erf(a) -> np.ndarray:
    """Exact GELU, 0.5 * a * (1 + erf(a / sqrt 2))  [EDGE0, "Arquitectura del cabezal
    Prerouter": the head's nonlinearity is the erf form of GELU]."""
    a = f64(a)
    erf = np.vectorize(math.erf, otypes=[np.float64])
    return 0.5 * a * (1.0 + erf(a / math.sqrt(2.0)))


def to_f16_f64(v) -> np.ndarray:
    """Round float64 to float16 (nearest even) and widen back: the fp16 layer interface."""
    return f64(np.asarray(v, dtype=np.float64).astype(np.float16))


# ----------------------------------------------------------------------------------------
# S1a router and S2 softmax top-K  [DEVICE, "Dos niveles de sparsity": each token uses the
# top-k experts the router picks; EDGE0, "Arquitectura del cabezal Prerouter": top-k routing]
# ----------------------------------------------------------------------------------------
def router_logits(w_router, x) -> np.ndarray:
    """logits[e] = sum_i W_r[e][i] x[i]; x may be [d] or [T][d] (-> [T][E])."""
    return f64(x) @ f64(w_router).T


def topk_indices(logits_row, K: int) -> List[int]:
    """Brute force: sort every (-logit, expert) pair and keep the first K.  Largest logit
    first; equal logits go to the lower expert index."""
    row = f64(logits_row)
    pairs = sorted((-float(v), e) for e, v in enumerate(row))
    return [e for _, e in pairs[:K]]


def topk_weights(logits_row, idx: Sequence[int], renorm: bool = True) -> np.ndarray:
    """Softmax weights of the selected experts.  renorm: exp(l_k - l_1) / sum over the K
    selected; otherwise the full softmax over all E logits, read at the selected experts."""
    row = f64(logits_row)
    if renorm:
        top = row[idx[0]]
        ex = np.array([math.exp(row[e] - top) for e in idx])
        return ex / ex.sum()
    m = row.max()
    den = sum(math.exp(v - m) for v in row)
    return np.array([math.exp(row[e] - m) / den for e in idx])


def route_topk(logits, K: int, renorm: bool = True):
    """[T][E] logits -> (idx int64 [T][K], w float64 [T][K])."""
    lg = f64(logits)
    lg = lg.reshape(-1, lg.shape[-1])
    idx = np.array([topk_indices(r, K) for r in lg], dtype=np.int64)
    w = np.array([topk_weights(r, i, renorm) for r, i in zip(lg, idx)])
    return idx, w


def topk_gaps(logits_row, K: int) -> np.ndarray:
    """Adjacent gaps among the K+1 largest logits (how far the selection is from a tie)."""
    s = np.sort(f64(logits_row))[::-1][: K + 1]
    return s[:-1] - s[1:]


# ----------------------------------------------------------------------------------------
# S1b prerouter head  [EDGE0, "Arquitectura del cabezal Prerouter": input is the hidden state
# concatenated with two top-k routing vectors (current and previous token), of dimension
# d_model + 2E; head(x) = fc2(erf-gelu(fc1(x))) + l(x), l a linear residual path]
# ----------------------------------------------------------------------------------------
def khot(idx_row, E: int) -> np.ndarray:
    v = np.zeros(E)
    if idx_row is not None:
        for e in idx_row:
            v[int(e)] = 1.0
    return v


def prerouter_logits(x, idx_cur, idx_prev, pw: dict, E: int) -> np.ndarray:
    """x [d]; idx_cur, idx_prev [K] (idx_prev None -> zero vector); pw holds the split
    layout (fc1_x [H][d], fc1_r [2E][H], fc2 [E][H], lin_x [E][d], lin_r [2E][E], biases or None).

    The dense fc1 and l are rebuilt as [fc1_x | fc1_r^T] and [lin_x | lin_r^T] and applied
    to the dense z = [x; khot(cur); khot(prev)]."""
    xv = f64(x)
    z = np.concatenate([xv, khot(idx_cur, E), khot(idx_prev, E)])
    fc1 = np.concatenate([f64(pw["fc1_x"]), f64(pw["fc1_r"]).T], axis=1)
    lin = np.concatenate([f64(pw["lin_x"]), f64(pw["lin_r"]).T], axis=1)
    H = fc1.shape[0]
    b1 = f64(pw["fc1_b"]) if pw.get("fc1_b") is not None else np.zeros(H)
    b2 = f64(pw["fc2_b"]) if pw.get("fc2_b") is not None else np.zeros(E)
    bl = f64(pw["lin_b"]) if pw.get("lin_b") is not None else np.zeros(E)
    a = fc1 @ z + b1
    return f64(pw["fc2"]) @ gelu_erf(a) + b2 + lin @ z + bl


# ----------------------------------------------------------------------------------------
# S3-S5 expert FFN  [METAL, "Arquitectura del Sistema": dequantised 4/2-bit matvecs and a
# fused SwiGLU; EDGE0, "Ejecucion del adaptador no fusionado": y = W_int4 x + (alpha/r) B A x]
# ----------------------------------------------------------------------------------------
def lora_delta(A, B, alpha: float, v) -> np.ndarray:
    A = f64(A)
    return (alpha / A.shape[0]) * (f64(B) @ (A @ f64(v)))


def expert_ffn(x, Wg, Wu, Wd, lora: Optional[dict] = None) -> np.ndarray:
    """o = Wd (silu(Wg x) * (Wu x)), W already dequantised float64; x [d] or [T][d].
    lora: {"gate": (A, B), "up": (A, B), "down": (A, B), "alpha": a} adds the unmerged delta
    to each projection."""
    xv = f64(x)
    gate = xv @ Wg.T
    up = xv @ Wu.T
    if lora is not None:
        gate = gate + lora_delta(*lora["gate"], lora["alpha"], xv.T).T
        up = up + lora_delta(*lora["up"], lora["alpha"], xv.T).T
    a = silu(gate) * up
    o = a @ Wd.T
    if lora is not None:
        o = o + lora_delta(*lora["down"], lora["alpha"], a.T).T
    return o


def expert_ffn_packed(x, gate, up, down, bits: int, group: int, lora=None) -> np.ndarray:
    """Same as expert_ffn, from packed (q, scales, biases) triples of one expert."""
    return expert_ffn(x, dequant(*gate, bits, group), dequant(*up, bits, group),
                      dequant(*down, bits, group), lora)


# ----------------------------------------------------------------------------------------
# ReLU activation-sparse expert  [DEVICE, "Dos niveles de sparsity", level 2 (sparse FFN):
# under a ReLU-type nonlinearity many intermediate neurons are exactly zero for a token, and a
# zero neuron's weights need not be read or multiplied.  Reading taken: the gated unit keeps its
# gate / up / down matrices and ReLU replaces SiLU on the gate branch; the down projection is
# stored neuron-major ([I][d], row i = the weights neuron i feeds, groups along d) so that a
# skipped neuron is a skipped contiguous row.  Skipping is exact, so the definition below is the
# dense product.]
# ----------------------------------------------------------------------------------------
def relu(v) -> np.ndarray:
    return np.maximum(f64(v), 0.0)


def expert_ffn_relu(x, Wg, Wu, WdT):
    """(o, a): a = relu(Wg x) * (Wu x) and o = sum_i a_i WdT[i] = WdT^T a, float64.  WdT is the
    down projection neuron-major, [I][d]; x [d] or [T][d]."""
    xv = f64(x)
    a = relu(xv @ Wg.T) * (xv @ Wu.T)
    return a @ WdT, a


def expert_ffn_relu_packed(x, gate, up, down_nm, bits: int, group: int):
    """Same as expert_ffn_relu from packed triples; down_nm is [I][d*bits/32] words with
    [I][d/group] scales and biases (its groups run along d, the stored row)."""
    return expert_ffn_relu(x, dequant(*gate, bits, group), dequant(*up, bits, group),
                           dequant(*down_nm, bits, group))


def active_neurons(a) -> np.ndarray:
    """Number of intermediate neurons with a nonzero output (the rows the down projection
    reads), over the last axis."""
    return np.count_nonzero(f64(a) != 0.0, axis=-1)


# ----------------------------------------------------------------------------------------
# S6 combine  [METAL, "Arquitectura del Sistema": expert combination and residual in one step]
# ----------------------------------------------------------------------------------------
def combine(o, w, r, shared=None) -> np.ndarray:
    """y = r + sum_k w_k o_k (+ shared).  o [K][d] (or [T][K][d]), w [K] (or [T][K])."""
    o, w = f64(o), f64(w)
    y = f64(r) + np.einsum("...k,...kd->...d", w, o)
    if shared is not None:
        y = y + f64(shared)
    return y


# ----------------------------------------------------------------------------------------
# S7 batched grouping: tokens sorted by expert (stable counting sort)
# ----------------------------------------------------------------------------------------
def group_by_expert(idx, E: int):
    """idx [T][K] -> (counts [E], offsets [E+1], perm [T*K]); perm lists the flat (t*K + k)
    pairs grouped by expert, ascending (t, k) inside each expert."""
    flat = np.asarray(idx, dtype=np.int64).reshape(-1)
    counts = np.zeros(E, dtype=np.int64)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    fill = offsets[:-1].copy()
    perm = np.zeros(flat.size, dtype=np.int64)
    for p, e in enumerate(flat):
        perm[fill[e]] = p
        fill[e] += 1
    return counts, offsets, perm


# ----------------------------------------------------------------------------------------
# whole layer and the prerouted decode chain
# ----------------------------------------------------------------------------------------
def moe_layer(x, r, idx, w, expert_get: Callable, bits: int, group: int,
              shared=None, lora=None) -> np.ndarray:
    """One layer for T tokens with given routing: y_t = r_t + sum_k w_tk FFN_{idx_tk}(x_t)
    (+ FFN_shared(x_t) with its LoRA).  expert_get(e) -> (gate, up, down) packed triples."""
    xv = np.atleast_2d(f64(x))
    rv = np.atleast_2d(f64(r))
    idx = np.atleast_2d(idx)
    w = np.atleast_2d(f64(w))
    T, K = idx.shape
    cache = {}
    y = np.zeros_like(rv)
    for t in range(T):
        o = []
        for k in range(K):
            e = int(idx[t, k])
            if e not in cache:
                g, u, dn = expert_get(e)
                cache[e] = (dequant(*g, bits, group), dequant(*u, bits, group), dequant(*dn, bits, group))
            o.append(expert_ffn(xv[t], *cache[e]))
        sh = None
        if shared is not None:
            g, u, dn = shared
            sh = expert_ffn_packed(xv[t], g, u, dn, bits, group, lora)
        y[t] = combine(np.array(o), w[t], rv[t], sh)
    return y


@dataclass
class ChainState:
    """Routing carried between tokens: pred[l] = (idx, w) predicted for layer l by the head of
    layer l-1 at the previous token; prev[l] = routing layer l used at the previous token."""
    L: int
    pred: List[Optional[tuple]] = field(default_factory=list)
    prev: List[Optional[np.ndarray]] = field(default_factory=list)

    def __post_init__(self):
        if not self.pred:
            self.pred = [None] * self.L
        if not self.prev:
            self.prev = [None] * self.L


@dataclass
class LayerTrace:
    idx: np.ndarray
    w: np.ndarray
    route_logits: Optional[np.ndarray]      # router logits when the layer routed itself
    head_logits: Optional[np.ndarray]       # logits of this layer's head (for layer l+1, token t+1)
    y: np.ndarray                           # layer output rounded to float16 (as float64)


def chain_token(h0, state: ChainState, *, E: int, K: int, bits: int, group: int,
                router_get: Callable, head_get: Callable, expert_get: Callable,
                renorm: bool = True, gain_get: Optional[Callable] = None):
    """One decode token through the L layers of a prerouted stack.

    Layer l: x = rmsnorm(h).  Routing: layer 0 (and any layer with no prediction yet, i.e.
    every layer at the first token) runs its own router and top-K; otherwise it uses the set
    and weights the head of layer l-1 predicted one token earlier ([EDGE0, "Ideas clave":
    the prediction is the routing, with no fallback]).  The head of layer l (l < L-1)
    reads [x; khot(routing of layer l at t); khot(routing of layer l at t-1)] and its top-K
    becomes layer l+1's routing at token t+1 ([EDGE0, "Arquitectura del cabezal Prerouter"]).
    y = h + sum_k w_k FFN_k(x), rounded to float16, is the next layer's h.

    router_get(l) -> W_r [E][d]; head_get(l) -> split head dict; expert_get(l, e) -> packed
    (gate, up, down); gain_get(l) -> the layer's RMS-norm gain [d] or None (weightless).
    Returns (h_L, new_state, traces)."""
    L = state.L
    new = ChainState(L)
    h = f64(h0)
    traces = []
    for l in range(L):
        x = rmsnorm(h, None if gain_get is None else gain_get(l))
        rl = None
        if l == 0 or state.pred[l] is None:
            rl = router_logits(router_get(l), x)
            idx = np.array(topk_indices(rl, K))
            w = topk_weights(rl, idx, renorm)
        else:
            idx, w = state.pred[l]
        hl = None
        if l < L - 1:
            pw = head_get(l)
            if pw is not None:
                hl = prerouter_logits(x, idx, state.prev[l], pw, E)
                pidx = np.array(topk_indices(hl, K))
                new.pred[l + 1] = (pidx, topk_weights(hl, pidx, renorm))
        o = [expert_ffn_packed(x, *expert_get(l, int(e)), bits, group) for e in idx]
        y = to_f16_f64(combine(np.array(o), w, h))
        new.prev[l] = np.array(idx)
        traces.append(LayerTrace(np.array(idx), np.array(w), rl, hl, y))
        h = y
    return h, new, traces


# ----------------------------------------------------------------------------------------
# Expert streaming from a slower memory tier  [DEVICE, "Las matemáticas que importan": the
# resident set is the active experts plus a cache of recent / likely ones, and the number of
# experts one window of compute can bring in; DEVICE, "El pre-attention router": the load is
# hidden when the compute window is at least the load time; EDGE0, "Ideas clave": experts are
# streamed into a compact pool and the one-token-ahead prediction is the routing, so the
# prepared set is the routed set]
# ----------------------------------------------------------------------------------------
def experts_per_window(window_s: float, bandwidth_Bps: float, expert_bytes: float) -> int:
    """How many whole experts a load of `bandwidth_Bps` brings in during `window_s`:
    floor(window / t_one) with t_one = expert_bytes / bandwidth."""
    t_one = expert_bytes / bandwidth_Bps
    return int(math.floor(window_s / t_one * (1 + 1e-12)))


def stall_time(n_needed: int, window_s: float, bandwidth_Bps: float, expert_bytes: float) -> float:
    """Wait exposed in one window: the experts past what the window covers load after it, each
    costing t_one; zero when every needed expert fits under the window."""
    t_one = expert_bytes / bandwidth_Bps
    n_free = experts_per_window(window_s, bandwidth_Bps, expert_bytes)
    return max(0, n_needed - n_free) * t_one


@dataclass
class PoolState:
    """One layer's pool of `n_slots` expert slots: the expert each slot holds (-1 = empty) and the
    last token that used it (-1 = never)."""
    n_slots: int
    expert: List[int] = field(default_factory=list)
    stamp: List[int] = field(default_factory=list)

    def __post_init__(self):
        if not self.expert:
            self.expert = [-1] * self.n_slots
        if not self.stamp:
            self.stamp = [-1] * self.n_slots


def pool_plan(state: PoolState, idx: Sequence[int], token: int):
    """Place a token's selected experts in the pool, least recently used slot first.

    Reading taken (the pages keep "recent / likely" experts and say no more): every selected
    expert already in a slot is a hit and its slot is stamped with the token; then, in slot-k
    order, each missing expert takes the slot with the oldest stamp among those this token has
    not stamped (empty slots first, then ties to the lowest slot index), and must be copied in.
    Returns (slot of each k, list of (k, slot, expert) copies) and updates `state`."""
    idx = [int(e) for e in idx]
    slot = [-1] * len(idx)
    for k, e in enumerate(idx):
        if e in state.expert:
            s = state.expert.index(e)
            slot[k] = s
            state.stamp[s] = token
    copies = []
    for k, e in enumerate(idx):
        if slot[k] >= 0:
            continue
        free = [(state.stamp[s], s) for s in range(state.n_slots) if state.stamp[s] < token]
        _, s = min(free)
        state.expert[s] = e
        state.stamp[s] = token
        slot[k] = s
        copies.append((k, s, e))
    return slot, copies
