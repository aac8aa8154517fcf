"""Seeded synthetic inputs for the decode-time fine-grained MoE layer.

This module is the only code shared by the oracle and the GPU path.  It holds
the workload shapes and a counter-based random generator, and none of the
layer's arithmetic (no dequantisation, routing, activation or combine).

Generator
---------
SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014).  Element ``i`` (0-based) of a stream with 64-bit key
``k`` is ``mix64(k + (i + 1) * GAMMA)`` with the published constants.  Every
tensor gets its own stream key, derived from
``(seed, config, layer, expert, tensor)``, so any slice of any tensor can be
regenerated on its own, on any device.  The implementation is torch integer
arithmetic (int64, two's-complement wrap), identical bit for bit on CPU and
GPU; ``splitmix64_py`` is the plain big-integer definition it is tested against.

Value recipes (the workloads' distributions)
--------------------------------------------
* packed codes: a uniform 32-bit word holds 8 uniform 4-bit or 16 uniform
  2-bit codes, so code words are the top 32 bits of a hash;
* uniform U[a, b): 24-bit uniform ``u = (h >> 40) * 2**-24``, ``a + (b - a) u``
  in float64;
* normal N(0, std**2): Irwin-Hall sum of twelve 16-bit uniforms drawn from three
  hashes, ``z = (S + 6) * 2**-16 - 6`` (exact in float64, mean 0, variance 1,
  tails cut at 6 sigma), then ``z * std`` in float64;
* every float16 value is rounded float64 -> float32 -> float16, round to
  nearest even at each step, so CPU and GPU agree.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional, Sequence

import torch

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB


def _signed(c: int) -> int:
    c &= MASK64
    return c - (1 << 64) if c >= (1 << 63) else c


def mix64_py(z: int) -> int:
    """SplitMix64 output function on a Python integer (the published definition)."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * MIX1) & MASK64
    z = ((z ^ (z >> 27)) * MIX2) & MASK64
    return z ^ (z >> 31)


def splitmix64_py(key: int, i: int) -> int:
    """Element ``i`` of the stream with key ``key`` (pure Python, for tests)."""
    return mix64_py((key + (i + 1) * GAMMA) & MASK64)


# tensor identifiers inside a (config, layer, expert) triple
T_ROUTER = 1
T_HIDDEN = 2
T_LOGITS = 3
T_Q, T_SCALE, T_BIASNOISE = 10, 11, 12          # + 4 * matrix (gate 0, up 1, down 2)
T_FC1X, T_FC1R, T_FC1B, T_FC2, T_FC2B, T_LINR, T_LINB = 20, 21, 22, 23, 24, 26, 27
T_LORA_A, T_LORA_B = 30, 31                    # + 2 * matrix
T_NORM = 40                                     # RMS-norm gain of a layer input
T_DOWN_NM = 50                                  # neuron-major down projection: + 0 codes, 1 scales, 2 bias noise
MATS = ("gate", "up", "down")


def stream_key(seed: int, cfg: int, layer: int, expert: int, tensor: int) -> int:
    k = mix64_py(seed)
    for v in (cfg, layer, expert, tensor):
        k = mix64_py(k ^ (((v + 1) * GAMMA) & MASK64))
    return k


def _shr(z: torch.Tensor, s: int) -> torch.Tensor:
    """Logical right shift of int64 bit patterns."""
    return (z >> s) & ((1 << (64 - s)) - 1)


def hash_block(keys: Sequence[int], start: int, n: int, device="cpu") -> torch.Tensor:
    """int64 bit patterns of elements [start, start+n) of each stream: shape [len(keys), n]."""
    kt = torch.tensor([_signed(k) for k in keys], dtype=torch.int64, device=device)
    z = torch.arange(start + 1, start + n + 1, dtype=torch.int64, device=device)
    z = z.mul_(_signed(GAMMA)).unsqueeze(0) + kt.unsqueeze(1)
    z ^= _shr(z, 30)
    z.mul_(_signed(MIX1))
    z ^= _shr(z, 27)
    z.mul_(_signed(MIX2))
    z ^= _shr(z, 31)
    return z


def _hi32_as_int32(h: torch.Tensor) -> torch.Tensor:
    v = _shr(h, 32)
    return torch.where(v >= (1 << 31), v - (1 << 32), v).to(torch.int32)


def _uniform24(h: torch.Tensor) -> torch.Tensor:
    return _shr(h, 40).to(torch.float64) * (2.0 ** -24)


def _irwin_hall12(h3: torch.Tensor) -> torch.Tensor:
    """h3: [..., 3] hashes -> float64 approximately N(0,1), exact arithmetic."""
    s = (_shr(h3, 48) + ((h3 >> 32) & 0xFFFF) + ((h3 >> 16) & 0xFFFF) + (h3 & 0xFFFF)).sum(-1)
    return (s + 6).to(torch.float64) * (2.0 ** -16) - 6.0


def to_f16(v64: torch.Tensor) -> torch.Tensor:
    return v64.to(torch.float32).to(torch.float16)


def normal_f16(keys: Sequence[int], n: int, std: float, device="cpu") -> torch.Tensor:
    h = hash_block(keys, 0, 3 * n, device).view(len(keys), n, 3)
    return to_f16(_irwin_hall12(h) * std)


def words_u32(keys: Sequence[int], n: int, device="cpu") -> torch.Tensor:
    return _hi32_as_int32(hash_block(keys, 0, n, device))


def uniform_f64(keys: Sequence[int], n: int, lo: float, hi: float, device="cpu") -> torch.Tensor:
    return _uniform24(hash_block(keys, 0, n, device)) * (hi - lo) + lo


# --------------------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------------------
@dataclass(frozen=True)
class MoEConfig:
    cid: int
    name: str
    d: int              # d_model
    E: int              # routed experts
    K: int              # experts per token
    I: int              # expert intermediate size
    group: int          # quantisation group along the input dimension
    bits: int           # 4 or 2
    L: int              # layers
    T: int = 1          # tokens per call
    head_hidden: int = 0        # prerouter fc1 width (0 = no prerouter)
    router: str = "gauss"       # "gauss": N(0, 1/d); "orthonormal": orthonormal rows
    shared_expert: bool = False
    lora_rank: int = 0
    lora_alpha: float = 0.0
    scale_lo: float = 0.005
    scale_hi: float = 0.02
    bias_noise: float = 1e-3

    def words_per_row(self, cols: int) -> int:
        return cols * self.bits // 32

    def mat_shape(self, mat: str):
        """[rows][cols] of a matrix; "down_nm" is the down projection stored neuron-major."""
        return (self.I, self.d) if mat in ("gate", "up", "down_nm") else (self.d, self.I)

    def qmat_bytes(self, mat: str) -> int:
        rows, cols = self.mat_shape(mat)
        return rows * cols * self.bits // 8 + rows * (cols // self.group) * 4

    def expert_bytes(self) -> int:
        return sum(self.qmat_bytes(m) for m in MATS)

    def with_bits(self, bits: int, name: Optional[str] = None) -> "MoEConfig":
        from dataclasses import replace
        return replace(self, bits=bits, name=name or f"{self.name}-int{bits}")


CONFIGS = {
    "tiny": MoEConfig(0, "tiny", d=256, E=16, K=2, I=128, group=32, bits=4, L=1),
    "decode35b": MoEConfig(1, "decode35b", d=2048, E=256, K=4, I=512, group=64, bits=4, L=40,
                           head_hidden=1024),
    "widek8": MoEConfig(2, "widek8", d=2048, E=256, K=8, I=512, group=64, bits=4, L=24,
                        router="orthonormal"),
    "large-int4": MoEConfig(3, "large-int4", d=4096, E=512, K=4, I=1024, group=64, bits=4, L=15),
    "large-int2": MoEConfig(3, "large-int2", d=4096, E=512, K=4, I=1024, group=64, bits=2, L=15),
    "batched": MoEConfig(4, "batched", d=2048, E=256, K=4, I=512, group=64, bits=4, L=1, T=256,
                         shared_expert=True, lora_rank=16, lora_alpha=32.0),
}


class Synth:
    """Seeded tensors of one workload.  ``device`` picks where they are made."""

    def __init__(self, cfg: MoEConfig, seed: int = 0):
        self.cfg = cfg
        self.seed = seed
        # the 2-bit variant of the large config gets its own streams
        self._cid = cfg.cid * 10 + (cfg.bits if cfg.bits != 4 else 0)

    def key(self, layer: int, expert: int, tensor: int) -> int:
        return stream_key(self.seed, self._cid, layer, expert, tensor)

    # ---- routed / shared expert weights -------------------------------------------
    def expert_mat(self, layer: int, experts: Sequence[int], mat: str, device="cpu"):
        """(q int32 [n][rows][words], scales f16 [n][rows][groups], biases f16 [n][rows][groups]).

        Codes uniform over 0..2^bits-1, scale U[scale_lo, scale_hi), and
        bias = -2^(bits-1) * scale + N(0, bias_noise^2), all float16.
        """
        c = self.cfg
        if mat == "down_nm":
            tq, ts, tb = T_DOWN_NM, T_DOWN_NM + 1, T_DOWN_NM + 2
        else:
            m = MATS.index(mat)
            tq, ts, tb = T_Q + 4 * m, T_SCALE + 4 * m, T_BIASNOISE + 4 * m
        rows, cols = c.mat_shape(mat)
        nw = rows * c.words_per_row(cols)
        ng = rows * (cols // c.group)
        n = len(experts)
        q = words_u32([self.key(layer, e, tq) for e in experts], nw, device)
        s64 = uniform_f64([self.key(layer, e, ts) for e in experts], ng, c.scale_lo, c.scale_hi, device)
        s16 = to_f16(s64)
        hn = hash_block([self.key(layer, e, tb) for e in experts], 0, 3 * ng, device)
        noise = _irwin_hall12(hn.view(n, ng, 3)) * c.bias_noise
        b16 = to_f16(s16.to(torch.float64) * -float(1 << (c.bits - 1)) + noise)
        return (q.view(n, rows, -1), s16.view(n, rows, -1), b16.view(n, rows, -1))

    def shared_expert_id(self) -> int:
        return self.cfg.E   # the shared expert is drawn as expert number E

    # ---- router ------------------------------------------------------------------
    def router(self, layer: int, device="cpu") -> torch.Tensor:
        """[E][d] float16.  "gauss": N(0, 1/d) (variance 1/d, so logits ~ N(0, 1) for
        unit-RMS input); "orthonormal": rows of an orthonormal basis of a seeded
        Gaussian whose rows were first made orthogonal to the all-ones vector (each row
        minus its mean; QR in float64 on the CPU), so logits of isotropic input are iid
        N(0,1) and a component shared by every column of the input moves no logit.  (The
        affine 4-bit weights of the recipe have mean -scale/2, so every expert adds such a
        component to the residual stream and, left in the routers, it steers every token of
        a deep chain to the same few experts.)"""
        c = self.cfg
        if c.router == "gauss":
            return normal_f16([self.key(layer, 0, T_ROUTER)], c.E * c.d, 1.0 / math.sqrt(c.d),
                              device).view(c.E, c.d)
        g = normal_f16([self.key(layer, 0, T_ROUTER)], c.E * c.d, 1.0, "cpu").view(c.E, c.d).to(torch.float64)
        g = g - g.mean(dim=1, keepdim=True)
        qm, _ = torch.linalg.qr(g.t())                        # [d][E], orthonormal columns
        return to_f16(qm.t().contiguous()).to(device)

    # ---- prerouter head of layer `layer` (predicts layer+1) --------------------------
    def head(self, layer: int, device="cpu") -> dict:
        """Split-layout head weights, float16:
        fc1_x [H][d], fc1_r [2E][H] (row j = fc1 column d+j), fc1_b [H],
        fc2 [E][H], fc2_b [E], lin_x [E][d] (= the next layer's router), lin_r [2E][E], lin_b [E].
        fc1 ~ N(0, 1/(d+2E)), fc2 ~ N(0, 1/H), lin_r ~ N(0, 1/(d+2E)), biases N(0, 0.02^2)."""
        c = self.cfg
        H, d, E = c.head_hidden, c.d, c.E
        fan1 = d + 2 * E
        k = lambda t: [self.key(layer, 0, t)]
        return {
            "fc1_x": normal_f16(k(T_FC1X), H * d, 1 / math.sqrt(fan1), device).view(H, d),
            "fc1_r": normal_f16(k(T_FC1R), 2 * E * H, 1 / math.sqrt(fan1), device).view(2 * E, H),
            "fc1_b": normal_f16(k(T_FC1B), H, 0.02, device).view(H),
            "fc2": normal_f16(k(T_FC2), E * H, 1 / math.sqrt(H), device).view(E, H),
            "fc2_b": normal_f16(k(T_FC2B), E, 0.02, device).view(E),
            "lin_x": self.router(layer + 1, device),
            "lin_r": normal_f16(k(T_LINR), 2 * E * E, 1 / math.sqrt(fan1), device).view(2 * E, E),
            "lin_b": normal_f16(k(T_LINB), E, 0.02, device).view(E),
        }

    # ---- RMS-norm gain of a layer input -------------------------------------------------
    def norm_gain(self, layer: int, device="cpu") -> torch.Tensor:
        """[d] float16 gain of layer `layer`'s input normalisation, U[0.5, 1.5) (a trained gain sits
        around 1; the spread makes a dropped or misplaced gain visible)."""
        c = self.cfg
        return to_f16(uniform_f64([self.key(layer, 0, T_NORM)], c.d, 0.5, 1.5)).view(c.d).to(device)

    # ---- shared-path LoRA -----------------------------------------------------------
    def lora(self, layer: int, device="cpu") -> dict:
        """Per projection m: A [r][in], B [out][r], float16 N(0, 0.02^2)."""
        c = self.cfg
        r = c.lora_rank
        out = {}
        for m, mat in enumerate(MATS):
            rows, cols = c.mat_shape(mat)
            out[mat] = (
                normal_f16([self.key(layer, c.E, T_LORA_A + 2 * m)], r * cols, 0.02, device).view(r, cols),
                normal_f16([self.key(layer, c.E, T_LORA_B + 2 * m)], rows * r, 0.02, device).view(rows, r),
            )
        return out

    # ---- activations ----------------------------------------------------------------
    def hidden(self, stream: int, T: int, device="cpu") -> torch.Tensor:
        """[T][d] float16 N(0, 1); `stream` numbers independent draws (token, redraw...)."""
        c = self.cfg
        return normal_f16([self.key(0, stream, T_HIDDEN)], T * c.d, 1.0, device).view(T, c.d)

    def logits(self, stream: int, T: int, device="cpu") -> torch.Tensor:
        """[T][E] float32 N(0,1) logits (for the logits-input top-K path)."""
        c = self.cfg
        h = hash_block([self.key(0, stream, T_LOGITS)], 0, 3 * T * c.E, device).view(T * c.E, 3)
        return (_irwin_hall12(h)).to(torch.float32).view(T, c.E)


def fill_experts(syn: Synth, layer: int, device, chunk: int = 32, relu: bool = False):
    """All E routed experts of one layer on `device`: dict mat -> (q, s, b) stacked [E][...].
    relu: the down projection is drawn neuron-major ([E][I][d], groups along d), the layout of
    the ReLU activation-sparse expert, with its scales and biases stored group-major ([E][d/group][I],
    a transposed copy of the drawn [E][I][d/group] values); gate and up are the same draws either way."""
    c = syn.cfg
    out = {}
    for mat in MATS:
        src = "down_nm" if (relu and mat == "down") else mat
        rows, cols = c.mat_shape(src)
        q = torch.empty((c.E, rows, c.words_per_row(cols)), dtype=torch.int32, device=device)
        s = torch.empty((c.E, rows, cols // c.group), dtype=torch.float16, device=device)
        b = torch.empty_like(s)
        for e0 in range(0, c.E, chunk):
            ids = list(range(e0, min(c.E, e0 + chunk)))
            qq, ss, bb = syn.expert_mat(layer, ids, src, device)
            q[e0:e0 + len(ids)] = qq
            s[e0:e0 + len(ids)] = ss
            b[e0:e0 + len(ids)] = bb
        if src == "down_nm":
            s, b = s.transpose(1, 2).contiguous(), b.transpose(1, 2).contiguous()
        out[mat] = (q, s, b)
    return out
