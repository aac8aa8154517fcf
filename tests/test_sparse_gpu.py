"""GPU parity of the ReLU activation-sparse expert FFN (moe_expert_ffn_sparse) against the fp64
oracle on the same seeded inputs.

Bar: o_k and the fused y per token row within max|y - y_ref| <= 2e-3 * max|y_ref| (float16 in,
float32 accumulation).  The active-neuron count is an integer decided by a float: it must equal
the oracle's count of clearly positive gates plus some of the gates within rounding of zero
(|gate| <= 1e-4 * max|gate|, where float32 and float64 may disagree on the sign)."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import moe_synth as S
import oracle as O
from parity_util import assert_rows_close, log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GATE_BAND = 1e-4


@pytest.fixture(scope="module")
def M():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int4_expert_ffn_amd as m
    return m


def sparse_layer(M, syn, layer):
    """All E experts of one layer on the device, the down projection neuron-major."""
    c = syn.cfg
    mats = S.fill_experts(syn, layer, DEV, relu=True)
    return M.Experts(mats["gate"], mats["up"], mats["down"], c.bits, c.group, neuron_major_down=True), mats


class DenseCache:
    """Dequantised (Wg, Wu, WdT) float64 matrices of an expert, drawn on the CPU (oracle side)."""

    def __init__(self, syn, layer, patch=None):
        self.syn, self.layer, self.c, self.patch = syn, layer, {}, patch

    def packed(self, e):
        out = []
        for m in ("gate", "up", "down_nm"):
            q, s, b = self.syn.expert_mat(self.layer, [int(e)], m, "cpu")
            out.append([q[0].numpy(), s[0].numpy(), b[0].numpy()])
        if self.patch:
            self.patch(int(e), out)
        return out

    def __call__(self, e):
        e = int(e)
        if e not in self.c:
            c = self.syn.cfg
            self.c[e] = tuple(O.dequant(*p, c.bits, c.group) for p in self.packed(e))
        return self.c[e]


def oracle_case(cache, x, idx, w, r):
    """o [T][K][d], y [T][d], and the per-(t, k) band [sure, sure + unsure] of active counts."""
    T, K = idx.shape
    o = np.zeros((T, K, x.shape[1]))
    lo = np.zeros((T, K), dtype=np.int64)
    hi = np.zeros((T, K), dtype=np.int64)
    for t in range(T):
        for k in range(K):
            Wg, Wu, WdT = cache(idx[t, k])
            o[t, k], a = O.expert_ffn_relu(x[t], Wg, Wu, WdT)
            g = Wg @ x[t]
            band = GATE_BAND * max(np.max(np.abs(g)), 1e-300)
            on = a != 0
            lo[t, k] = int(np.count_nonzero(on & (g > band)))
            hi[t, k] = lo[t, k] + int(np.count_nonzero(np.abs(g) <= band))
    return o, O.combine(o, w, r), lo, hi


def run_sparse(M, ex, T, K, flags, x, idx, w, r, with_out=True):
    out = torch.full((T, K, ex.d), float("nan"), dtype=torch.float32, device=DEV) if with_out else None
    y = torch.empty((T, ex.d), dtype=torch.float16, device=DEV)
    n = torch.full((T, K), -7, dtype=torch.int32, device=DEV)
    ws = torch.empty(M.moe_expert_ffn_sparse_workspace_size(T, K, ex), dtype=torch.uint8, device=DEV)
    M.moe_expert_ffn_sparse(T, K, flags, x, idx, ex, out, w, r, y, n, ws)
    return out, y, n


def sparse_case(M, cfg, T, rms=False, seed=0, layer=0, h=None, patch_dev=None, patch_cpu=None):
    log(f"sparse case {cfg.name} T={T} rms={rms} seed={seed}")
    syn = S.Synth(cfg, seed)
    ex, mats = sparse_layer(M, syn, layer)
    if patch_dev:
        patch_dev(mats)
    if h is None:
        h = syn.hidden(500, T)
    x = O.rmsnorm(h.numpy()) if rms else O.f64(h.numpy())
    idx, w = O.route_topk(syn.logits(77, T).numpy(), cfg.K)
    o_ref, y_ref, lo, hi = oracle_case(DenseCache(syn, layer, patch_cpu), x, idx, w, O.f64(h.numpy()))
    hd = h.to(DEV)
    idx_d = torch.tensor(idx, dtype=torch.int32, device=DEV)
    w_d = torch.tensor(w, dtype=torch.float32, device=DEV)
    out, y, n = run_sparse(M, ex, T, cfg.K, M.MOE_INPUT_RMSNORM if rms else 0, hd, idx_d, w_d, hd)
    torch.cuda.synchronize()
    o_np = out.cpu().numpy().reshape(T * cfg.K, -1)
    live = np.abs(o_ref).reshape(T * cfg.K, -1).max(axis=1) > 0
    assert_rows_close(o_np[live], o_ref.reshape(T * cfg.K, -1)[live], what=f"{cfg.name} o_k")
    assert (o_np[~live] == 0).all(), "a slot with no active neuron must give exactly zero"
    assert_rows_close(y.cpu().numpy(), y_ref, what=f"{cfg.name} y")
    n_np = n.cpu().numpy()
    assert ((n_np >= lo) & (n_np <= hi)).all(), f"active counts {n_np} outside [{lo}, {hi}]"
    return dict(ex=ex, out=out, y=y, n=n_np, idx=idx_d, w=w_d, h=hd, lo=lo, hi=hi, o_ref=o_ref)


@pytest.mark.parametrize("name,T", [("tiny", 5), ("decode35b", 1), ("decode35b", 3), ("widek8", 2),
                                    ("large-int4", 2), ("large-int2", 2)])
def test_sparse_ffn(M, name, T):
    r = sparse_case(M, S.CONFIGS[name], T)
    cfg = S.CONFIGS[name]
    frac = r["n"].mean() / cfg.I
    log(f"{name}: active fraction {frac:.3f}")
    assert 0.3 < frac < 0.7        # symmetric gates: about half the neurons are on


def test_sparse_ffn_rmsnorm_input(M):
    sparse_case(M, S.CONFIGS["decode35b"], 2, rms=True)


@pytest.mark.parametrize("bits,group,d,I,E,K", [
    (2, 32, 256, 128, 4, 2),      # a 2-bit segment spans two groups
    (2, 128, 512, 256, 4, 2),
    (4, 128, 512, 256, 4, 3),
    (4, 32, 192, 160, 5, 3),      # 3 slabs: not a multiple of 8 (plain slab order), ragged neuron ranges
    (4, 64, 8192, 256, 3, 2),     # 128 slabs
    (4, 64, 256, 4096, 2, 2),     # the largest d_ff: 4 row rounds per lane
    (4, 32, 256, 128, 16, 16),    # K = E
    (4, 32, 256, 96, 16, 1),      # d_ff below one wave's range
])
def test_sparse_ffn_shapes(M, bits, group, d, I, E, K):
    cfg = replace(S.CONFIGS["tiny"], name=f"sparse{bits}-{group}-{d}-{I}", bits=bits, group=group, d=d, I=I, E=E, K=K)
    sparse_case(M, cfg, 3)


def test_sparse_ffn_many_tokens(M):
    sparse_case(M, S.CONFIGS["tiny"], 40)


def test_sparse_ffn_all_neurons_on(M):
    """Gate biases set to zero and a positive input: every gate is positive, every down row is read
    (the list is full, several rounds of loads per lane)."""
    cfg = replace(S.CONFIGS["tiny"], name="allon", d=512, I=1024, group=64)

    def patch_dev(mats):
        mats["gate"][2].zero_()

    def patch_cpu(e, packed):
        packed[0][2] = np.zeros_like(packed[0][2])

    syn = S.Synth(cfg)
    h = syn.hidden(500, 2).abs() + 0.0625
    r = sparse_case(M, cfg, 2, h=h, patch_dev=patch_dev, patch_cpu=patch_cpu)
    assert (r["n"] >= r["lo"]).all() and (r["lo"] >= cfg.I - 2).all()


def test_sparse_ffn_zero_input(M):
    """x = 0: every gate is zero, so no neuron is on; o is exactly zero and y is the residual."""
    cfg = S.CONFIGS["decode35b"]
    syn = S.Synth(cfg)
    ex, _ = sparse_layer(M, syn, 0)
    x = torch.zeros((2, cfg.d), dtype=torch.float16, device=DEV)
    r = syn.hidden(9, 2).to(DEV)
    idx = torch.tensor([[1, 2, 3, 4], [5, 6, 7, 8]], dtype=torch.int32, device=DEV)
    w = torch.full((2, 4), 0.25, dtype=torch.float32, device=DEV)
    out, y, n = run_sparse(M, ex, 2, 4, 0, x, idx, w, r)
    torch.cuda.synchronize()
    assert (n == 0).all() and (out == 0).all() and torch.equal(y, r)


def test_sparse_inactive_rows_are_not_read(M):
    """The down rows of neurons whose gate is clearly negative get NaN scales on the device; the
    output stays finite and equal to the oracle's on the clean weights, so those rows were skipped
    rather than multiplied by zero."""
    cfg = S.CONFIGS["decode35b"]
    syn = S.Synth(cfg)
    ex, mats = sparse_layer(M, syn, 0)
    h = syn.hidden(500, 1)
    x = O.f64(h.numpy())
    idx, w = O.route_topk(syn.logits(77, 1).numpy(), cfg.K)
    cache = DenseCache(syn, 0)
    poisoned = 0
    for k in range(cfg.K):
        e = int(idx[0, k])
        g = cache(e)[0] @ x[0]
        off = np.nonzero(g < -1e-3 * np.max(np.abs(g)))[0]
        mats["down"][1][e, :, torch.as_tensor(off, device=DEV)] = float("nan")   # scales [E][d/group][I]
        poisoned += len(off)
    log(f"poisoned {poisoned} down rows")
    assert poisoned > cfg.K * cfg.I // 4
    o_ref, y_ref, lo, hi = oracle_case(cache, x, idx, w, x)
    out, y, n = run_sparse(M, ex, 1, cfg.K, 0, h.to(DEV), torch.tensor(idx, dtype=torch.int32, device=DEV),
                           torch.tensor(w, dtype=torch.float32, device=DEV), h.to(DEV))
    torch.cuda.synchronize()
    assert_rows_close(out.cpu().numpy().reshape(cfg.K, -1), o_ref.reshape(cfg.K, -1), what="o_k")
    assert_rows_close(y.cpu().numpy(), y_ref, what="y")


def test_sparse_bad_index_gives_nan(M):
    cfg = S.CONFIGS["tiny"]
    syn = S.Synth(cfg)
    ex, _ = sparse_layer(M, syn, 0)
    h = syn.hidden(1, 1).to(DEV)
    idx = torch.tensor([[3, cfg.E]], dtype=torch.int32, device=DEV)
    w = torch.tensor([[0.5, 0.5]], dtype=torch.float32, device=DEV)
    out, y, n = run_sparse(M, ex, 1, 2, 0, h, idx, w, h)
    torch.cuda.synchronize()
    assert torch.isfinite(out[0, 0]).all() and torch.isnan(out[0, 1]).all() and torch.isnan(y.float()).all()
    assert int(n[0, 1]) == -1 and int(n[0, 0]) > 0
    ref, _ = O.expert_ffn_relu(O.f64(h.cpu().numpy()[0]), *DenseCache(syn, 0)(3))
    assert_rows_close(out[0, 0].cpu().numpy(), ref[None], what="valid slot")


def test_sparse_deterministic_and_fused_only(M):
    """Two runs give identical bits; the fused output alone (out = NULL) equals the fused output
    of the call that also writes o_k."""
    cfg = S.CONFIGS["decode35b"]
    syn = S.Synth(cfg)
    ex, _ = sparse_layer(M, syn, 1)
    h = syn.hidden(3, 2).to(DEV)
    idx = torch.tensor([[7, 100, 3, 255], [9, 8, 200, 1]], dtype=torch.int32, device=DEV)
    w = torch.tensor([[0.4, 0.3, 0.2, 0.1]] * 2, dtype=torch.float32, device=DEV)
    a = run_sparse(M, ex, 2, 4, 0, h, idx, w, h)
    b = run_sparse(M, ex, 2, 4, 0, h, idx, w, h)
    c = run_sparse(M, ex, 2, 4, 0, h, idx, w, h, with_out=False)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
    assert torch.equal(a[1], c[1]) and torch.equal(a[2], c[2])


def test_sparse_fused_combine_repeated(M):
    """The fused combine is formed by whichever of a slab's K blocks finishes last, from the o_k the
    other blocks stored: over many calls with fresh inputs, the fused-only output must equal, bit
    for bit, the one of the call that also returns o_k, and that one the combine of its o_k."""
    cfg = S.CONFIGS["decode35b"]
    syn = S.Synth(cfg)
    ex, _ = sparse_layer(M, syn, 2)
    T, K = 4, cfg.K
    hs = syn.hidden(40, 48 * T).to(DEV).view(48, T, cfg.d)
    lg = syn.logits(41, 48 * T).to(DEV)
    idx = torch.empty((48 * T, K), dtype=torch.int32, device=DEV)
    w = torch.empty((48 * T, K), dtype=torch.float32, device=DEV)
    M.moe_route_topk(48 * T, cfg.d, cfg.E, K, M.MOE_TOPK_RENORM, None, None, lg, idx, w)
    idx, w = idx.view(48, T, K), w.view(48, T, K)
    y_ref = torch.empty((T, cfg.d), dtype=torch.float16, device=DEV)
    for i in range(48):
        h = hs[i]
        out, y, _ = run_sparse(M, ex, T, K, 0, h, idx[i], w[i], h)
        _, y2, _ = run_sparse(M, ex, T, K, 0, h, idx[i], w[i], h, with_out=False)
        M.moe_combine(T, K, cfg.d, out, w[i], h, None, y_ref)
        torch.cuda.synchronize()
        assert torch.equal(y, y2), f"call {i}: fused-only output differs"
        assert torch.equal(y, y_ref), f"call {i}: fused output differs from the combine of o_k"
