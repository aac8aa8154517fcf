"""Pins of the fp64 oracle to facts fixed outside it: hand-worked fixtures, closed forms,
brute force on tiny inputs and special cases that reduce to plain linear algebra.

Each test is chosen so that a plausible slip in the oracle (a dropped bias term, a wrong
group or nibble index, a transposed operand, a sign error, a wrong tie rule) fails it."""
import math

import numpy as np
import pytest
import scipy.special

import oracle as O
import golden_io
from golden_io import read_fixture
from moe_synth import CONFIGS, Synth

RNG = np.random.default_rng(1234)


def _fixture_row(name):
    fx = read_fixture(name)
    bits = int(fx["bits"][0][0])
    group = int(fx["group"][0][0])
    words = np.array([[int(w, 16) for w in fx["words"][0]]], dtype=np.uint32)
    codes = np.array([int(c) for c in fx["codes"][0]])
    s = np.array([[float(fx["scale"][0][0])]], dtype=np.float16)
    b = np.array([[float(fx["bias"][0][0])]], dtype=np.float16)
    return fx, bits, group, words, codes, s, b


@pytest.mark.parametrize("name", ["dequant_int4_hand_packed.txt", "dequant_int2_hand_packed.txt"])
def test_hand_packed_dequant(name):
    fx, bits, group, words, codes, s, b = _fixture_row(name)
    assert (O.codes(words, bits)[0] == codes).all()
    W = O.dequant(words, s, b, bits, group)
    head = [float(v) for v in fx["weights_head"][0]]
    assert W[0, : len(head)].tolist() == head
    # x = e_j returns column j exactly; x = ones returns the hand-computed sum
    for j in (0, 5, 17, 63):
        e = np.zeros(64)
        e[j] = 1.0
        assert (W @ e)[0] == W[0, j]
    assert (W @ np.ones(64))[0] == float(fx["dot_ones"][0][0])


def test_group_index_along_input_dim():
    # two groups of 32 columns: codes all 1; group 0 -> 1*1+0, group 1 -> 1*2+10
    words = np.full((1, 8), 0x11111111, dtype=np.uint32)
    s = np.array([[1.0, 2.0]], dtype=np.float16)
    b = np.array([[0.0, 10.0]], dtype=np.float16)
    W = O.dequant(words, s, b, 4, 32)
    assert W[0, :32].tolist() == [1.0] * 32 and W[0, 32:].tolist() == [12.0] * 32


def _bytewise_codes(words, bits):
    """Independent unpack: walk the little-endian bytes, low bit-field first."""
    out = []
    for row in words:
        vals = []
        for byte in row.astype("<u4").tobytes():
            for f in range(8 // bits):
                vals.append((byte >> (bits * f)) & ((1 << bits) - 1))
        out.append(vals)
    return np.array(out)


@pytest.mark.parametrize("bits,group", [(4, 32), (4, 64), (4, 128), (2, 32), (2, 64), (2, 128)])
def test_dequant_matvec_vs_fma_grouped_form(bits, group):
    """sum_j (q_j s + b) x_j == s * sum_j q_j x_j + b * sum_j x_j per group (the FMA rewrite of
    the Metal listing), with codes unpacked by an independent byte walk."""
    rows, cols = 3, 256
    words = RNG.integers(0, 2 ** 32, size=(rows, cols * bits // 32), dtype=np.uint64).astype(np.uint32)
    s = RNG.uniform(0.005, 0.02, size=(rows, cols // group)).astype(np.float16)
    b = (-(2 ** (bits - 1)) * s.astype(np.float64) + RNG.normal(0, 1e-3, s.shape)).astype(np.float16)
    x = RNG.normal(size=cols)
    q = _bytewise_codes(words, bits)
    assert (q == O.codes(words, bits)).all()
    ref = np.zeros(rows)
    for o in range(rows):
        for gi in range(cols // group):
            sl = slice(gi * group, (gi + 1) * group)
            sx = float(s[o, gi]) * x[sl]
            bx = float(b[o, gi]) * x[sl]
            ref[o] += np.sum(q[o, sl] * sx + bx)
    got = O.dequant(words, s, b, bits, group) @ x
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_activation_closed_forms():
    fx = read_fixture("activations.txt")
    for v, want in fx["silu"]:
        assert O.silu(np.array([float(v)]))[0] == pytest.approx(float(want), abs=1e-15)
    for v, want in fx["gelu"]:
        assert O.gelu_erf(np.array([float(v)]))[0] == pytest.approx(float(want), abs=1e-15)


def test_rmsnorm_closed_form():
    h = np.full(64, 3.0)
    assert O.rmsnorm(h)[0] == pytest.approx(3.0 / math.sqrt(9.0 + 1e-6), rel=1e-15)
    h = np.array([3.0, -4.0])
    assert O.rmsnorm(h).tolist() == pytest.approx([3 / math.sqrt(12.5 + 1e-6), -4 / math.sqrt(12.5 + 1e-6)])


def test_rmsnorm_gain():
    """The gain multiplies each normalised element; the sum of squares is of h alone."""
    h = np.array([3.0, -4.0])
    r = math.sqrt(12.5 + 1e-6)
    assert O.rmsnorm(h, np.array([2.0, 0.5])).tolist() == pytest.approx([6 / r, -2 / r], rel=1e-15)
    rng = np.random.default_rng(3)
    hh = rng.standard_normal((5, 64))
    assert np.array_equal(O.rmsnorm(hh, np.ones(64)), O.rmsnorm(hh))          # unit gain = weightless
    g = rng.uniform(0.5, 1.5, 64)
    np.testing.assert_allclose(O.rmsnorm(hh, g), O.rmsnorm(hh) * g, rtol=1e-15)  # per column, every row
    np.testing.assert_allclose(O.rmsnorm(7.0 * hh, g), O.rmsnorm(hh, g), rtol=1e-6)  # scale-free (up to eps)
    # the mean square is of h, not of g * h: a gain that zeroes a column leaves the others unchanged
    g0 = np.ones(64)
    g0[5] = 0.0
    x0 = O.rmsnorm(hh, g0)
    assert np.all(x0[:, 5] == 0) and np.array_equal(np.delete(x0, 5, 1), np.delete(O.rmsnorm(hh), 5, 1))


# ------------------------------------------------------------------------------- top-K
def test_topk_crafted_ties():
    assert O.topk_indices(np.zeros(16), 4) == [0, 1, 2, 3]
    assert O.topk_indices(np.array([1.0, 3.0, 3.0, 2.0]), 2) == [1, 2]
    assert O.topk_indices(np.array([1.0, 3.0, 3.0, 2.0]), 3) == [1, 2, 3]
    assert O.topk_indices(np.array([-1.0, -0.0, 0.0, -2.0]), 2) == [1, 2]


def test_topk_vs_lexsort_and_invariants():
    for E, K in [(16, 2), (256, 4), (256, 8), (512, 4), (64, 64)]:
        for _ in range(5):
            lg = np.round(RNG.normal(size=E), 1)    # many exact ties
            idx = O.topk_indices(lg, K)
            ref = list(np.lexsort((np.arange(E), -lg))[:K])
            assert idx == ref
            assert len(set(idx)) == K and all(0 <= e < E for e in idx)
            vals = lg[idx]
            assert (np.diff(vals) <= 0).all()
            w = O.topk_weights(lg, idx, True)
            assert w.sum() == pytest.approx(1.0, abs=1e-12)
            for i in range(K):
                for j in range(K):
                    assert w[i] / w[j] == pytest.approx(math.exp(vals[i] - vals[j]), rel=1e-12)
            wf = O.topk_weights(lg, idx, False)
            full = scipy.special.softmax(lg)
            np.testing.assert_allclose(wf, full[idx], rtol=1e-12)


# ------------------------------------------------------------------------------- experts
def _tiny_layer(seed=0):
    cfg = CONFIGS["tiny"]
    syn = Synth(cfg, seed)
    experts = {}
    for mat in ("gate", "up", "down"):
        q, s, b = syn.expert_mat(0, list(range(cfg.E)), mat)
        experts[mat] = (q.numpy(), s.numpy(), b.numpy())
    get = lambda e: tuple((experts[m][0][e], experts[m][1][e], experts[m][2][e]) for m in ("gate", "up", "down"))
    return cfg, syn, get


def test_k_equals_e_dense_equivalence():
    """K = E: the top-K layer equals the dense mixture r + sum_e softmax(l)_e FFN_e(x),
    computed here with no top-K code at all."""
    cfg, syn, get = _tiny_layer()
    x = syn.hidden(7, 1)[0].numpy()
    wr = syn.router(0).numpy()
    lg = O.router_logits(wr, x)
    p = scipy.special.softmax(lg)
    dense = O.f64(x).copy()
    for e in range(cfg.E):
        dense += p[e] * O.expert_ffn_packed(x, *get(e), cfg.bits, cfg.group)
    for renorm in (True, False):
        idx, w = O.route_topk(lg[None], cfg.E, renorm)
        y = O.moe_layer(x, x, idx, w, get, cfg.bits, cfg.group)
        np.testing.assert_allclose(y[0], dense, rtol=1e-12, atol=1e-12)


def test_one_hot_routing_is_single_expert():
    cfg, syn, get = _tiny_layer()
    x = syn.hidden(3, 1)[0].numpy()
    j = 11
    lg = np.zeros(cfg.E)
    lg[j] = 100.0
    idx, w = O.route_topk(lg[None], 1)
    assert idx[0].tolist() == [j] and w[0].tolist() == [1.0]
    y = O.moe_layer(x, x, idx, w, get, cfg.bits, cfg.group)
    single = O.f64(x) + O.expert_ffn_packed(x, *get(j), cfg.bits, cfg.group)
    np.testing.assert_array_equal(y[0], single)
    idx2, w2 = O.route_topk(lg[None], 2)
    assert idx2[0].tolist() == [j, 0]
    assert w2[0, 1] == pytest.approx(math.exp(-100.0) / (1 + math.exp(-100.0)), rel=1e-12)


def test_scalar_ffn_by_hand():
    Wg, Wu, Wd = np.array([[2.0]]), np.array([[3.0]]), np.array([[0.5]])
    o = O.expert_ffn(np.array([1.0]), Wg, Wu, Wd)
    silu2 = 2.0 / (1.0 + math.exp(-2.0))
    assert o[0] == pytest.approx(0.5 * silu2 * 3.0, rel=1e-15)
    # SiLU on the gate branch, not the up branch
    assert o[0] != pytest.approx(0.5 * 2.0 * (3.0 / (1.0 + math.exp(-3.0))), rel=1e-6)


def test_expert_ffn_matches_explicit_loops():
    """Small random expert, every product written as a Python loop (catches a transposed
    operand or a swapped gate/up)."""
    d, I = 8, 5
    Wg, Wu, Wd = RNG.normal(size=(I, d)), RNG.normal(size=(I, d)), RNG.normal(size=(d, I))
    x = RNG.normal(size=d)
    a = []
    for i in range(I):
        g = sum(Wg[i, c] * x[c] for c in range(d))
        u = sum(Wu[i, c] * x[c] for c in range(d))
        a.append(g / (1 + math.exp(-g)) * u)
    ref = [sum(Wd[j, i] * a[i] for i in range(I)) for j in range(d)]
    np.testing.assert_allclose(O.expert_ffn(x, Wg, Wu, Wd), ref, rtol=1e-12)


def test_combine_by_hand():
    o = np.array([[1.0, 2.0], [10.0, 20.0]])
    w = np.array([0.25, 0.75])
    r = np.array([100.0, 200.0])
    assert O.combine(o, w, r).tolist() == [100 + 0.25 + 7.5, 200 + 0.5 + 15.0]
    assert O.combine(o, w, r, shared=np.array([1.0, -1.0])).tolist() == [108.75, 214.5]


# ------------------------------------------------------------------------------- LoRA
def test_lora_zero_b_is_base_and_merge_identity():
    d, I, r, alpha = 64, 32, 4, 8.0
    Wg, Wu, Wd = RNG.normal(size=(I, d)), RNG.normal(size=(I, d)), RNG.normal(size=(d, I))
    x = RNG.normal(size=d)
    lora = {m: (RNG.normal(0, 0.02, (r, c)), RNG.normal(0, 0.02, (rw, r)))
            for m, (rw, c) in (("gate", (I, d)), ("up", (I, d)), ("down", (d, I)))}
    lora["alpha"] = alpha
    zero = {m: (lora[m][0], np.zeros_like(lora[m][1])) for m in ("gate", "up", "down")}
    zero["alpha"] = alpha
    np.testing.assert_array_equal(O.expert_ffn(x, Wg, Wu, Wd, zero), O.expert_ffn(x, Wg, Wu, Wd))
    merged = [W + (alpha / r) * lora[m][1] @ lora[m][0] for W, m in ((Wg, "gate"), (Wu, "up"), (Wd, "down"))]
    np.testing.assert_allclose(O.expert_ffn(x, Wg, Wu, Wd, lora), O.expert_ffn(x, *merged), rtol=1e-10, atol=1e-12)
    # the delta is scaled by alpha / rank (= 2 for rank 16, alpha 32)
    A, B = lora["gate"]
    assert np.allclose(O.lora_delta(A, B, alpha, x), 2.0 * (B @ (A @ x)))


# ------------------------------------------------------------------------------- prerouter
def _rand_head(d, E, H):
    return {"fc1_x": RNG.normal(size=(H, d)), "fc1_r": RNG.normal(size=(2 * E, H)),
            "fc1_b": RNG.normal(size=H), "fc2": RNG.normal(size=(E, H)), "fc2_b": RNG.normal(size=E),
            "lin_x": RNG.normal(size=(E, d)), "lin_r": RNG.normal(size=(2 * E, E)), "lin_b": RNG.normal(size=E)}


def test_router_on_basis_vectors_returns_columns():
    """logits = W_r x with x = e_j is column j of W_r, exactly (catches a transposed router)."""
    E, d = 16, 32
    W = RNG.normal(size=(E, d)).astype(np.float16)
    for j in (0, 7, 31):
        x = np.zeros(d)
        x[j] = 1.0
        assert O.router_logits(W, x).tolist() == W[:, j].astype(np.float64).tolist()
    X = np.eye(d)[[3, 9]]
    np.testing.assert_array_equal(O.router_logits(W, X), W[:, [3, 9]].T.astype(np.float64))


def test_prerouter_reduces_to_router():
    d, E, H, K = 32, 16, 8, 2
    pw = _rand_head(d, E, H)
    pw.update(fc2=np.zeros((E, H)), fc2_b=None, lin_r=np.zeros((2 * E, E)), lin_b=None)
    x = RNG.normal(size=d)
    got = O.prerouter_logits(x, [3, 5], [1, 2], pw, E)
    np.testing.assert_allclose(got, O.router_logits(pw["lin_x"], x), rtol=1e-13)


def test_prerouter_khot_gather_exact():
    """fc1_x = 0 and fc1 routing rows set to distinct constants: the pre-activation is the exact
    sum of the selected rows (cur rows m, prev rows E + m), read out through fc2 = I."""
    d, E, K = 16, 8, 3
    H = E
    fc1_r = np.array([[m + 1.0] * H for m in range(2 * E)])
    pw = {"fc1_x": np.zeros((H, d)), "fc1_r": fc1_r, "fc1_b": None, "fc2": np.eye(E), "fc2_b": None,
          "lin_x": np.zeros((E, d)), "lin_r": np.zeros((2 * E, E)), "lin_b": None}
    cur, prev = [6, 1, 3], [0, 7, 2]
    a = sum(m + 1.0 for m in cur) + sum(E + m + 1.0 for m in prev)
    got = O.prerouter_logits(RNG.normal(size=d), cur, prev, pw, E)
    np.testing.assert_allclose(got, [a * 0.5 * (1 + math.erf(a / math.sqrt(2)))] * E, rtol=1e-15)
    a0 = sum(m + 1.0 for m in cur)        # no previous token -> zero vector
    got0 = O.prerouter_logits(RNG.normal(size=d), cur, None, pw, E)
    np.testing.assert_allclose(got0, [a0 * 0.5 * (1 + math.erf(a0 / math.sqrt(2)))] * E, rtol=1e-15)


def test_prerouter_by_hand():
    """d=2, E=2, K=1, H=1 worked out by hand: z = [x0, x1, cur0, cur1, prev0, prev1]."""
    x = np.array([1.0, -2.0])
    pw = {"fc1_x": np.array([[0.5, 0.25]]), "fc1_r": np.array([[1.0], [2.0], [3.0], [4.0]]),
          "fc1_b": np.array([0.1]), "fc2": np.array([[2.0], [-1.0]]), "fc2_b": np.array([0.0, 1.0]),
          "lin_x": np.array([[1.0, 0.0], [0.0, 1.0]]),
          "lin_r": np.array([[1.0, 0.0], [0.0, 1.0], [5.0, 6.0], [7.0, 8.0]]), "lin_b": np.array([0.5, 0.0])}
    # cur = [1] -> z[3] = 1 ; prev = [0] -> z[4] = 1
    a = 0.5 * 1 + 0.25 * -2 + 2.0 + 3.0 + 0.1          # = 5.1
    g = 0.5 * a * (1 + math.erf(a / math.sqrt(2)))
    want = [2 * g + 0 + (1.0 + 0.0 + 5.0) + 0.5, -g + 1 + (-2.0 + 1.0 + 6.0)]
    np.testing.assert_allclose(O.prerouter_logits(x, [1], [0], pw, 2), want, rtol=1e-15)


# ------------------------------------------------------------------------------- grouping
def test_group_by_expert_brute_force():
    for T, K, E in [(256, 4, 256), (7, 2, 16), (1, 1, 4)]:
        idx = np.array([RNG.choice(E, size=K, replace=False) for _ in range(T)])
        counts, off, perm = O.group_by_expert(idx, E)
        ref = [p for _, p in sorted((int(e), p) for p, e in enumerate(idx.reshape(-1)))]
        assert perm.tolist() == ref
        assert off[-1] == T * K and (np.diff(off) == counts).all()
        assert counts.tolist() == np.bincount(idx.reshape(-1), minlength=E).tolist()


# ------------------------------------------------------------------------------- bytes
def test_expert_byte_accounting():
    fx = read_fixture("byte_accounting.txt")
    for name, v in fx.items():
        assert CONFIGS[name].expert_bytes() == int(v[0][0])
    assert CONFIGS["large-int4"].expert_bytes() == 6.75 * 2 ** 20


# ------------------------------------------------------------------------------- chain
def test_chain_single_layer_is_routed_layer():
    cfg, syn, get = _tiny_layer()
    h = syn.hidden(11, 1)[0].numpy()
    st = O.ChainState(1)
    hL, st2, tr = O.chain_token(h, st, E=cfg.E, K=cfg.K, bits=cfg.bits, group=cfg.group,
                                router_get=lambda l: syn.router(l).numpy(), head_get=lambda l: None,
                                expert_get=lambda l, e: get(e))
    x = O.rmsnorm(h)
    idx, w = O.route_topk(O.router_logits(syn.router(0).numpy(), x)[None], cfg.K)
    y = O.moe_layer(x, h, idx, w, get, cfg.bits, cfg.group)
    np.testing.assert_array_equal(hL, O.to_f16_f64(y[0]))
    assert st2.prev[0].tolist() == idx[0].tolist()


def _hand_chain_stack(fx):
    """The hand-worked stack of prerouted_chain_hand.txt: zero experts, permutation routers,
    heads that read only the two K-hot vectors."""
    d, E, I, H, bits = fx["d"], fx["E"], fx["d_ff"], fx["H"], fx["bits"]
    zero_up = (np.zeros((I, d * bits // 32), np.uint32), np.zeros((I, d // fx["group"]), np.float16),
               np.zeros((I, d // fx["group"]), np.float16))
    zero_dn = (np.zeros((d, I * bits // 32), np.uint32), np.zeros((d, I // fx["group"]), np.float16),
               np.zeros((d, I // fx["group"]), np.float16))

    def head_get(l):
        if l not in fx["heads"]:
            return None
        return {"fc1_x": np.zeros((H, d), np.float16), "fc1_r": np.zeros((2 * E, H), np.float16), "fc1_b": None,
                "fc2": np.zeros((E, H), np.float16), "fc2_b": None, "lin_x": np.zeros((E, d), np.float16),
                "lin_r": fx["lin_r"][l], "lin_b": None}

    return dict(E=E, K=fx["K"], bits=bits, group=fx["group"], router_get=lambda l: fx["router"][l],
                head_get=head_get, expert_get=lambda l, e: (zero_up, zero_up, zero_dn))


def test_prerouted_chain_hand_worked():
    """Three tokens through the hand-worked 4-layer stack: which routing each layer uses (own
    router at t = 0, after a head-less layer and at layer 0; else the head of layer l-1 at t-1),
    the head's current / previous K-hot inputs, and where its prediction lands (layer l+1, token
    t+1).  Each of these slips changes an expected line: a prediction stored for layer l instead
    of l+1, the two K-hot vectors swapped, the previous-token vector filled at t = 0, the next
    layer's routing fed to the head, a layer after a head-less layer not routing itself."""
    fx = golden_io.hand_chain()
    kw = _hand_chain_stack(fx)
    r = math.sqrt(np.mean(fx["h"][0].astype(np.float64) ** 2) + O.RMS_EPS)
    st = O.ChainState(fx["L"])
    prev_idx = [None] * fx["L"]
    for t in range(fx["h"].shape[0]):
        h = fx["h"][t]
        hL, new, tr = O.chain_token(h, st, **kw)
        for l in range(fx["L"]):
            src, idx, w = fx["route"][(t, l)]
            assert tr[l].idx.tolist() == idx, (t, l)
            np.testing.assert_allclose(tr[l].w, w, rtol=0, atol=1e-15)
            assert (tr[l].route_logits is not None) == (src == "router"), (t, l)
            if src == "router":
                np.testing.assert_allclose(tr[l].route_logits, np.array(fx["router_num"][(t, l)]) / r, rtol=1e-15)
            np.testing.assert_array_equal(tr[l].y, h.astype(np.float64))  # zero experts: y = h
            if l in fx["heads"]:
                cur, prev = fx["head_in"][(t, l)]
                assert sorted(cur) == sorted(idx) and prev == prev_idx[l], (t, l)
                np.testing.assert_array_equal(tr[l].head_logits, fx["head_logits"][(t, l)])
                pidx, pw = fx["pred"][(t, l + 1)]
                assert new.pred[l + 1][0].tolist() == pidx, (t, l)
                np.testing.assert_allclose(new.pred[l + 1][1], pw, rtol=0, atol=1e-15)
            else:
                assert tr[l].head_logits is None and (l + 1 >= fx["L"] or new.pred[l + 1] is None)
            prev_idx[l] = idx
        assert new.pred[0] is None
        np.testing.assert_array_equal(hL, h.astype(np.float64))
        st = new


def test_chain_threads_layer_outputs():
    """Three head-less layers: the chain equals three routed layers applied in turn, each on
    rmsnorm of the float16-rounded output of the one before (every layer routes itself)."""
    cfg, syn, get = _tiny_layer()
    h = syn.hidden(5, 1)[0].numpy()
    routers = [syn.router(0).numpy(), syn.router(0).numpy()[::-1].copy(), -syn.router(0).numpy()]
    hL, _, tr = O.chain_token(h, O.ChainState(3), E=cfg.E, K=cfg.K, bits=cfg.bits, group=cfg.group,
                              router_get=lambda l: routers[l], head_get=lambda l: None,
                              expert_get=lambda l, e: get(e))
    cur = O.f64(h)
    for l in range(3):
        x = O.rmsnorm(cur)
        idx, w = O.route_topk(O.router_logits(routers[l], x)[None], cfg.K)
        assert tr[l].idx.tolist() == idx[0].tolist()
        cur = O.to_f16_f64(O.moe_layer(x, cur, idx, w, get, cfg.bits, cfg.group)[0])
        np.testing.assert_array_equal(tr[l].y, cur)
    np.testing.assert_array_equal(hL, cur)


# ------------------------------------------------------------------ ReLU activation-sparse expert
def _hand_relu_mats():
    fx = read_fixture("relu_sparse_hand.txt")
    bits, group = int(fx["bits"][0][0]), int(fx["group"][0][0])

    def mat(name):
        q = np.array([[int(w, 16) for w in row] for row in fx[name + "_words"]], dtype=np.uint32)
        sb = np.array([[float(v) for v in row] for row in fx[name + "_sb"]])
        return q, sb[:, 0::2].astype(np.float16), sb[:, 1::2].astype(np.float16)

    return fx, bits, group, mat("gate"), mat("up"), mat("down")


def test_relu_sparse_expert_by_hand():
    """Hand-worked example: neuron 0's gate is negative (its ReLU output is exactly zero, so its
    down row never contributes), neuron 1 is on; the output pins the neuron-major orientation of
    the down projection and its groups along d."""
    fx, bits, group, gate, up, down = _hand_relu_mats()
    x = np.ones(int(fx["d"][0][0]))
    o, a = O.expert_ffn_relu_packed(x, gate, up, down, bits, group)
    assert a.tolist() == [float(v) for v in fx["act"][0]]
    assert int(O.active_neurons(a)) == int(fx["n_active"][0][0])
    assert o.tolist() == [float(v) for v in fx["out"][0]]


def test_relu_expert_matches_explicit_loops():
    """Small random expert with every product as a Python loop and ReLU as a branch; the down
    matrix is indexed [neuron][output] (catches a transposed down or ReLU on the up branch)."""
    d, I = 8, 6
    Wg, Wu, WdT = RNG.normal(size=(I, d)), RNG.normal(size=(I, d)), RNG.normal(size=(I, d))
    x = RNG.normal(size=d)
    a = []
    for i in range(I):
        g = sum(Wg[i, c] * x[c] for c in range(d))
        u = sum(Wu[i, c] * x[c] for c in range(d))
        a.append(g * u if g > 0 else 0.0)
    ref = [sum(a[i] * WdT[i, j] for i in range(I)) for j in range(d)]
    o, av = O.expert_ffn_relu(x, Wg, Wu, WdT)
    np.testing.assert_allclose(o, ref, rtol=1e-12)
    assert int(O.active_neurons(av)) == sum(1 for v in a if v != 0.0)
    assert 0 < sum(1 for v in a if v != 0.0) < I      # the draw has neurons on and off


def test_relu_expert_all_off_and_all_on():
    """Every gate negative: the output is exactly zero and no neuron is active.  Every gate
    positive: ReLU is the identity and the unit is the bilinear product WdT^T((Wg x)(Wu x))."""
    d, I = 16, 8
    x = np.abs(RNG.normal(size=d)) + 0.1
    Wpos = np.abs(RNG.normal(size=(I, d)))
    Wu, WdT = RNG.normal(size=(I, d)), RNG.normal(size=(I, d))
    o, a = O.expert_ffn_relu(x, -Wpos, Wu, WdT)
    assert (o == 0).all() and int(O.active_neurons(a)) == 0
    o, a = O.expert_ffn_relu(x, Wpos, Wu, WdT)
    np.testing.assert_allclose(o, np.einsum("i,id->d", (Wpos @ x) * (Wu @ x), WdT), rtol=1e-12)
    assert int(O.active_neurons(a)) == I


# ------------------------------------------------------------------ expert streaming
def test_prefetch_window_worked_example():
    """The pages' own numbers: 5 GB/s, 2 MB experts, a 2 ms window -> 5 experts, 1.2 ms wait for 8."""
    fx = read_fixture("prefetch_window.txt")
    g = lambda k: float(fx[k][0][0])
    bw, X, Y = g("bandwidth_Bps"), g("expert_bytes"), g("window_s")
    assert X / bw == pytest.approx(g("t_one_s"), rel=1e-12)
    assert O.experts_per_window(Y, bw, X) == int(g("n_prefetch"))
    assert O.stall_time(int(g("needed")), Y, bw, X) == pytest.approx(g("stall_s"), rel=1e-12)
    assert O.stall_time(int(g("needed_small")), Y, bw, X) == g("stall_small_s")
    # one byte of bandwidth less and the fifth expert no longer fits
    assert O.experts_per_window(Y, bw * (1 - 1e-6), X) == 4


def test_pool_plan_hand_sequence():
    fx = read_fixture("pool_lru_hand.txt")
    st = O.PoolState(3)
    ints = lambda s: [int(v) for v in s.split(",")]
    for row in fx["step"]:
        tok, sel, slots, pool, stamps, cp = row
        slot, copies = O.pool_plan(st, ints(sel), int(tok))
        assert slot == ints(slots)
        assert st.expert == ints(pool) and st.stamp == ints(stamps)
        want = [] if cp == "-" else [tuple(int(v) for v in c.split(":")) for c in cp.split(",")]
        assert copies == want


def test_pool_plan_invariants_random():
    """Over a long random sequence with reuse: every selected expert sits in exactly the slot
    returned, no expert is in two slots, and copies happen exactly for the selected experts that
    were not pooled before."""
    rng = np.random.default_rng(7)
    E, K, S = 40, 4, 9
    st = O.PoolState(S)
    for t in range(300):
        sel = list(rng.choice(E if t % 3 else 12, size=K, replace=False))
        before = set(e for e in st.expert if e >= 0)
        slot, copies = O.pool_plan(st, sel, t)
        for k, e in enumerate(sel):
            assert st.expert[slot[k]] == e and st.stamp[slot[k]] == t
        pooled = [e for e in st.expert if e >= 0]
        assert len(pooled) == len(set(pooled))
        assert sorted(e for _, _, e in copies) == sorted(e for e in sel if e not in before)
        assert len(set(slot)) == K
