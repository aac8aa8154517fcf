"""GPU parity of moe_decode_step (the whole token in one persistent kernel) against the fp64
oracle's prerouted chain, and against the per-layer C-ABI path on the same weights."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import moe_synth as S
import oracle as O
from parity_util import ExpertCache, assert_rows_close, device_layer, log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def M():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int4_expert_ffn_amd as m
    return m


def build(M, cfg, heads: bool):
    from int4_expert_ffn_amd.chain import DecodeStack, LayerWeights
    syn = S.Synth(cfg)
    layers, heads_cpu = [], []
    for l in range(cfg.L):
        head = None
        if heads and l < cfg.L - 1:
            head = M.PrerouterWeights(syn.head(l, DEV))
            heads_cpu.append({k: v.numpy() for k, v in syn.head(l, "cpu").items()})
        layers.append(LayerWeights(device_layer(syn, l, DEV), syn.router(l, DEV), head))
    routers_cpu = [syn.router(l, "cpu").numpy() for l in range(cfg.L)]
    return syn, layers, heads_cpu, routers_cpu


def run_oracle(cfg, syn, heads_cpu, routers_cpu, tokens):
    caches = [ExpertCache(syn, l) for l in range(cfg.L)]
    st = O.ChainState(cfg.L)
    out = []
    for h0 in tokens:
        hL, st, tr = O.chain_token(h0.numpy(), st, E=cfg.E, K=cfg.K, bits=cfg.bits, group=cfg.group,
                                   router_get=lambda l: routers_cpu[l],
                                   head_get=lambda l: heads_cpu[l] if l < len(heads_cpu) else None,
                                   expert_get=lambda l, e: caches[l](e))
        out.append((hL, tr))
    return out


def screened_tokens(cfg, syn, routers_cpu, n, seed0=7000, gap=1e-4):
    """n hidden states whose oracle routing has every adjacent gap among the top K+1 logits of
    every layer at least `gap` (the rule for bit-exact indices); a token that fails it is redrawn
    with the next seed.  Only for stacks without heads, whose tokens do not depend on each other."""
    caches = [ExpertCache(syn, l) for l in range(cfg.L)]
    out, seed = [], seed0
    while len(out) < n:
        h0 = syn.hidden(seed, 1)[0]
        seed += 1
        _, _, tr = O.chain_token(h0.numpy(), O.ChainState(cfg.L), E=cfg.E, K=cfg.K, bits=cfg.bits, group=cfg.group,
                                 router_get=lambda l: routers_cpu[l], head_get=lambda l: None,
                                 expert_get=lambda l, e: caches[l](e))
        if min(O.topk_gaps(t.route_logits, cfg.K).min() for t in tr) >= gap:
            out.append(h0)
    log(f"{len(out)} tokens after {seed - seed0 - len(out)} redraws")
    return out


def check_against_oracle(cfg, ref, got_h, got_routes):
    """Per token: every layer's routing equal to the oracle's until a near-tie lets the chains
    diverge (then the rest is not compared), and the final hidden state within tolerance."""
    prev_tr = None
    for t, ((hL, tr), h, routes) in enumerate(zip(ref, got_h, got_routes)):
        for l in range(cfg.L):
            if not np.array_equal(routes[l], tr[l].idx):
                src = tr[l].route_logits if tr[l].route_logits is not None else prev_tr[l - 1].head_logits
                log(f"token {t} layer {l}: routing {routes[l]} vs oracle {tr[l].idx}")
                assert O.topk_gaps(src, cfg.K).min() < 1e-4, "routing differs away from a tie"
                return t
        assert_rows_close(h, hL[None], what=f"token {t} output")
        prev_tr = tr
    return len(ref)


CASES = {
    "decode35b": (replace(S.CONFIGS["decode35b"], L=4), True),
    "widek8": (replace(S.CONFIGS["widek8"], L=3), False),
    "large-int4": (replace(S.CONFIGS["large-int4"], L=2), False),
    "large-int2": (replace(S.CONFIGS["large-int2"], L=2), False),
    # four router rows per workgroup: more than LDS stages, so the router phase reads its rows from memory
    "widek8-E1024": (replace(S.CONFIGS["widek8"], L=2, E=1024), False),
}


@pytest.mark.parametrize("name", list(CASES))
def test_decode_step_matches_oracle_chain(M, name):
    from int4_expert_ffn_amd.chain import DecodeStack
    cfg, heads = CASES[name]
    syn, layers, heads_cpu, routers_cpu = build(M, cfg, heads)
    stack = DecodeStack(layers, cfg.K, DEV)
    if heads:   # the chain carries state from token to token: near-ties end the comparison instead
        tokens = [syn.hidden(7000 + t, 1)[0] for t in range(4)]
    else:
        tokens = screened_tokens(cfg, syn, routers_cpu, 4)
    got_h, got_r = [], []
    for t, h0 in enumerate(tokens):
        stack.step(t, h0.to(DEV))
        torch.cuda.synchronize()
        assert stack.step_error_word() == 0
        got_h.append(stack.h[cfg.L].float().cpu().numpy()[None])
        got_r.append(stack.route_idx[t % 3].cpu().numpy())
        log(f"{name} token {t}: routing {[r.tolist() for r in got_r[-1]]}")
    ref = run_oracle(cfg, syn, heads_cpu, routers_cpu, tokens)
    n = check_against_oracle(cfg, ref, got_h, got_r)
    assert n >= 2, "too few tokens compared"


@pytest.mark.parametrize("name", ["decode35b", "widek8"])
def test_decode_step_equals_per_layer_path(M, name):
    """Same weights, same tokens: the persistent kernel and the per-layer calls pick the same
    experts and agree on every output within the tolerance, token after token (without heads,
    every layer of the per-layer path routes itself at every token)."""
    from int4_expert_ffn_amd.chain import DecodeStack
    cfg, heads = CASES[name]
    syn, layers, _, _ = build(M, cfg, heads)
    a = DecodeStack(layers, cfg.K, DEV)
    b = DecodeStack(layers, cfg.K, DEV)
    for t in range(6):
        h0 = syn.hidden(8100 + t, 1)[0].to(DEV)
        ya = a.step(t, h0).float().cpu().numpy()
        yb = b.token(t, h0).float().cpu().numpy()
        torch.cuda.synchronize()
        ra, rb = a.route_idx[t % 3].cpu().numpy(), b.route_idx[t % 3].cpu().numpy()
        if not np.array_equal(ra, rb):
            log(f"token {t}: paths diverge at a routing tie ({ra.tolist()} vs {rb.tolist()})")
            break
        assert_rows_close(ya[None], yb[None], what=f"token {t} step vs per-layer")
    assert a.step_error_word() == 0


def test_decode_step_deterministic_and_mixable(M):
    """Two fresh stacks fed the same tokens through the persistent kernel give bit-identical outputs
    and routing.  A third stack that runs the first token through the per-layer calls and the
    rest through the persistent kernel (the routing state carries over between the two paths) picks
    the same experts and agrees within the tolerance.  The two paths differ in rounding (the
    persistent kernel exchanges the SwiGLU outputs with a 16-bit significand), so they are not
    compared bit for bit."""
    from int4_expert_ffn_amd.chain import DecodeStack
    cfg, heads = CASES["decode35b"]
    syn, layers, _, _ = build(M, cfg, heads)
    a = DecodeStack(layers, cfg.K, DEV)
    a2 = DecodeStack(layers, cfg.K, DEV)
    b = DecodeStack(layers, cfg.K, DEV)
    for t in range(5):
        h0 = syn.hidden(8200 + t, 1)[0].to(DEV)
        ya = a.step(t, h0).clone()
        ya2 = a2.step(t, h0).clone()
        yb = (b.token(t, h0) if t == 0 else b.step(t, h0)).clone()
        torch.cuda.synchronize()
        assert torch.equal(ya, ya2), f"token {t}: persistent kernel not deterministic"
        assert torch.equal(a.route_idx[t % 3], a2.route_idx[t % 3])
        if t >= 1:
            assert torch.equal(a.route_idx[t % 3], b.route_idx[t % 3]), f"token {t}: routing after the switch"
        assert_rows_close(yb.float().cpu().numpy()[None], ya.float().cpu().numpy()[None],
                          what=f"token {t} mixed vs persistent")
    assert a.step_error_word() == 0 and a2.step_error_word() == 0 and b.step_error_word() == 0


TIE_CASES = {
    "widek8": replace(S.CONFIGS["widek8"], L=2),            # E 256, K 8: 4 logits per lane
    "large-int4": replace(S.CONFIGS["large-int4"], L=2),    # E 512, K 4: 8 per lane
    "widek8-E1024": replace(S.CONFIGS["widek8"], L=2, E=1024),  # 16 per lane
}


@pytest.mark.parametrize("renorm", [True, False])
@pytest.mark.parametrize("name", list(TIE_CASES))
def test_decode_step_topk_exact_ties(M, name, renorm):
    """Router rows repeated in runs of three, so every logit occurs three times (bit-identical
    dot products, in the kernel as in float64): the top-K takes whole runs and then the
    lower-indexed members of the run cut at K, in the oracle's order (larger logit first, equal
    logits by lower expert index).  renorm False: weights from the softmax over all E logits.
    Tokens are screened for gaps between distinct logits only."""
    from int4_expert_ffn_amd.chain import DecodeStack, LayerWeights
    cfg = TIE_CASES[name]
    syn = S.Synth(cfg)
    rep = (np.arange(cfg.E) // 3) * 3
    routers_cpu = [syn.router(l, "cpu").numpy()[rep] for l in range(cfg.L)]
    layers = [LayerWeights(device_layer(syn, l, DEV), torch.from_numpy(routers_cpu[l]).to(DEV), None)
              for l in range(cfg.L)]
    stack = DecodeStack(layers, cfg.K, DEV, renorm=renorm)
    caches = [ExpertCache(syn, l) for l in range(cfg.L)]

    def oracle(h0):
        return O.chain_token(h0.numpy(), O.ChainState(cfg.L), E=cfg.E, K=cfg.K, bits=cfg.bits, group=cfg.group,
                             router_get=lambda l: routers_cpu[l], head_get=lambda l: None,
                             expert_get=lambda l, e: caches[l](e), renorm=renorm)

    compared, seed = 0, 9100
    while compared < 2:
        assert seed < 9140, "no token with distinct logits well apart"
        h0 = syn.hidden(seed, 1)[0]
        seed += 1
        hL, _, tr = oracle(h0)
        distinct = [np.unique(t.route_logits)[::-1][: cfg.K + 1] for t in tr]
        if min(np.min(u[:-1] - u[1:]) for u in distinct) < 1e-4:
            continue
        assert any(len(set(t.route_logits[t.idx].tolist())) < cfg.K for t in tr), "no tie inside the top-K"
        stack.step(compared, h0.to(DEV))
        torch.cuda.synchronize()
        assert stack.step_error_word() == 0
        slot = compared % 3
        for l, t in enumerate(tr):
            got_i = stack.route_idx[slot, l].cpu().numpy()
            got_w = stack.route_w[slot, l].cpu().numpy().astype(np.float64)
            assert np.array_equal(got_i, t.idx), f"layer {l}: {got_i.tolist()} vs oracle {t.idx.tolist()}"
            assert np.allclose(got_w, t.w, rtol=1e-3, atol=1e-6), f"layer {l}: weights {got_w} vs {t.w}"
        assert_rows_close(stack.h[cfg.L].float().cpu().numpy()[None], hL[None], what=f"{name} output")
        log(f"{name} renorm={renorm} token {compared}: routing {[t.idx.tolist() for t in tr]}")
        compared += 1


@pytest.mark.parametrize("name", list(CASES))
def test_decode_step_grid_matches_plan_for_this_device(M, name):
    """The grid a launch uses on this device is the host-only plan for its compute-unit count."""
    from int4_expert_ffn_amd.chain import DecodeStack
    cfg, heads = CASES[name]
    _, layers, _, _ = build(M, cfg, heads)
    stack = DecodeStack(layers, cfg.K, DEV)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    st = stack._step_state()[1]
    assert stack.grid() == M.moe_decode_step_grid_for(st, cus)
    assert 1 <= stack.grid() <= cus


@pytest.mark.parametrize("name", ["decode35b", "widek8"])
def test_decode_step_stamped(M, name):
    """moe_decode_step_stamped gives bit-identical outputs and routing to the plain launch, and its
    phase stamps are ordered: inside a workgroup, layer start <= h_l unpacked <= h_l seen by the
    compute waves <= SwiGLU outputs stored <= down phase <= layer output stored; across the grid,
    no workgroup has h_{l+1} before the last workgroup stored its rows of it (a real exchange), and
    none has all SwiGLU outputs before the last one stored its own."""
    from int4_expert_ffn_amd.chain import DecodeStack
    cfg, heads = CASES[name]
    syn, layers, _, _ = build(M, cfg, heads)
    a, b = DecodeStack(layers, cfg.K, DEV), DecodeStack(layers, cfg.K, DEV)
    G = a.grid()
    assert G > 0
    st = torch.zeros((G, cfg.L, 16), dtype=torch.int64, device=DEV)
    for t in range(3):
        h0 = syn.hidden(8300 + t, 1)[0].to(DEV)
        ya = a.step(t, h0).clone()
        yb = b.step(t, h0, stamps=st).clone()
        torch.cuda.synchronize()
        assert torch.equal(ya, yb) and torch.equal(a.route_idx[t % 3], b.route_idx[t % 3])
        s = st.cpu().numpy()
        assert (s > 0).all()
        for x, y in ((0, 1), (1, 3), (3, 4), (4, 5), (2, 5), (5, 6)):
            assert (s[:, :, y] >= s[:, :, x]).all(), (x, y)
        for l in range(cfg.L - 1):
            assert s[:, l + 1, 1].min() >= s[:, l, 6].max(), l
        assert (s[:, :, 2].min(axis=0) >= s[:, :, 4].max(axis=0)).all()
    assert a.step_error_word() == 0 and b.step_error_word() == 0


def given_routing(syn, cfg, t):
    """Seeded routing for every layer of token t: the oracle's top-K (renormalised softmax) of N(0,1)
    logits, i.e. K distinct experts drawn uniformly per layer."""
    lg = syn.logits(7000 + t, cfg.L).numpy()
    idx, w = O.route_topk(lg, cfg.K)
    return idx.astype(np.int32), w.astype(np.float32)


@pytest.mark.parametrize("name", list(CASES))
def test_decode_step_given_routing(M, name):
    """MOE_DECODE_GIVEN_ROUTING: the expert FFN steps alone on caller-supplied routing.  Every layer
    output equals the oracle layer applied to the kernel's own input of that layer with the given
    experts and weights; the routing slots are left as the caller wrote them, whatever heads and
    routers the descriptors carry."""
    from int4_expert_ffn_amd.chain import DecodeStack
    cfg, heads = CASES[name]
    syn, layers, _, _ = build(M, cfg, heads)
    stack = DecodeStack(layers, cfg.K, DEV)
    caches = [ExpertCache(syn, l) for l in range(cfg.L)]
    hl = torch.empty((cfg.L + 1, cfg.d), dtype=torch.float16, device=DEV)
    stack.route_idx.fill_(-7)
    stack.route_w.fill_(-7.0)
    for t in range(3):
        idx, w = given_routing(syn, cfg, t)
        stack.set_routing(t, torch.from_numpy(idx).to(DEV), torch.from_numpy(w).to(DEV))
        before_i, before_w = stack.route_idx.clone(), stack.route_w.clone()
        h0 = syn.hidden(9100 + t, 1)[0]
        out = stack.step(t, h0.to(DEV), h_layers=hl, given_routing=True)
        torch.cuda.synchronize()
        assert stack.step_error_word() == 0
        assert torch.equal(stack.route_idx, before_i) and torch.equal(stack.route_w, before_w), \
            "the kernel wrote routing state"
        H = hl.cpu().numpy()
        assert np.array_equal(H[0], h0.numpy()) and np.array_equal(H[cfg.L], out.cpu().numpy())
        for l in range(cfg.L):
            x = O.rmsnorm(H[l])
            y_ref = O.f64(H[l]).copy()
            for k in range(cfg.K):
                y_ref += float(w[l][k]) * O.expert_ffn_packed(x, *caches[l](idx[l][k]), bits=cfg.bits, group=cfg.group)
            assert_rows_close(H[l + 1][None], y_ref[None], what=f"{name} t{t} layer {l} (given routing)")
    log(f"{name}: given routing checked at all {cfg.L} layers of 3 tokens")


# ------------------------------------------------------------------------- RMS norm with a gain
@pytest.mark.parametrize("d", [2048, 4096, 264])
@pytest.mark.parametrize("gained", [True, False])
def test_rmsnorm_matches_oracle(M, d, gained):
    """moe_rmsnorm against the oracle, rows within the tolerance; in place as well."""
    cfg = replace(S.CONFIGS["decode35b"], d=d)
    syn = S.Synth(cfg)
    T = 7
    h = syn.hidden(4242, T)
    g = syn.norm_gain(3) if gained else None
    x = torch.empty((T, d), dtype=torch.float16, device=DEV)
    hd = h.to(DEV)
    M.moe_rmsnorm(T, d, hd, None if g is None else g.to(DEV), x)
    ref = O.rmsnorm(h.numpy(), None if g is None else g.numpy())
    assert_rows_close(x.float().cpu().numpy(), ref, what=f"rmsnorm d {d}")
    M.moe_rmsnorm(T, d, hd, None if g is None else g.to(DEV), hd)     # x may be h
    torch.cuda.synchronize()
    assert torch.equal(hd, x)


def gained_stack(M, cfg, heads):
    from int4_expert_ffn_amd.chain import LayerWeights
    syn, layers, heads_cpu, routers_cpu = build(M, cfg, heads)
    gains = [syn.norm_gain(l) for l in range(cfg.L)]
    layers = [LayerWeights(lw.experts, lw.router, lw.head, gains[l].to(DEV)) for l, lw in enumerate(layers)]
    return syn, layers, heads_cpu, routers_cpu, [g.numpy() for g in gains]


@pytest.mark.parametrize("name", ["decode35b", "widek8", "large-int4"])
def test_decode_step_norm_gain_layer_by_layer(M, name):
    """Layers with an input-norm gain (x = g * h / rms(h)) through the persistent kernel: per
    token and layer, the routing a self-routed layer chose equals the oracle's top-K of the gained
    input, the layer output equals the oracle layer on the kernel's own input, and every head
    predicts the oracle head's top-K (near ties excepted)."""
    from int4_expert_ffn_amd.chain import DecodeStack
    from test_fullsize_gpu import _check_topk
    cfg, heads = CASES[name]
    syn, layers, heads_cpu, routers_cpu, gains = gained_stack(M, cfg, heads)
    stack = DecodeStack(layers, cfg.K, DEV)
    caches = [ExpertCache(syn, l) for l in range(cfg.L)]
    hl = torch.empty((cfg.L + 1, cfg.d), dtype=torch.float16, device=DEV)
    prev_idx, routed, predicted = None, 0, 0
    for t in range(3):
        h0 = syn.hidden(9300 + t, 1)[0]
        out = stack.step(t, h0.to(DEV), h_layers=hl)
        torch.cuda.synchronize()
        assert stack.step_error_word() == 0
        H = hl.cpu().numpy()
        assert np.array_equal(H[0], h0.numpy()) and np.array_equal(H[cfg.L], out.cpu().numpy())
        idx = stack.route_idx[t % 3].cpu().numpy()
        w = stack.route_w[t % 3].cpu().numpy()
        nxt_idx = stack.route_idx[(t + 1) % 3].cpu().numpy()
        nxt_w = stack.route_w[(t + 1) % 3].cpu().numpy()
        for l in range(cfg.L):
            x = O.rmsnorm(H[l], gains[l])
            if t == 0 or l == 0 or not heads:
                routed += _check_topk(O.router_logits(routers_cpu[l], x), idx[l], w[l], cfg.K, f"{name} t{t} l{l}")
            y_ref = O.f64(H[l]).copy()
            for k in range(cfg.K):
                y_ref += float(w[l][k]) * O.expert_ffn_packed(x, *caches[l](idx[l][k]), bits=cfg.bits, group=cfg.group)
            assert_rows_close(H[l + 1][None], y_ref[None], what=f"{name} t{t} layer {l} (gained)")
            if heads and l + 1 < cfg.L:
                lg = O.prerouter_logits(x, idx[l], None if t == 0 else prev_idx[l], heads_cpu[l], cfg.E)
                predicted += _check_topk(lg, nxt_idx[l + 1], nxt_w[l + 1], cfg.K, f"{name} t{t} head {l}")
        prev_idx = idx
    log(f"{name} gained: {routed} router top-Ks, {predicted} head predictions compared")
    assert routed >= 1


@pytest.mark.parametrize("name", ["decode35b", "widek8"])
def test_norm_gain_step_matches_per_layer_path(M, name):
    """The per-layer calls (moe_rmsnorm, then the calls on x) and the persistent kernel (the gain
    applied inside) pick the same experts and agree within the tolerance, token by token; for the
    stack without heads this also exercises the per-layer path's own routing at every layer."""
    from int4_expert_ffn_amd.chain import DecodeStack
    cfg, heads = CASES[name]
    syn, layers, _, _, _ = gained_stack(M, cfg, heads)
    a = DecodeStack(layers, cfg.K, DEV)
    b = DecodeStack(layers, cfg.K, DEV)
    for t in range(4):
        h0 = syn.hidden(9400 + t, 1)[0].to(DEV)
        ya = a.step(t, h0).clone()
        yb = b.token(t, h0).clone()
        torch.cuda.synchronize()
        ra, rb = a.route_idx[t % 3].cpu().numpy(), b.route_idx[t % 3].cpu().numpy()
        if not np.array_equal(ra, rb):
            log(f"{name} token {t}: paths diverge at a routing tie ({ra.tolist()} vs {rb.tolist()})")
            break
        assert_rows_close(ya.float().cpu().numpy()[None], yb.float().cpu().numpy()[None], what=f"{name} token {t}")
    assert a.step_error_word() == 0
