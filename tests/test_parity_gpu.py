"""GPU parity: every C-ABI call against the fp64 oracle on the same seeded inputs.

Bar: expert indices bit-exact (tokens drawn with top-(K+1) logit gaps >= 1e-4); float outputs per
token row within max|y - y_ref| <= 2e-3 * max|y_ref| (float16 in, float32 accumulation)."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import moe_synth as S
import oracle as O
from parity_util import (ExpertCache, assert_rows_close, device_layer, gap_tokens, log)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def M():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int4_expert_ffn_amd as m
    return m


def ws_for(M, T, K, ex):
    return torch.empty(M.moe_expert_ffn_workspace_size(T, K, ex), dtype=torch.uint8, device=DEV)


# ------------------------------------------------------------------------------------ generator
def test_generator_same_on_gpu_and_cpu(M):
    syn = S.Synth(S.CONFIGS["decode35b"])
    for m in S.MATS:
        g = syn.expert_mat(3, [0, 255], m, DEV)
        c = syn.expert_mat(3, [0, 255], m, "cpu")
        for a, b in zip(g, c):
            assert torch.equal(a.cpu(), b)
    hg, hc = syn.head(1, DEV), syn.head(1, "cpu")
    for k in hc:
        assert torch.equal(hg[k].cpu(), hc[k]), k
    assert torch.equal(syn.hidden(5, 3, DEV).cpu(), syn.hidden(5, 3))
    syn2 = S.Synth(S.CONFIGS["large-int2"])
    for a, b in zip(syn2.expert_mat(0, [511], "down", DEV), syn2.expert_mat(0, [511], "down")):
        assert torch.equal(a.cpu(), b)


# ------------------------------------------------------------------------------------ top-K
@pytest.mark.parametrize("E,K", [(16, 2), (16, 16), (256, 4), (256, 8), (512, 4), (1024, 16), (100, 3), (1, 1)])
@pytest.mark.parametrize("renorm", [True, False])
def test_topk_from_logits(M, E, K, renorm):
    T = 37
    cfg = replace(S.CONFIGS["tiny"], E=E, K=K)
    lg = S.Synth(cfg).logits(11, T)
    lg[0] = 0.0                                      # all tied
    lg[1, : min(E, 4)] = torch.tensor([1.0, 3.0, 3.0, 2.0])[: min(E, 4)]
    if E >= 3:
        lg[2] = -5.0
        lg[2, :3] = torch.tensor([-0.0, 0.0, -1.0])    # signed zeros tie
    lgd = lg.to(DEV)
    idx = torch.empty((T, K), dtype=torch.int32, device=DEV)
    w = torch.empty((T, K), dtype=torch.float32, device=DEV)
    M.moe_route_topk(T, 8, E, K, M.MOE_TOPK_RENORM if renorm else 0, None, None, lgd, idx, w)
    ridx, rw = O.route_topk(lg.numpy(), K, renorm)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert_rows_close(w.cpu().numpy(), rw, what="weights")


@pytest.mark.parametrize("name", ["tiny", "decode35b", "widek8", "large-int4", "batched"])
@pytest.mark.parametrize("rms", [False, True])
def test_router_topk(M, name, rms):
    cfg = S.CONFIGS[name]
    syn = S.Synth(cfg)
    T = {"batched": 256, "tiny": 64, "large-int4": 48}.get(name, 8)  # T >= 32: the MFMA router
    wr = syn.router(0)
    h, redraws = gap_tokens(syn, O.f64(wr.numpy()), T, cfg.K, rmsnorm=rms)
    log(f"{name}: {T} tokens, {redraws} redraws for the logit gap")
    logits = torch.empty((T, cfg.E), dtype=torch.float32, device=DEV)
    idx = torch.empty((T, cfg.K), dtype=torch.int32, device=DEV)
    w = torch.empty((T, cfg.K), dtype=torch.float32, device=DEV)
    flags = M.MOE_TOPK_RENORM | (M.MOE_INPUT_RMSNORM if rms else 0)
    M.moe_route_topk(T, cfg.d, cfg.E, cfg.K, flags, h.to(DEV), wr.to(DEV), logits, idx, w)
    x = O.rmsnorm(h.numpy()) if rms else O.f64(h.numpy())
    rl = O.router_logits(wr.numpy(), x)
    ridx, rw = O.route_topk(rl, cfg.K)
    assert_rows_close(logits.cpu().numpy(), rl, what="logits")
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert_rows_close(w.cpu().numpy(), rw, what="weights")


# ------------------------------------------------------------------------------------ expert FFN
def _oracle_ffn(cache, x, idx, w, r, bits, group):
    T, K = idx.shape
    o = np.zeros((T, K, x.shape[1]))
    for t in range(T):
        for k in range(K):
            o[t, k] = O.expert_ffn_packed(x[t], *cache(idx[t, k]), bits, group)
    return o, O.combine(o, w, r)


def _run_ffn(M, ex, T, K, flags, x, idx, w, r):
    out = torch.full((T, K, ex.d), float("nan"), dtype=torch.float32, device=DEV)
    y = torch.empty((T, ex.d), dtype=torch.float16, device=DEV)
    M.moe_expert_ffn_q4(T, K, flags, x, idx, ex, None, out, w, r, y, ws_for(M, T, K, ex))
    return out, y


def _ffn_case(M, cfg, T, rms=False, seed=0, layer=0):
    syn = S.Synth(cfg, seed)
    ex = device_layer(syn, layer, DEV)
    h = syn.hidden(500, T)
    x = O.rmsnorm(h.numpy()) if rms else O.f64(h.numpy())
    lg = syn.logits(77, T).numpy()
    idx, w = O.route_topk(lg, cfg.K)
    o_ref, y_ref = _oracle_ffn(ExpertCache(syn, layer), x, idx, w, O.f64(h.numpy()), cfg.bits, cfg.group)
    hd = h.to(DEV)
    out, y = _run_ffn(M, ex, T, cfg.K, M.MOE_INPUT_RMSNORM if rms else 0, hd,
                      torch.tensor(idx, dtype=torch.int32, device=DEV), torch.tensor(w, dtype=torch.float32, device=DEV), hd)
    assert_rows_close(out.cpu().numpy().reshape(T * cfg.K, -1), o_ref.reshape(T * cfg.K, -1), what=f"{cfg.name} o_k")
    assert_rows_close(y.cpu().numpy(), y_ref, what=f"{cfg.name} y")
    return ex, out, y


@pytest.mark.parametrize("name,T", [("tiny", 8), ("decode35b", 2), ("widek8", 2), ("large-int4", 2), ("large-int2", 2)])
def test_expert_ffn_decode(M, name, T):
    _ffn_case(M, S.CONFIGS[name], T)


def test_expert_ffn_rmsnorm_input(M):
    _ffn_case(M, S.CONFIGS["decode35b"], 1, rms=True)


@pytest.mark.parametrize("bits,group,d,I,E,K", [
    (2, 32, 256, 128, 4, 2),      # a 16-byte segment spans two 2-bit groups
    (2, 128, 512, 256, 4, 2),
    (4, 128, 512, 256, 4, 3),
    (4, 32, 96, 160, 5, 3),       # ragged: 3 and 5 segments per row (idle lanes)
    (4, 64, 8192, 256, 3, 2),     # widest rows: 4 segments per lane
    (2, 64, 8192, 128, 3, 1),
    (4, 32, 256, 128, 16, 16),    # K = E
    (4, 32, 256, 128, 16, 1),
])
def test_expert_ffn_shapes(M, bits, group, d, I, E, K):
    cfg = replace(S.CONFIGS["tiny"], name=f"shape{bits}-{group}-{d}-{I}", bits=bits, group=group, d=d, I=I, E=E, K=K)
    _ffn_case(M, cfg, 3)


def test_expert_ffn_bad_index_gives_nan(M):
    cfg = S.CONFIGS["tiny"]
    syn = S.Synth(cfg)
    ex = device_layer(syn, 0, DEV)
    h = syn.hidden(1, 1).to(DEV)
    idx = torch.tensor([[3, cfg.E]], dtype=torch.int32, device=DEV)
    w = torch.tensor([[0.5, 0.5]], dtype=torch.float32, device=DEV)
    out, y = _run_ffn(M, ex, 1, 2, 0, h, idx, w, h)
    torch.cuda.synchronize()
    assert torch.isfinite(out[0, 0]).all() and torch.isnan(out[0, 1]).all() and torch.isnan(y.float()).all()
    ref = O.expert_ffn_packed(O.f64(h.cpu().numpy()[0]), *ExpertCache(syn, 0)(3), cfg.bits, cfg.group)
    assert_rows_close(out[0, 0].cpu().numpy(), ref[None], what="valid slot")


def test_expert_ffn_deterministic(M):
    cfg = S.CONFIGS["decode35b"]
    syn = S.Synth(cfg)
    ex = device_layer(syn, 1, DEV)
    h = syn.hidden(3, 1).to(DEV)
    idx = torch.tensor([[7, 100, 3, 255]], dtype=torch.int32, device=DEV)
    w = torch.tensor([[0.4, 0.3, 0.2, 0.1]], dtype=torch.float32, device=DEV)
    a = _run_ffn(M, ex, 1, 4, 0, h, idx, w, h)
    b = _run_ffn(M, ex, 1, 4, 0, h, idx, w, h)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# ------------------------------------------------------------------------------------ combine
def test_combine(M):
    g = torch.Generator().manual_seed(5)
    T, K, d = 5, 4, 2048
    o = torch.randn((T, K, d), generator=g) * 4
    w = torch.softmax(torch.randn((T, K), generator=g), -1)
    r = torch.randn((T, d), generator=g).half()
    sh = torch.randn((T, d), generator=g)
    for shared in (None, sh):
        y = torch.empty((T, d), dtype=torch.float16, device=DEV)
        M.moe_combine(T, K, d, o.to(DEV), w.to(DEV), r.to(DEV), None if shared is None else shared.to(DEV), y)
        ref = O.combine(o.numpy(), w.numpy(), r.numpy(), None if shared is None else shared.numpy())
        assert_rows_close(y.cpu().numpy(), ref, what="combine")


def test_combine_vector_and_scalar_paths_agree(M):
    """moe_combine takes four columns per thread when d % 4 == 0 and the buffers are aligned, one
    otherwise; both do each element's arithmetic in the same order, so they agree to the bit."""
    g = torch.Generator().manual_seed(6)
    T, K, d = 37, 4, 2048
    o = torch.randn((T * K * d + 1,), generator=g).to(DEV)
    w = torch.softmax(torch.randn((T, K), generator=g), -1).to(DEV)
    r = torch.randn((T * d + 1,), generator=g).half().to(DEV)
    sh = torch.randn((T * d + 1,), generator=g).to(DEV)
    for shared in (False, True):
        ya = torch.empty((T, d), dtype=torch.float16, device=DEV)
        yb = torch.empty((T * d + 1,), dtype=torch.float16, device=DEV)
        oa, ra, sa = o[:-1].clone(), r[:-1].clone(), sh[:-1].clone()
        M.moe_combine(T, K, d, oa, w, ra, sa if shared else None, ya)   # aligned: four columns per thread
        ob, rb, sb = o[1:], r[1:], sh[1:]
        ob.copy_(oa)
        rb.copy_(ra)
        sb.copy_(sa)
        M.moe_combine(T, K, d, ob, w, rb, sb if shared else None, yb[1:])   # offset by one element: scalar
        torch.cuda.synchronize()
        assert torch.equal(ya.view(-1), yb[1:])


# ------------------------------------------------------------------------------------ prerouter
def test_prerouter_head(M):
    cfg = S.CONFIGS["decode35b"]
    syn = S.Synth(cfg)
    T, E, K = 4, cfg.E, cfg.K
    hw = syn.head(0, DEV)
    hc = {k: v.numpy() for k, v in syn.head(0, "cpu").items()}
    pw = M.PrerouterWeights(hw)
    h = syn.hidden(42, T)
    cur, _ = O.route_topk(syn.logits(1, T).numpy(), K)
    prev, _ = O.route_topk(syn.logits(2, T).numpy(), K)
    ws = torch.empty(M.moe_prerouter_workspace_size(T, E, pw.H), dtype=torch.uint8, device=DEV)
    for use_prev in (True, False):
        for rms in (False, True):
            lg = torch.empty((T, E), dtype=torch.float32, device=DEV)
            M.moe_prerouter(T, cfg.d, E, K, M.MOE_INPUT_RMSNORM if rms else 0, h.to(DEV),
                            torch.tensor(cur, dtype=torch.int32, device=DEV),
                            torch.tensor(prev, dtype=torch.int32, device=DEV) if use_prev else None, pw, lg, ws)
            x = O.rmsnorm(h.numpy()) if rms else O.f64(h.numpy())
            ref = np.stack([O.prerouter_logits(x[t], cur[t], prev[t] if use_prev else None, hc, E) for t in range(T)])
            assert_rows_close(lg.cpu().numpy(), ref, what="head logits")
            # the head's top-K (the next layer's routing) wherever the oracle is clear of ties
            idx = torch.empty((T, K), dtype=torch.int32, device=DEV)
            w = torch.empty((T, K), dtype=torch.float32, device=DEV)
            M.moe_route_topk(T, cfg.d, E, K, M.MOE_TOPK_RENORM, None, None, lg, idx, w)
            ridx, rw = O.route_topk(ref, K)
            for t in range(T):
                if O.topk_gaps(ref[t], K).min() >= 1e-4:
                    assert idx[t].cpu().tolist() == ridx[t].tolist()


# ------------------------------------------------------------------------------------ chain
def test_prerouted_chain(M):
    """Four decode35b-shaped layers, three tokens: per layer routing and outputs against the
    oracle's chain.  A layer whose oracle routing logits are within 1e-4 of a tie ends the
    comparison of that token (both sides may legitimately diverge from there)."""
    from int4_expert_ffn_amd.chain import DecodeStack, LayerWeights
    cfg = replace(S.CONFIGS["decode35b"], L=4)
    syn = S.Synth(cfg)
    layers, heads_cpu, routers_cpu = [], [], []
    for l in range(cfg.L):
        ex = device_layer(syn, l, DEV)
        router = syn.router(l, DEV)
        head = None
        if l < cfg.L - 1:
            hw = syn.head(l, DEV)
            head = M.PrerouterWeights(hw)
            heads_cpu.append({k: v.numpy() for k, v in syn.head(l, "cpu").items()})
        routers_cpu.append(syn.router(l, "cpu").numpy())
        layers.append(LayerWeights(ex, router, head))
    stack = DecodeStack(layers, cfg.K, DEV)
    caches = [ExpertCache(syn, l) for l in range(cfg.L)]
    st = O.ChainState(cfg.L)
    prev_tr = None
    for t in range(3):
        h0 = syn.hidden(9000 + t, 1)[0]
        stack.token(t, h0.to(DEV))
        torch.cuda.synchronize()
        hs = stack.h.cpu().numpy()
        ridx = stack.route_idx[t % 3].cpu().numpy()
        _, st, tr = O.chain_token(h0.numpy(), st, E=cfg.E, K=cfg.K, bits=cfg.bits, group=cfg.group,
                                  router_get=lambda l: routers_cpu[l],
                                  head_get=lambda l: heads_cpu[l] if l < len(heads_cpu) else None,
                                  expert_get=lambda l, e: caches[l](e))
        log(f"token {t}: routing {[r.tolist() for r in ridx]}")
        for l in range(cfg.L):
            if not np.array_equal(ridx[l], tr[l].idx):
                src = tr[l].route_logits if tr[l].route_logits is not None else prev_tr[l - 1].head_logits
                log(f"token {t} layer {l}: routing differs {ridx[l]} vs {tr[l].idx}")
                assert O.topk_gaps(src, cfg.K).min() < 1e-4, "routing differs away from a tie"
                return      # both chains legitimately diverge from here on
            assert_rows_close(hs[l + 1], tr[l].y[None], what=f"token {t} layer {l} y")
        prev_tr = tr
