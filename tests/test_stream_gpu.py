"""GPU checks of expert streaming into an HBM pool (moe_stream_in) and of the streamed decode stack.

Placement is integer work: slots, pool state and hit / miss counts must equal the oracle's
`pool_plan` exactly, and every slot must hold its expert's bytes exactly.  The streamed stack runs
the resident stack's kernels on the same bytes, so its outputs must equal the resident per-layer
path's bit for bit (which the other tests hold to the oracle chain); one run is also checked
against the oracle directly."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import moe_synth as S
import oracle as O
from parity_util import ExpertCache, assert_rows_close, log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def M():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int4_expert_ffn_amd as m
    return m


def host_copy(mats):
    """The same arrays in pinned host memory."""
    out = {}
    for m, arrs in mats.items():
        out[m] = tuple(torch.empty(a.shape, dtype=a.dtype, pin_memory=True).copy_(a) for a in arrs)
    return out


def experts_of(M, cfg, mats, host=False, nm=False):
    return M.Experts(mats["gate"], mats["up"], mats["down"], cfg.bits, cfg.group, neuron_major_down=nm, host=host)


def check_pool_bytes(pool, mats, state):
    """Every occupied slot holds exactly its expert's nine arrays."""
    exp = pool.slot_expert.cpu().tolist()
    for s, e in enumerate(exp):
        if e < 0:
            continue
        for m, arrs in zip(("gate", "up", "down"), pool.experts.tensors):
            for a_pool, a_src in zip(arrs, mats[m]):
                assert torch.equal(a_pool[s].cpu(), a_src[e].cpu()), f"slot {s} (expert {e}) {m} differs"
    assert exp == state.expert


@pytest.mark.parametrize("host", [True, False])
def test_stream_in_matches_oracle_plan(M, host):
    cfg = S.CONFIGS["tiny"]
    syn = S.Synth(cfg)
    mats = S.fill_experts(syn, 0, DEV)
    src_mats = host_copy(mats) if host else mats
    src = experts_of(M, cfg, src_mats, host=host)
    K, S_ = 3, 7
    pool = M.Pool(src, S_, DEV)
    st = O.PoolState(S_)
    idx_slot = torch.empty(K, dtype=torch.int32, device=DEV)
    counters = torch.zeros(2, dtype=torch.int32, device=DEV)
    ws = torch.empty(M.moe_stream_workspace_size(K), dtype=torch.uint8, device=DEV)
    rng = np.random.default_rng(11)
    hits = misses = 0
    for t in range(80):
        hot = 6 if t % 4 else cfg.E          # stretches of reuse among a few experts, then anything
        sel = [int(v) for v in rng.choice(hot, size=K, replace=False)]
        M.moe_stream_in(K, torch.tensor(sel, dtype=torch.int32, device=DEV), src, pool, idx_slot, counters, ws)
        slot, copies = O.pool_plan(st, sel, t)
        hits += K - len(copies)
        misses += len(copies)
        torch.cuda.synchronize()
        assert idx_slot.cpu().tolist() == slot, f"token {t}"
        assert pool.slot_stamp.cpu().tolist() == st.stamp, f"token {t}"
        if t % 10 == 9:
            check_pool_bytes(pool, mats, st)
    check_pool_bytes(pool, mats, st)
    assert counters.cpu().tolist() == [hits, misses]
    assert 0 < hits and 0 < misses


def test_stream_in_bad_index(M):
    """An index outside [0, E) gets slot -1 and no copy; the others are placed as usual."""
    cfg = S.CONFIGS["tiny"]
    syn = S.Synth(cfg)
    mats = S.fill_experts(syn, 0, DEV)
    src = experts_of(M, cfg, mats)
    pool = M.Pool(src, 4, DEV)
    idx_slot = torch.empty(2, dtype=torch.int32, device=DEV)
    counters = torch.zeros(2, dtype=torch.int32, device=DEV)
    ws = torch.empty(M.moe_stream_workspace_size(2), dtype=torch.uint8, device=DEV)
    M.moe_stream_in(2, torch.tensor([5, cfg.E], dtype=torch.int32, device=DEV), src, pool, idx_slot, counters, ws)
    torch.cuda.synchronize()
    assert idx_slot.cpu().tolist() == [0, -1]
    assert pool.slot_expert.cpu().tolist() == [5, -1, -1, -1]
    assert counters.cpu().tolist() == [0, 1]      # the bad index is neither a hit nor a copy
    st = O.PoolState(4)
    O.pool_plan(st, [5], 0)
    check_pool_bytes(pool, mats, st)


def build_host_stack(M, cfg):
    """A prerouted stack whose experts sit in pinned host memory, and the same stack resident."""
    from int4_expert_ffn_amd.chain import LayerWeights
    syn = S.Synth(cfg)
    host_layers, dev_layers, heads_cpu = [], [], []
    for l in range(cfg.L):
        mats = S.fill_experts(syn, l, DEV)
        head = None
        if l < cfg.L - 1:
            head = M.PrerouterWeights(syn.head(l, DEV))
            heads_cpu.append({k: v.numpy() for k, v in syn.head(l, "cpu").items()})
        router = syn.router(l, DEV)
        dev_layers.append(LayerWeights(experts_of(M, cfg, mats), router, head))
        host_layers.append(LayerWeights(experts_of(M, cfg, host_copy(mats), host=True), router, head))
    return syn, host_layers, dev_layers, heads_cpu


@pytest.mark.parametrize("prefetch", [True, False])
def test_streamed_stack_equals_resident(M, prefetch):
    from int4_expert_ffn_amd.chain import DecodeStack
    from int4_expert_ffn_amd.stream import StreamedStack
    cfg = replace(S.CONFIGS["decode35b"], L=4)
    syn, host_layers, dev_layers, heads_cpu = build_host_stack(M, cfg)
    res = DecodeStack(dev_layers, cfg.K, DEV)
    stm = StreamedStack(host_layers, cfg.K, DEV, n_slots=2 * cfg.K, prefetch=prefetch)
    toks = syn.hidden(31, 8)
    outs = []
    for t in range(8):
        log(f"streamed token {t} prefetch={prefetch}")
        a = res.token(t, toks[t].to(DEV)).clone()
        b = stm.token(t, toks[t].to(DEV)).clone()
        torch.cuda.synchronize()
        assert torch.equal(a, b), f"token {t}: streamed output differs from the resident one"
        assert torch.equal(res.route_idx, stm.route_idx)
        outs.append(b)
    hits, misses = stm.hits_misses()
    log(f"hits {hits} misses {misses}")
    # 8 tokens of L layers, plus, in prefetch mode, the copies for a ninth token the heads already predicted
    assert hits + misses == 8 * cfg.L * cfg.K + (cfg.L - 1) * cfg.K * prefetch and misses >= cfg.L * cfg.K
    if prefetch:   # one check against the oracle chain directly
        routers_cpu = [syn.router(l, "cpu").numpy() for l in range(cfg.L)]
        caches = [ExpertCache(syn, l) for l in range(cfg.L)]
        st = O.ChainState(cfg.L)
        for t in range(2):
            hL, st, _ = O.chain_token(toks[t].numpy(), st, E=cfg.E, K=cfg.K, bits=cfg.bits, group=cfg.group,
                                      router_get=lambda l: routers_cpu[l],
                                      head_get=lambda l: heads_cpu[l] if l < len(heads_cpu) else None,
                                      expert_get=lambda l, e: caches[l](e))
            assert_rows_close(outs[t].float().cpu().numpy()[None], hL[None], what=f"token {t}")


def test_stream_in_serves_the_sparse_layout(M):
    """Streaming is layout-blind: a pool of neuron-major ReLU experts gives moe_expert_ffn_sparse
    the same result as the full device stack."""
    cfg = S.CONFIGS["decode35b"]
    syn = S.Synth(cfg)
    mats = S.fill_experts(syn, 0, DEV, relu=True)
    full = experts_of(M, cfg, mats, nm=True)
    src = experts_of(M, cfg, host_copy(mats), host=True, nm=True)
    pool = M.Pool(src, 8, DEV)
    K = cfg.K
    idx = torch.tensor([[200, 3, 77, 150]], dtype=torch.int32, device=DEV)
    w = torch.tensor([[0.4, 0.3, 0.2, 0.1]], dtype=torch.float32, device=DEV)
    idx_slot = torch.empty(K, dtype=torch.int32, device=DEV)
    ws = torch.empty(M.moe_stream_workspace_size(K), dtype=torch.uint8, device=DEV)
    M.moe_stream_in(K, idx[0], src, pool, idx_slot, None, ws)
    h = syn.hidden(5, 1).to(DEV)
    fws = torch.empty(M.moe_expert_ffn_sparse_workspace_size(1, K, full), dtype=torch.uint8, device=DEV)
    ya = torch.empty_like(h)
    yb = torch.empty_like(h)
    M.moe_expert_ffn_sparse(1, K, 0, h, idx, full, None, w, h, ya, None, fws)
    M.moe_expert_ffn_sparse(1, K, 0, h, idx_slot.view(1, K), pool.experts, None, w, h, yb, None, fws)
    torch.cuda.synchronize()
    assert torch.equal(ya, yb)


def test_streamed_stack_graph_replays(M):
    """Each token as a HIP-graph replay (three graphs, one per routing slot) on several streams: every
    replay equals the resident stack's eager token, and after the run each pool holds what the
    oracle's placement gives for the routing its layer saw (slots age by the device clock, not by a
    token number baked into the graph)."""
    from int4_expert_ffn_amd.chain import DecodeStack
    from int4_expert_ffn_amd.stream import StreamedStack
    cfg = replace(S.CONFIGS["decode35b"], L=4)
    syn, host_layers, dev_layers, _ = build_host_stack(M, cfg)
    res = DecodeStack(dev_layers, cfg.K, DEV)
    n_slots = 3 * cfg.K
    stm = StreamedStack(host_layers, cfg.K, DEV, n_slots=n_slots, prefetch=True)
    T = 13
    toks = syn.hidden(41, T).to(DEV)
    ring = torch.empty((3, cfg.d), dtype=torch.float16, device=DEV)
    cs = torch.cuda.Stream()
    with torch.cuda.stream(cs):
        stm.token(0, toks[0])
    torch.cuda.synchronize()
    graphs = []
    for j in range(3):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cs):
            stm.token(j + 1, ring[j])
        graphs.append(g)
    torch.cuda.synchronize()
    used = [[] for _ in range(cfg.L)]            # routing of every layer at every token
    res.token(0, toks[0])
    torch.cuda.synchronize()
    for l in range(cfg.L):
        used[l].append(res.route_idx[0, l].cpu().tolist())
    for t in range(1, T):
        a = res.token(t, toks[t]).clone()
        torch.cuda.synchronize()
        for l in range(cfg.L):
            used[l].append(res.route_idx[t % 3, l].cpu().tolist())
        with torch.cuda.stream(cs):
            ring[(t - 1) % 3].copy_(toks[t])
            graphs[(t - 1) % 3].replay()
        cs.synchronize()
        assert torch.equal(stm.h[cfg.L], a), f"replay of token {t} differs from the resident token"
    # layer 0 places its own routing at every token; a layer after a head also places the prediction
    # for the token after the last (made during the last token)
    for l in range(cfg.L):
        calls = list(used[l])
        if l > 0:
            calls.append(res.route_idx[T % 3, l].cpu().tolist())
        st = O.PoolState(n_slots)
        for c, sel in enumerate(calls):
            O.pool_plan(st, sel, c)
        assert stm.pools[l].slot_expert.cpu().tolist() == st.expert, f"layer {l}"
        assert stm.pools[l].slot_stamp.cpu().tolist() == st.stamp, f"layer {l}"
        assert int(stm.pools[l].clock.item()) == len(calls)
    del graphs


def test_stream_in_many_equals_separate_calls(M):
    """moe_stream_in_many over several pools gives the pools, slots and counts of separate calls."""
    cfg = S.CONFIGS["tiny"]
    syn = S.Synth(cfg)
    srcs = [experts_of(M, cfg, S.fill_experts(syn, l, DEV)) for l in range(3)]
    K = 2
    a = [M.Pool(s_, 5, DEV) for s_ in srcs]
    b = [M.Pool(s_, 5, DEV) for s_ in srcs]
    ca, cb = torch.zeros((3, 2), dtype=torch.int32, device=DEV), torch.zeros((3, 2), dtype=torch.int32, device=DEV)
    sa, sb = torch.empty((3, K), dtype=torch.int32, device=DEV), torch.empty((3, K), dtype=torch.int32, device=DEV)
    ws1 = torch.empty(M.moe_stream_workspace_size(K), dtype=torch.uint8, device=DEV)
    wsn = torch.empty(3 * M.moe_stream_workspace_size(K), dtype=torch.uint8, device=DEV)
    rng = np.random.default_rng(5)
    for t in range(40):
        sel = torch.tensor(np.stack([rng.choice(8, size=K, replace=False) for _ in range(3)]), dtype=torch.int32,
                           device=DEV)
        for l in range(3):
            M.moe_stream_in(K, sel[l], srcs[l], a[l], sa[l], ca[l], ws1)
        M.moe_stream_in_many(K, [(sel[l], srcs[l], b[l], sb[l], cb[l]) for l in range(3)], wsn)
        torch.cuda.synchronize()
        assert torch.equal(sa, sb), f"token {t}"
    assert torch.equal(ca, cb)
    for l in range(3):
        assert torch.equal(a[l].slot_expert, b[l].slot_expert) and torch.equal(a[l].slot_stamp, b[l].slot_stamp)
        for ma, mb in zip(a[l].experts.tensors, b[l].experts.tensors):
            for xa, xb in zip(ma, mb):
                occupied = a[l].slot_expert >= 0
                assert torch.equal(xa[occupied], xb[occupied])
