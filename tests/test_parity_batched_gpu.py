"""GPU parity of the batched path (T >= 32: tokens sorted by expert, MFMA grouped GEMMs) and of
the shared expert with its unmerged LoRA, against the fp64 oracle."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import moe_synth as S
import oracle as O
from parity_util import ExpertCache, assert_rows_close, device_layer, gap_tokens, log

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


def oracle_routed(cache, x, idx, bits, group):
    """o[t][k] of every (token, slot), each expert dequantised once for all its tokens."""
    T, K = idx.shape
    o = np.zeros((T, K, x.shape[1]))
    for e in np.unique(idx):
        g, u, dn = cache(e)
        Wg, Wu, Wd = O.dequant(*g, bits, group), O.dequant(*u, bits, group), O.dequant(*dn, bits, group)
        tt, kk = np.nonzero(idx == e)
        o[tt, kk] = O.expert_ffn(x[tt], Wg, Wu, Wd)
    return o


def run(M, ex, T, K, flags, x, idx, w=None, r=None, lora=None, fused=True):
    out = torch.full((T, K, ex.d), float("nan"), dtype=torch.float32, device=DEV)
    y = torch.empty((T, ex.d), dtype=torch.float16, device=DEV) if fused else None
    M.moe_expert_ffn_q4(T, K, flags, x, idx, ex, lora, out, w if fused else None, r if fused else None, y,
                        ws_for(M, T, K, ex))
    return out, y


def case(M, cfg, T, rms=False, layer=0):
    syn = S.Synth(cfg)
    ex = device_layer(syn, layer, DEV)
    h = syn.hidden(321, T)
    x = O.rmsnorm(h.numpy()) if rms else O.f64(h.numpy())
    idx, w = O.route_topk(syn.logits(99, T).numpy(), cfg.K)
    o_ref = oracle_routed(ExpertCache(syn, layer), x, idx, cfg.bits, cfg.group)
    y_ref = O.combine(o_ref, w, O.f64(h.numpy()))
    hd = h.to(DEV)
    out, y = run(M, ex, T, cfg.K, M.MOE_INPUT_RMSNORM if rms else 0, hd,
                 torch.tensor(idx, dtype=torch.int32, device=DEV), torch.tensor(w, dtype=torch.float32, device=DEV), hd)
    assert_rows_close(out.cpu().numpy().reshape(T * cfg.K, -1), o_ref.reshape(T * cfg.K, -1), what=f"{cfg.name} o")
    assert_rows_close(y.cpu().numpy(), y_ref, what=f"{cfg.name} y")
    return syn, ex, h, idx, w, out, y


def test_sort_by_expert_matches_oracle(M):
    for T, K, E in [(256, 4, 256), (33, 2, 16), (1, 1, 1), (4096, 8, 1024), (64, 16, 16)]:
        cfg = replace(S.CONFIGS["tiny"], E=E, K=K)
        idx, _ = O.route_topk(S.Synth(cfg).logits(5, T).numpy(), K)
        idx_d = torch.tensor(idx, dtype=torch.int32, device=DEV)
        counts = torch.empty(E + 1, dtype=torch.int32, device=DEV)
        offsets = torch.empty(E + 2, dtype=torch.int32, device=DEV)
        perm = torch.empty(T * K, dtype=torch.int32, device=DEV)
        M.moe_sort_by_expert(T, K, E, idx_d, counts, offsets, perm)
        rc, ro, rp = O.group_by_expert(idx, E)
        assert counts[:E].cpu().tolist() == rc.tolist() and counts[E].item() == 0
        assert offsets[: E + 1].cpu().tolist() == ro.tolist() and offsets[E + 1].item() == T * K
        assert perm.cpu().tolist() == rp.tolist()


def test_sort_by_expert_out_of_range_bucket(M):
    idx = torch.tensor([[3, 9], [16, 3], [-1, 0]], dtype=torch.int32, device=DEV)
    E = 16
    counts = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    offsets = torch.empty(E + 2, dtype=torch.int32, device=DEV)
    perm = torch.empty(6, dtype=torch.int32, device=DEV)
    M.moe_sort_by_expert(3, 2, E, idx, counts, offsets, perm)
    assert counts[E].item() == 2 and perm[offsets[E].item():].cpu().tolist() == [2, 4]
    assert perm[: offsets[E].item()].cpu().tolist() == [5, 0, 3, 1]


@pytest.mark.parametrize("name,T", [("batched", 256), ("tiny", 64), ("decode35b", 32)])
def test_grouped_routed_experts(M, name, T):
    case(M, S.CONFIGS[name], T)


@pytest.mark.parametrize("bits", [2, 4])
def test_grouped_large_rows_many_tokens_per_expert(M, bits):
    """d_model 4096 / I 1024 rows with 8 experts, so each expert gathers ~20 tokens (two MFMA
    token tiles)."""
    cfg = replace(S.CONFIGS["large-int4" if bits == 4 else "large-int2"], E=8)
    case(M, cfg, 40)


def test_grouped_rmsnorm(M):
    case(M, S.CONFIGS["batched"], 48, rms=True)


@pytest.mark.parametrize("bits,group,d,I,E,K", [
    (2, 32, 256, 128, 4, 2),
    (4, 128, 512, 256, 4, 3),
    (4, 32, 96, 160, 5, 3),      # ragged rows and columns: partial MFMA tiles, zero-padded chunks
    (4, 64, 1088, 576, 6, 2),    # d and I not multiples of the 512-column LDS chunk
    (4, 32, 256, 128, 16, 16),   # K = E
    # 64-column groups with 16-byte aligned scale rows: the lane-contiguous kernel, with one and
    # several chunks and each chunk length
    (4, 64, 1024, 512, 8, 2),
    (4, 64, 4096, 1536, 8, 2),
    (2, 64, 2048, 512, 8, 3),
    (2, 64, 512, 1024, 6, 2),
])
def test_grouped_shapes(M, bits, group, d, I, E, K):
    cfg = replace(S.CONFIGS["tiny"], name=f"g{bits}-{group}-{d}-{I}", bits=bits, group=group, d=d, I=I, E=E, K=K)
    case(M, cfg, 37)


def test_grouped_matches_decode_path(M):
    """T = 32 through the grouped path equals 32 single-token decode calls (both within the
    oracle tolerance; compared to each other at the same bar)."""
    cfg = S.CONFIGS["decode35b"]
    syn, ex, h, idx, w, out_g, y_g = case(M, cfg, 32)
    hd = h.to(DEV)
    idx_d = torch.tensor(idx, dtype=torch.int32, device=DEV)
    w_d = torch.tensor(w, dtype=torch.float32, device=DEV)
    outs = []
    for t in range(32):
        o, _ = run(M, ex, 1, cfg.K, 0, hd[t:t + 1].contiguous(), idx_d[t:t + 1].contiguous(), fused=False)
        outs.append(o)
    out_d = torch.cat(outs).cpu().numpy()
    assert_rows_close(out_g.cpu().numpy().reshape(-1, cfg.d), out_d.reshape(-1, cfg.d), what="grouped vs decode")


def test_grouped_bad_index_gives_nan(M):
    cfg = S.CONFIGS["tiny"]
    syn = S.Synth(cfg)
    ex = device_layer(syn, 0, DEV)
    T = 40
    h = syn.hidden(8, T).to(DEV)
    idx, w = O.route_topk(syn.logits(3, T).numpy(), cfg.K)
    idx[5, 1] = cfg.E
    idx[7, 0] = -3
    out, y = run(M, ex, T, cfg.K, 0, h, torch.tensor(idx, dtype=torch.int32, device=DEV),
                 torch.tensor(w, dtype=torch.float32, device=DEV), h)
    torch.cuda.synchronize()
    o = out.cpu()
    assert torch.isnan(o[5, 1]).all() and torch.isnan(o[7, 0]).all()
    assert torch.isfinite(o[5, 0]).all() and torch.isfinite(o[6]).all()
    assert torch.isnan(y[5].float()).all() and torch.isfinite(y[6].float()).all()


# ---------------------------------------------------------------------------------- shared + LoRA
def _shared(M, cfg, syn, layer=0):
    se = syn.shared_expert_id()
    mats = [syn.expert_mat(layer, [se], m, DEV) for m in S.MATS]
    ex = M.Experts(*mats, cfg.bits, cfg.group)
    cpu = tuple(tuple(a[0].numpy() for a in syn.expert_mat(layer, [se], m, "cpu")) for m in S.MATS)
    lw = syn.lora(layer, DEV)
    lora = M.Lora3([lw[m] for m in S.MATS], cfg.lora_alpha)
    lw_cpu = syn.lora(layer, "cpu")      # the oracle's copy, drawn on the host
    lora_cpu = {m: (lw_cpu[m][0].numpy(), lw_cpu[m][1].numpy()) for m in S.MATS}
    lora_cpu["alpha"] = cfg.lora_alpha
    return ex, cpu, lora, lora_cpu, lw


@pytest.mark.parametrize("T,rms", [(256, False), (5, False), (64, True), (48, True), (33, True)])
def test_shared_expert_with_lora(M, T, rms):
    """Grouped (T >= 32) and decode (T = 5) paths of the always-on shared expert with an unmerged
    LoRA on gate, up and down (rank 16, alpha 32), on raw and on RMS-normed input.  The adapter's
    A . x runs on the matrix cores when T is a multiple of 16 and one wave per (token, rank row)
    otherwise (T = 33)."""
    cfg = S.CONFIGS["batched"]
    syn = S.Synth(cfg)
    ex, cpu, lora, lora_cpu, _ = _shared(M, cfg, syn)
    h = syn.hidden(77, T)
    x = O.rmsnorm(h.numpy()) if rms else O.f64(h.numpy())
    ref = O.expert_ffn_packed(x, *cpu, cfg.bits, cfg.group, lora_cpu)
    base = O.expert_ffn_packed(x, *cpu, cfg.bits, cfg.group)
    log(f"LoRA delta relative size {np.abs(ref - base).max() / np.abs(base).max():.3f}")
    idx = torch.zeros((T, 1), dtype=torch.int32, device=DEV)
    out, _ = run(M, ex, T, 1, M.MOE_INPUT_RMSNORM if rms else 0, h.to(DEV), idx, lora=lora, fused=False)
    assert_rows_close(out.cpu().numpy()[:, 0], ref, what="shared + LoRA")
    assert np.abs(ref - base).max() > 50 * 2e-3 * np.abs(ref).max() / 10   # the delta is visible


@pytest.mark.parametrize("T", [64, 5])
def test_lora_with_out_of_range_token(M, T):
    """A token whose index is outside [0, n_experts) gives a NaN row and leaves every other token's
    adapter terms alone: the down adapter's A . act must use each token's own activation row, not
    the row at the token's number in expert-sorted order (which shifts past the skipped token)."""
    cfg = S.CONFIGS["batched"]
    syn = S.Synth(cfg)
    ex, cpu, lora, lora_cpu, _ = _shared(M, cfg, syn)
    h = syn.hidden(78, T)
    ref = O.expert_ffn_packed(O.f64(h.numpy()), *cpu, cfg.bits, cfg.group, lora_cpu)
    idx = torch.zeros((T, 1), dtype=torch.int32)
    bad = T // 3
    idx[bad, 0] = 1
    out, _ = run(M, ex, T, 1, 0, h.to(DEV), idx.to(DEV), lora=lora, fused=False)
    o = out.cpu().numpy()[:, 0]
    assert np.isnan(o[bad]).all()
    keep = np.arange(T) != bad
    assert_rows_close(o[keep], ref[keep], what="shared + LoRA, one token out of range")


def test_lora_zero_b_is_base(M):
    cfg = S.CONFIGS["batched"]
    syn = S.Synth(cfg)
    ex, cpu, _, _, lw = _shared(M, cfg, syn)
    zero = M.Lora3([(lw[m][0], torch.zeros_like(lw[m][1])) for m in S.MATS], cfg.lora_alpha)
    T = 64
    h = syn.hidden(1, T).to(DEV)
    idx = torch.zeros((T, 1), dtype=torch.int32, device=DEV)
    a, _ = run(M, ex, T, 1, 0, h, idx, lora=zero, fused=False)
    b, _ = run(M, ex, T, 1, 0, h, idx, fused=False)
    assert torch.equal(a, b)


def test_batched_layer_end_to_end(M):
    """The whole batched layer: router + top-K for 256 tokens, routed experts (grouped), shared
    expert with LoRA, combine with the residual."""
    cfg = S.CONFIGS["batched"]
    syn = S.Synth(cfg)
    T, E, K, d = cfg.T, cfg.E, cfg.K, cfg.d
    ex = device_layer(syn, 0, DEV)
    sh_ex, sh_cpu, lora, lora_cpu, _ = _shared(M, cfg, syn)
    wr = syn.router(0)
    h, redraws = gap_tokens(syn, O.f64(wr.numpy()), T, K, first_stream=5000)
    log(f"batched: {redraws} redraws")
    hd = h.to(DEV)
    logits = torch.empty((T, E), dtype=torch.float32, device=DEV)
    idx = torch.empty((T, K), dtype=torch.int32, device=DEV)
    w = torch.empty((T, K), dtype=torch.float32, device=DEV)
    M.moe_route_topk(T, d, E, K, M.MOE_TOPK_RENORM, hd, wr.to(DEV), logits, idx, w)
    o = torch.empty((T, K, d), dtype=torch.float32, device=DEV)
    M.moe_expert_ffn_q4(T, K, 0, hd, idx, ex, None, o, None, None, None, ws_for(M, T, K, ex))
    sh = torch.empty((T, 1, d), dtype=torch.float32, device=DEV)
    zeros = torch.zeros((T, 1), dtype=torch.int32, device=DEV)
    M.moe_expert_ffn_q4(T, 1, 0, hd, zeros, sh_ex, lora, sh, None, None, None, ws_for(M, T, 1, sh_ex))
    y = torch.empty((T, d), dtype=torch.float16, device=DEV)
    M.moe_combine(T, K, d, o, w, hd, sh.view(T, d), y)
    x = O.f64(h.numpy())
    rl = O.router_logits(wr.numpy(), x)
    ridx, rw = O.route_topk(rl, K)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    o_ref = oracle_routed(ExpertCache(syn, 0), x, ridx, cfg.bits, cfg.group)
    sh_ref = O.expert_ffn_packed(x, *sh_cpu, cfg.bits, cfg.group, lora_cpu)
    y_ref = O.combine(o_ref, rw, x, sh_ref)
    assert_rows_close(o.cpu().numpy().reshape(T * K, d), o_ref.reshape(T * K, d), what="routed o")
    assert_rows_close(y.cpu().numpy(), y_ref, what="layer y")


def _separate(M, T, K, flags, x, idx, w, ex, sh_ex, lora):
    """The three-call reference of moe_expert_ffn_q4_shared: routed experts, shared expert (K = 1,
    with its LoRA), combine."""
    d = ex.d
    o = torch.empty((T, K, d), dtype=torch.float32, device=DEV)
    M.moe_expert_ffn_q4(T, K, flags, x, idx, ex, None, o, None, None, None, ws_for(M, T, K, ex))
    sh = torch.empty((T, 1, d), dtype=torch.float32, device=DEV)
    zeros = torch.zeros((T, 1), dtype=torch.int32, device=DEV)
    M.moe_expert_ffn_q4(T, 1, flags, x, zeros, sh_ex, lora, sh, None, None, None, ws_for(M, T, 1, sh_ex))
    y = torch.empty((T, d), dtype=torch.float16, device=DEV)
    M.moe_combine(T, K, d, o, w, x, sh.view(T, d), y)
    return y


def _merged(M, T, K, flags, x, idx, w, ex, sh_ex, lora):
    y = torch.full((T, ex.d), float("nan"), dtype=torch.float16, device=DEV)
    ws = torch.empty(M.moe_expert_ffn_shared_workspace_size(T, K, ex), dtype=torch.uint8, device=DEV)
    M.moe_expert_ffn_q4_shared(T, K, flags, x, idx, ex, sh_ex, lora, w, x, y, ws)
    return y


@pytest.mark.parametrize("bits,group,d,I,E,K,T,rms,lora", [
    (4, 64, 2048, 512, 256, 4, 256, False, True),    # the batched configuration's shapes
    (4, 64, 2048, 512, 256, 4, 256, True, False),
    (4, 32, 96, 160, 5, 3, 37, False, True),         # ragged rows and columns (the 16-column kernel)
    (2, 64, 2048, 512, 8, 3, 40, False, True),       # 2-bit, lane-contiguous kernel
    (4, 64, 4096, 1536, 8, 2, 33, True, True),
    (4, 32, 256, 128, 16, 16, 32, False, False),     # K = E
])
def test_shared_expert_in_the_routed_call(M, bits, group, d, I, E, K, T, rms, lora):
    """moe_expert_ffn_q4_shared (the shared expert's rows sorted in with the routed pairs, one GEMM
    launch per projection) equals the routed call, the shared call and moe_combine, bit for bit;
    a token whose index is out of range gives a NaN row in both."""
    cfg = replace(S.CONFIGS["batched"], name=f"s{bits}-{group}-{d}-{I}", bits=bits, group=group, d=d, I=I, E=E, K=K,
                  T=T)
    syn = S.Synth(cfg)
    ex = device_layer(syn, 0, DEV)
    sh_ex, _, lo, _, _ = _shared(M, cfg, syn)
    lo = lo if lora else None
    h = syn.hidden(4321, T).to(DEV)
    idx_np, w_np = O.route_topk(syn.logits(98, T).numpy(), K)
    idx_np[T // 2, 0] = E + 3                          # outside [0, E): that token's row is NaN
    idx = torch.tensor(idx_np, dtype=torch.int32, device=DEV)
    w = torch.tensor(w_np, dtype=torch.float32, device=DEV)
    flags = M.MOE_INPUT_RMSNORM if rms else 0
    a = _separate(M, T, K, flags, h, idx, w, ex, sh_ex, lo)
    b = _merged(M, T, K, flags, h, idx, w, ex, sh_ex, lo)
    torch.cuda.synchronize()
    assert torch.isnan(a[T // 2]).all() and torch.isnan(b[T // 2]).all()
    keep = torch.ones(T, dtype=torch.bool)
    keep[T // 2] = False
    assert torch.isfinite(a[keep]).all()
    assert torch.equal(a[keep], b[keep])


def test_shared_call_small_T_unsupported(M):
    cfg = S.CONFIGS["batched"]
    syn = S.Synth(cfg)
    ex = device_layer(syn, 0, DEV)
    sh_ex, _, lo, _, _ = _shared(M, cfg, syn)
    assert M.moe_expert_ffn_shared_workspace_size(31, 4, ex) == 0
    T = 31
    x = syn.hidden(1, T).to(DEV)
    idx = torch.zeros((T, 4), dtype=torch.int32, device=DEV) + torch.arange(4, dtype=torch.int32, device=DEV)
    w = torch.full((T, 4), 0.25, dtype=torch.float32, device=DEV)
    y = torch.empty((T, cfg.d), dtype=torch.float16, device=DEV)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=DEV)
    with pytest.raises(M.MoEError, match="UNSUPPORTED"):
        M.moe_expert_ffn_q4_shared(T, 4, 0, x, idx, ex, sh_ex, lo, w, x, y, ws)


def test_batched_layer_schedules(M):
    """The packaged batched layer: the shared expert inside the routed call (default), on a second
    stream, or on the same stream after the routed experts, all equal bit for bit, eagerly and as
    graph replays with eager work in between."""
    from int4_expert_ffn_amd.batched import BatchedLayer
    cfg = S.CONFIGS["batched"]
    syn = S.Synth(cfg)
    T, K, d = cfg.T, cfg.K, cfg.d
    ex = device_layer(syn, 0, DEV)
    sh_ex, _, lora, _, _ = _shared(M, cfg, syn)
    router = syn.router(0, DEV)
    merged = BatchedLayer(ex, router, T, K, DEV, shared=sh_ex, lora3=lora)
    assert merged.merged
    two = BatchedLayer(ex, router, T, K, DEV, shared=sh_ex, lora3=lora, two_streams=True, separate=True)
    one = BatchedLayer(ex, router, T, K, DEV, shared=sh_ex, lora3=lora, two_streams=False, separate=True)
    hs0 = syn.hidden(78, T).to(DEV)
    ym = torch.empty((T, d), dtype=torch.float16, device=DEV)
    yo = torch.empty_like(ym)
    merged(hs0, ym)
    one(hs0, yo)
    torch.cuda.synchronize()
    assert torch.equal(ym, yo)
    gm = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    h_m = hs0.clone()
    with torch.cuda.graph(gm, stream=cs):
        merged(h_m, ym)
    torch.cuda.synchronize()
    for i in range(3):
        hi = syn.hidden(90 + i, T).to(DEV)
        h_m.copy_(hi)
        torch.cuda.synchronize()
        with torch.cuda.stream(cs):
            gm.replay()
        cs.synchronize()
        one(hi, yo)
        torch.cuda.synchronize()
        assert torch.equal(ym, yo), f"merged replay {i}"
    hs = syn.hidden(77, 4 * T).to(DEV).view(4, T, d)
    y1 = torch.empty((T, d), dtype=torch.float16, device=DEV)
    y2 = torch.empty_like(y1)
    cs = torch.cuda.Stream()
    h_in = hs[0].clone()
    with torch.cuda.stream(cs):
        two(h_in, y2)
    cs.synchronize()
    one(hs[0], y1)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cs):
        two(h_in, y2)
    torch.cuda.synchronize()
    for i in range(4):
        h_in.copy_(hs[i])
        torch.cuda.synchronize()
        with torch.cuda.stream(cs):
            g.replay()
        cs.synchronize()
        one(hs[i], y1)
        torch.cuda.synchronize()
        assert torch.equal(y1, y2), f"replay {i}"
