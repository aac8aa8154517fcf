#!/usr/bin/env python3
"""Decode benchmark of the prerouted MoE stack on one MI355X.

Workload (one step = one token through the whole stack): the 35B-shaped decode layer --
d_model 2048, 256 experts, top-4, expert intermediate 512, int4 affine group 64, 40 layers
resident in HBM, prerouter heads (fc1 2560->1024, erf-GELU, fc2 1024->256, linear 2560->256) on
layers 0..38, layer 0 routed by its own router -- batch 1, synthetic seeded weights and hidden
states (a fresh draw per token).  Each token is one HIP-graph replay of every C-ABI call of the 40
layers; inputs are resident in HBM before the timed region.

Prints one JSON line: tokens/s, the roofline of the dominant step (the expert FFN of one layer,
timed with HIP events on its own stream) and the CPU oracle timed on a bounded sample.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def build_stack(cfg, syn, dev, M):
    from int4_expert_ffn_amd.chain import DecodeStack, LayerWeights
    import moe_synth as S
    layers = []
    routers = [syn.router(l, dev) for l in range(cfg.L + 1)]
    for l in range(cfg.L):
        mats = S.fill_experts(syn, l, dev)
        ex = M.Experts(mats["gate"], mats["up"], mats["down"], cfg.bits, cfg.group)
        head = None
        if l < cfg.L - 1:
            hw = syn.head(l, dev)
            hw["lin_x"] = routers[l + 1]          # the head's linear path is the next router
            head = M.PrerouterWeights(hw)
        layers.append(LayerWeights(ex, routers[l], head))
    return layers


def algorithmic_bytes(cfg):
    """Bytes a token must move: K selected experts per layer, each head (dense rows + the 2K
    gathered K-hot rows), the layer-0 router, and the float16 in/out vectors."""
    E, d, K, H = cfg.E, cfg.d, cfg.K, cfg.head_hidden
    expert = K * cfg.expert_bytes()
    head = (H * d + 2 * K * H + H + E * H + E + E * d + 2 * K * E + E) * 2
    vec = 2 * d * 2
    ffn_call = expert + 3 * d * 2 + K * 8          # x, r in; y out; idx, w
    total = cfg.L * expert + (cfg.L - 1) * head + E * d * 2 + cfg.L * vec
    return total, ffn_call


def cpu_baseline(cfg, layers, syn, tokens=2):
    """Time the fp64 oracle (single thread) on `tokens` steady-state tokens of the same stack."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(1)
    except Exception:  # pragma: no cover
        limiter = None
    routers = [lw.router.cpu().numpy() for lw in layers]
    heads = [None if lw.head is None else {k: (None if v is None else v.cpu().numpy())
                                           for k, v in lw.head.tensors.items()} for lw in layers]
    packed = {}

    def expert_get(l, e):
        key = (l, int(e))
        if key not in packed:
            mats = layers[l].experts.tensors
            packed[key] = tuple(tuple(a[int(e)].cpu().numpy() for a in m) for m in mats)
        return packed[key]

    st = O.ChainState(cfg.L)
    kw = dict(E=cfg.E, K=cfg.K, bits=cfg.bits, group=cfg.group, router_get=lambda l: routers[l],
              head_get=lambda l: heads[l], expert_get=expert_get)
    _, st, _ = O.chain_token(syn.hidden(10**6, 1)[0].numpy(), st, **kw)      # bootstrap token, untimed
    t0 = time.perf_counter()
    for i in range(tokens):
        _, st, _ = O.chain_token(syn.hidden(10**6 + 1 + i, 1)[0].numpy(), st, **kw)
    elapsed = time.perf_counter() - t0
    return {"value": round(tokens / elapsed, 5), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{tokens} steady-state decode tokens through all {cfg.L} layers (fp64, explicit dequant, "
                      f"1 BLAS thread; includes copying each selected expert's packed bytes from HBM once)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=600)
    ap.add_argument("--warmup", type=int, default=60)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import int4_expert_ffn_amd as M
    import moe_synth as S

    dev = torch.device("cuda:0")
    cfg = S.CONFIGS["decode35b"]
    syn = S.Synth(cfg)
    t0 = time.time()
    layers = build_stack(cfg, syn, dev, M)
    torch.cuda.synchronize()
    log(f"stack resident: {cfg.L} layers, {torch.cuda.memory_allocated() / 2**30:.1f} GiB, {time.time() - t0:.1f} s")

    from int4_expert_ffn_amd.chain import DecodeStack
    stack = DecodeStack(layers, cfg.K, dev)
    n_pool = 3 * 64
    pool = syn.hidden(7, n_pool, dev)
    ring = torch.empty((3, cfg.d), dtype=torch.float16, device=dev)

    stream = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(stream):
        stack.token(0, pool[0])                 # bootstrap token: every layer routes itself
        ring.copy_(pool[0:3])
    stream.synchronize()
    graphs = []
    for j in range(3):                          # tokens 1, 2, 3 -> routing slots 1, 2, 0
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            stack.token(j + 1, ring[(j + 1) % 3])
        graphs.append(g)
    torch.cuda.synchronize()

    def run(n, start):
        for i in range(n):
            t = start + i
            slot = t % 3
            if slot == 1:                       # refill the three inputs of tokens t, t+1, t+2
                p = (t // 3 * 3) % n_pool
                ring.copy_(pool[p:p + 3])
            graphs[(t - 1) % 3].replay()

    args.warmup = -(-args.warmup // 3) * 3      # whole routing-slot rotations keep tokens consecutive
    with torch.cuda.stream(stream):
        run(args.warmup, 1)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start = 1 + args.warmup
    with torch.cuda.stream(stream):
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        ev0.record(stream)
        run(args.steps, start)
        ev1.record(stream)
        torch.cuda.synchronize()
        w1 = time.perf_counter()
    wall = w1 - w0
    ev_ms = ev0.elapsed_time(ev1)
    tok_s = args.steps / wall
    total_bytes, ffn_bytes = algorithmic_bytes(cfg)
    h_out = stack.h[cfg.L].float()
    assert torch.isfinite(h_out).all(), "non-finite decode output"

    # dominant step: the expert FFN of one layer (gate/up + SwiGLU kernel, down + combine kernel),
    # timed with HIP events on its stream over graph replays of all 40 layers' FFN calls.  Three
    # graphs use the three routing sets left by the decode run (480 distinct experts, 850 MB), so
    # the 256 MB last-level cache cannot hold a replay's weights.
    ffn_graphs = []
    fixed = [(stack.route_idx[s].clone(), stack.route_w[s].clone()) for s in range(3)]
    for idx_fixed, w_fixed in fixed:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for l, lw in enumerate(layers):
                x = stack.h[l]
                M.moe_expert_ffn_q4(1, cfg.K, M.MOE_INPUT_RMSNORM, x, idx_fixed[l], lw.experts, None, None,
                                    w_fixed[l], x, stack.h[l + 1], stack.ffn_ws)
        ffn_graphs.append(g)
    reps = 60
    with torch.cuda.stream(stream):
        for g in ffn_graphs:
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            ffn_graphs[i % 3].replay()
        e1.record(stream)
        torch.cuda.synchronize()
    ffn_us = e0.elapsed_time(e1) * 1e3 / (reps * cfg.L)
    achieved = ffn_bytes / (ffn_us * 1e-6) / 1e9

    rec = {
        "metric": "MoE-layer decode tokens/s at batch 1 + achieved HBM GB/s (% of peak)",
        "value": round(tok_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "decode35b: d_model 2048, 256 experts, top-4, expert I 512, int4 affine g64, 40 layers "
                        "resident, prerouter heads 2560->1024->256 (+linear 2560->256), batch 1",
            "global_batch": 1, "layers": cfg.L, "accumulate": "f32", "weights": "int4 affine g64 (fp16 scale/bias)",
            "parallelism": "none (1 GPU)",
        },
        "hbm": {
            "algorithmic_bytes_per_token": total_bytes,
            "achieved_GBps": round(total_bytes * tok_s / 1e9, 1),
            "frac_of_peak": round(total_bytes * tok_s / 1e9 / HBM_PEAK_GBPS, 4),
            "event_ms_per_step": round(ev_ms / args.steps, 4),
        },
        "roofline": {
            "kernel": "expert FFN of one layer (k_gateup + k_down)",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": None,
            "bytes_per_launch": ffn_bytes,
            "avg_us": round(ffn_us, 3),
        },
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        rec["cpu_baseline"] = cpu_baseline(cfg, layers, syn)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
