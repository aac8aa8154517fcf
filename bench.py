#!/usr/bin/env python3
"""Decode benchmark of the prerouted MoE stack on one MI355X.

Workload (one step = one token through the whole stack): the 35B-shaped decode layer --
d_model 2048, 256 experts, top-4, expert intermediate 512, int4 affine group 64, 40 layers
resident in HBM, prerouter heads (fc1 2560->1024, erf-GELU, fc2 1024->256, linear 2560->256) on
layers 0..38, layer 0 routed by its own router -- batch 1, synthetic seeded weights and hidden
states (a fresh draw per token).  Each token is one HIP-graph replay holding one moe_decode_step
launch (the persistent kernel that runs all 40 layers); inputs are resident in HBM before the
timed region.  The same schedule issued as per-layer C-ABI calls is timed beside it for context.

Prints one JSON line: tokens/s, the roofline of the dominant kernel (k_decode_step, timed with
HIP events on its stream: algorithmic bytes per token / time per token) and the CPU oracle timed
on a bounded sample.
"""
import argparse
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
STEP_KERNEL_SOURCES = ("int4_expert_ffn_amd/csrc/k_decode_step.hip", "int4_expert_ffn_amd/csrc/moe_device.h",
                       "int4_expert_ffn_amd/csrc/moe_launch.h", "include/moe.h")
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "k_decode_step_decode35b_traffic.json")


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


_CODE_TOKENS = re.compile(r'"(?:\\.|[^"\\\n])*"|//[^\n]*|/\*.*?\*/', re.S)


def kernel_source_hash():
    """sha256 over the code of the sources the persistent kernel is built from, with comments
    dropped and whitespace runs collapsed (to tell whether a stored counter record still
    describes the kernel that runs; an edit of a comment does not change the kernel)."""
    import hashlib
    h = hashlib.sha256()
    for rel in STEP_KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            src = f.read()
        code = _CODE_TOKENS.sub(lambda m: m.group(0) if m.group(0).startswith('"') else " ", src)
        h.update(" ".join(code.split()).encode())
    return h.hexdigest()


def stored_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter record, or None when there is
    none or the kernel sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_RECORD) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def copy_calibration(mib):
    """A plain device copy of `mib` MiB (reads and writes that many bytes), three times: the
    reference that scales the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    n = mib << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "copies": 3}), flush=True)


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
    ap.add_argument("--no-per-layer", action="store_true", help="skip the per-layer-calls context timing")
    ap.add_argument("--eager", action="store_true",
                    help="launch each timed token directly instead of replaying a HIP graph (for counter profiling)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (the reference for HBM byte counters)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
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
    n_pool = 3 * 64
    pool = syn.hidden(7, n_pool, dev)
    ring = torch.empty((3, cfg.d), dtype=torch.float16, device=dev)
    stream = torch.cuda.Stream(device=dev)

    def capture(stack, use_step):
        """Three graphs, one per routing slot (tokens 1, 2, 3), each reading its ring slot."""
        with torch.cuda.stream(stream):
            if use_step:
                stack.step(0, pool[0])          # token 0: every layer routes itself
            else:
                stack.token(0, pool[0])
            ring.copy_(pool[0:3])
        stream.synchronize()
        graphs = []
        for j in range(3):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                if use_step:
                    stack.step(j + 1, ring[(j + 1) % 3])
                else:
                    stack.token(j + 1, ring[(j + 1) % 3])
            graphs.append(g)
        torch.cuda.synchronize()
        return graphs

    def run(graphs, n, start):
        for i in range(n):
            t = start + i
            if t % 3 == 1:                       # refill the inputs of tokens t, t+1, t+2
                p = (t // 3 * 3) % n_pool
                ring.copy_(pool[p:p + 3])
            if callable(graphs):
                graphs(t)
            else:
                graphs[(t - 1) % 3].replay()

    def timed(graphs, steps, warmup):
        warmup = -(-warmup // 3) * 3             # whole slot rotations keep tokens consecutive
        with torch.cuda.stream(stream):
            run(graphs, warmup, 1)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            torch.cuda.synchronize()
            w0 = time.perf_counter()
            e0.record(stream)
            run(graphs, steps, 1 + warmup)
            e1.record(stream)
            torch.cuda.synchronize()
            w1 = time.perf_counter()
        return w1 - w0, e0.elapsed_time(e1), warmup

    # the timed step: one persistent-kernel launch (moe_decode_step) per token
    stack = DecodeStack(layers, cfg.K, dev)
    graphs = capture(stack, True)
    if args.eager:                               # same tokens, direct launches (graphs captured but unused)
        graphs = lambda t: stack.step(t, ring[t % 3])
    wall, ev_ms, args.warmup = timed(graphs, args.steps, args.warmup)
    assert stack.step_error_word() == 0, "a wait inside the decode kernel ran out of time"
    h_out = stack.h[cfg.L].float()
    assert torch.isfinite(h_out).all(), "non-finite decode output"
    tok_s = args.steps / wall
    total_bytes, ffn_bytes = algorithmic_bytes(cfg)
    step_us = ev_ms * 1e3 / args.steps                 # HIP-event time per token on the stream
    achieved = total_bytes / (step_us * 1e-6) / 1e9

    # context: the same schedule as per-layer C-ABI calls (5 launches per layer)
    del graphs
    per_layer_tok_s = None
    if not args.no_per_layer:
        stack2 = DecodeStack(layers, cfg.K, dev)
        graphs2 = capture(stack2, False)
        n2 = max(30, args.steps // 4)
        wall2, ev2, _ = timed(graphs2, n2, 30)
        per_layer_tok_s = round(n2 / wall2, 2)
        del graphs2
    traffic = stored_traffic()

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
        },
        "roofline": {
            "kernel": "k_decode_step (moe_decode_step: all 40 layers of one token in one launch)",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "bytes_per_launch": total_bytes,
            "avg_us": round(step_us, 2),
        },
        "per_layer_calls": {"tokens_per_s": per_layer_tok_s, "launches_per_token": 5 * cfg.L - 2,
                            "note": "same schedule issued as per-layer C-ABI calls in a HIP graph"},
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        rec["cpu_baseline"] = cpu_baseline(cfg, layers, syn)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
