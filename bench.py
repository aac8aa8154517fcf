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


def build_stack(cfg, syn, dev, M, norm_gain=False):
    from int4_expert_ffn_amd.chain import DecodeStack, LayerWeights
    import moe_synth as S
    layers = []
    routers = [syn.router(l, dev) for l in range(cfg.L + 1)]
    for l in range(cfg.L):
        mats = S.fill_experts(syn, l, dev)
        ex = M.Experts(mats["gate"], mats["up"], mats["down"], cfg.bits, cfg.group)
        head = None
        if cfg.head_hidden and l < cfg.L - 1:
            hw = syn.head(l, dev)
            hw["lin_x"] = routers[l + 1]          # the head's linear path is the next router
            head = M.PrerouterWeights(hw)
        layers.append(LayerWeights(ex, routers[l], head, syn.norm_gain(l, dev) if norm_gain else None))
    return layers


def algorithmic_bytes(cfg):
    """Bytes a token must move through the whole stack, and through its expert FFN steps alone.
    With prerouter heads: K selected experts per layer, each head (dense rows + the 2K gathered
    K-hot rows), the layer-0 router and the float16 in/out vectors of every layer.  Without: K
    experts, the layer's router and the in/out vectors of every layer.  Expert FFN alone: the
    experts and the vectors."""
    E, d, K, H = cfg.E, cfg.d, cfg.K, cfg.head_hidden
    expert = K * cfg.expert_bytes()
    vec = 2 * d * 2
    router = E * d * 2
    if H:
        head = (H * d + 2 * K * H + H + E * H + E + E * d + 2 * K * E + E) * 2
        total = cfg.L * expert + (cfg.L - 1) * head + router + cfg.L * vec
    else:
        total = cfg.L * (expert + router + vec)
    return total, cfg.L * (expert + vec)


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


def host_cores():
    """Cores this process may run on (the box's share of the host)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_baseline(cfg, layers, syn, tokens, streams=1):
    """Time the fp64 oracle (oracle.chain_token, as it stands) on steady-state tokens of the same
    stack, one BLAS thread per stream.  streams == 1: `tokens` tokens of one token stream.
    streams > 1: that many independent token streams (each its own hidden states and routing
    state, all starting from one bootstrap token) run `tokens` tokens each in as many Python
    threads, one per core; numpy releases the interpreter lock inside its array operations, so
    the streams run in parallel, and the figure is their aggregate tokens/s (the oracle on every
    core, for independent decode streams, since one stream's tokens depend on each other)."""
    import copy
    import threading

    import oracle as O
    limiter = None
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(1)
    except Exception:  # pragma: no cover
        limiter = None
    routers = [lw.router.cpu().numpy() for lw in layers]
    heads = [None if lw.head is None else {k: (None if v is None else v.cpu().numpy())
                                           for k, v in lw.head.tensors.items()} for lw in layers]
    packed = {}
    lock = threading.Lock()

    def expert_get(l, e):
        key = (l, int(e))
        with lock:
            got = packed.get(key)
        if got is None:
            mats = layers[l].experts.tensors
            got = tuple(tuple(a[int(e)].cpu().numpy() for a in m) for m in mats)
            with lock:
                packed[key] = got
        return got

    kw = dict(E=cfg.E, K=cfg.K, bits=cfg.bits, group=cfg.group, router_get=lambda l: routers[l],
              head_get=lambda l: heads[l], expert_get=expert_get)
    _, st0, _ = O.chain_token(syn.hidden(10**6, 1)[0].numpy(), O.ChainState(cfg.L), **kw)  # bootstrap, untimed
    hs = syn.hidden(10**6 + 1, streams * tokens).numpy()

    def stream(i):
        st = copy.deepcopy(st0)
        for j in range(tokens):
            _, st, _ = O.chain_token(hs[i * tokens + j], st, **kw)

    t0 = time.perf_counter()
    if streams == 1:
        stream(0)
    else:
        ths = [threading.Thread(target=stream, args=(i,)) for i in range(streams)]
        for t in ths:
            t.start()
        for t in ths:
            t.join()
    elapsed = time.perf_counter() - t0
    if limiter is not None:
        limiter.restore_original_limits()
    n = streams * tokens
    what = (f"{tokens} steady-state decode tokens through all {cfg.L} layers" if streams == 1 else
            f"{streams} independent token streams x {tokens} steady-state tokens through all {cfg.L} layers, one "
            f"Python thread per stream")
    return {"value": round(n / elapsed, 5), "unit": "tokens/s", "cores": streams, "host_cores": host_cores(),
            "kind": "oracle", "cpu": cpu_model(),
            "sample": what + " (fp64, explicit dequant, 1 BLAS thread per stream; includes copying each selected "
                             "expert's packed bytes from HBM once)"}


def cpu_model():
    """The host CPU as /proc/cpuinfo names it (model name, family, model, stepping)."""
    info = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if ":" in line:
                    k, v = line.split(":", 1)
                    info.setdefault(k.strip(), v.strip())
    except OSError:
        return None
    name = info.get("model name")
    if name is None:
        return None
    extra = ", ".join(f"{k} {info[k]}" for k in ("cpu family", "model", "stepping") if k in info)
    return f"{name} ({extra})" if extra else name


STACK_WORKLOADS = ("decode35b", "widek8", "large-int4", "large-int2")
WORKLOADS = STACK_WORKLOADS + ("tiny", "batched", "relu-sparse", "stream", "exchange")
METRIC = "MoE-layer decode tokens/s at batch 1 + achieved HBM GB/s (% of peak)"


def describe(cfg):
    w = (f"{cfg.name}: d_model {cfg.d}, {cfg.E} experts, top-{cfg.K}, expert I {cfg.I}, "
         f"int{cfg.bits} affine g{cfg.group}, {cfg.L} layer{'s' if cfg.L > 1 else ''} resident")
    if cfg.head_hidden:
        w += (f", prerouter heads {cfg.d + 2 * cfg.E}->{cfg.head_hidden}->{cfg.E} "
              f"(+linear {cfg.d + 2 * cfg.E}->{cfg.E})")
    elif cfg.T == 1:
        w += ", every layer routed by its own router"
    if cfg.shared_expert:
        w += f", shared expert + LoRA r{cfg.lora_rank} alpha {cfg.lora_alpha:g}"
    return w + (f", batch {cfg.T}" if cfg.T > 1 else ", batch 1")


def base_record(args, cfg, value, wall, steps):
    return {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": describe(cfg),
            "global_batch": cfg.T, "layers": cfg.L, "accumulate": "f32",
            "weights": f"int{cfg.bits} affine g{cfg.group} (fp16 scale/bias)",
            "parallelism": "none (1 GPU)",
        },
    }


def roofline(kernel, nbytes, avg_us, traffic):
    achieved = nbytes / (avg_us * 1e-6) / 1e9
    return {"kernel": kernel, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic, "bytes_per_launch": nbytes,
            "avg_us": round(avg_us, 2)}


class Timer:
    """Token loops on one stream: graph replays (or direct launches), HIP events around the timed
    region, fresh inputs from a resident pool written into a 3-slot ring every three tokens."""

    def __init__(self, torch, dev, pool):
        self.torch, self.pool = torch, pool
        self.n_pool = pool.shape[0]
        self.ring = torch.empty((3,) + tuple(pool.shape[1:]), dtype=pool.dtype, device=dev)
        self.stream = torch.cuda.Stream(device=dev)

    def capture(self, enqueue):
        """Three graphs, one per routing slot (tokens 1, 2, 3), each reading its ring slot;
        enqueue(t, h) issues token t (token 0 runs eagerly first)."""
        torch = self.torch
        with torch.cuda.stream(self.stream):
            enqueue(0, self.pool[0])
            self.ring.copy_(self.pool[0:3])
        self.stream.synchronize()
        graphs = []
        for j in range(3):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=self.stream):
                enqueue(j + 1, self.ring[(j + 1) % 3])
            graphs.append(g)
        torch.cuda.synchronize()
        return graphs

    def run(self, graphs, n, start, refill=None):
        for i in range(n):
            t = start + i
            if t % 3 == 1:                       # refill the inputs of tokens t, t+1, t+2
                p = (t // 3 * 3) % self.n_pool
                self.ring.copy_(self.pool[p:p + 3])
                if refill is not None:
                    refill(p)
            if callable(graphs):
                graphs(t)
            else:
                graphs[(t - 1) % 3].replay()

    def timed(self, graphs, steps, warmup, refill=None, start=1):
        """(wall seconds, HIP-event milliseconds, warm-up tokens actually run); tokens are numbered
        from `start` (1 more than a multiple of 3)."""
        torch = self.torch
        warmup = -(-warmup // 3) * 3             # whole slot rotations keep tokens consecutive
        with torch.cuda.stream(self.stream):
            self.run(graphs, warmup, start, refill)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(self.stream):
            torch.cuda.synchronize()
            w0 = time.perf_counter()
            e0.record(self.stream)
            self.run(graphs, steps, start + warmup, refill)
            e1.record(self.stream)
            torch.cuda.synchronize()
            w1 = time.perf_counter()
        return w1 - w0, e0.elapsed_time(e1), warmup


def routing_histogram(cfg, layers, syn, torch, dev, tokens=1024):
    """Experts chosen per layer over `tokens` decode tokens of the chain (a fresh hidden state per
    token): min and max count per expert against the uniform expectation tokens*K/E, and Pearson's
    chi-square over the E experts (E - 1 degrees of freedom)."""
    from int4_expert_ffn_amd.chain import DecodeStack
    stack = DecodeStack(layers, cfg.K, dev)
    hs = syn.hidden(11, tokens, dev)
    rec = torch.empty((tokens, cfg.L, cfg.K), dtype=torch.int32, device=dev)
    for t in range(tokens):
        stack.step(t, hs[t])
        rec[t].copy_(stack.route_idx[t % 3])
    torch.cuda.synchronize()
    assert stack.step_error_word() == 0, "a wait inside the decode kernel ran out of time (histogram)"
    idx = rec.cpu().long()
    expect = tokens * cfg.K / cfg.E
    mins, maxs, chi2 = [], [], []
    for l in range(cfg.L):
        n = torch.bincount(idx[:, l].reshape(-1), minlength=cfg.E).double()
        mins.append(int(n.min()))
        maxs.append(int(n.max()))
        chi2.append(round(float(((n - expect) ** 2).sum() / expect), 1))
    srt = sorted(chi2)
    return {"tokens": tokens, "expected_per_expert": expect, "dof": cfg.E - 1,
            "min_count": min(mins), "max_count": max(maxs), "chi2_median": srt[len(srt) // 2], "chi2_max": srt[-1],
            "chi2_per_layer": chi2,
            "note": "routing the full path chose (layer 0 and the first token self-routed, the rest as the stack routes)"}


def exchange_probe(M, torch, dev, words):
    """The committed exchange-latency probe (moe_exchange_probe): one workgroup per compute unit.
    ring: one tagged word passed workgroup to workgroup (consecutive workgroups sit on different
    XCDs), the latency of one dependent hand-off; all: every workgroup publishes its slice of a
    `words`-word vector and polls it whole, phase after phase (the shape of the decode kernel's
    exchanges: polled with 8-byte agent-scope atomic loads from one of eight copies, as the kernel
    does, up to 1,024 words; 16-byte buffer loads beyond, a form the probe offers there), the
    period of such an exchange loop."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.zeros(1 + 3 * cus, dtype=torch.int32, device=dev)
    res = {}
    wide = 2 if words <= 1024 else 1
    for name, pat, gs, w, it, reps_, wd in (("ring_hop_us", M.MOE_XCHG_RING, 8, 0, 200, 1, 0),
                                           ("all_exchange_us", M.MOE_XCHG_ALL, cus, words, 200, 8, wide)):
        cfg = M.moe_xchg_cfg(pat, cus, gs, 0, w, it, M.MOE_XCHG_SCOPE_DEVICE, M.MOE_XCHG_SCOPE_DEVICE, 1, reps_, wd)
        ws = torch.zeros(M.moe_exchange_probe_workspace_size(cfg), dtype=torch.uint8, device=dev)
        vals = []
        for rep in range(3):
            cfg.epoch = rep + 1
            out.zero_()
            M.moe_exchange_probe(cfg, ws, out)
            torch.cuda.synchronize()
            o = out.cpu().numpy().view("uint32").astype("int64")
            assert o[0] == 0, "a wait of the exchange probe ran out of time"
            ticks = o[1::3] | (o[2::3] << 32)
            if pat == M.MOE_XCHG_RING:
                vals.append(float(ticks[0::gs].max()) / 100.0 / (it * gs))   # member 0 of each ring
            else:
                vals.append(float(ticks.max()) / 100.0 / it)
        res[name] = round(sorted(vals)[1], 3)
    res["workgroups"] = cus
    res["words"] = words
    res["all_exchange_loads"] = ("8-byte agent-scope atomic loads" if wide == 2 else "16-byte buffer loads") + ", 8 copies"
    return res


def bench_exchange(args, torch, M, dev):
    """The exchange-latency probe over the shapes the decode kernel's design rests on (one
    workgroup per compute unit): single hand-offs (rings across XCDs and inside one), and
    all-to-all exchanges of 256..2,048 tagged words with the three polling-load forms, grouped
    across the chip or inside one XCD, with and without eight copies."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    Dv, Xv = M.MOE_XCHG_SCOPE_DEVICE, M.MOE_XCHG_SCOPE_XCD
    forms = {0: "8-byte buffer loads", 1: "16-byte buffer loads", 2: "8-byte agent-scope atomic loads (global)"}
    rows = []
    epoch = [1]

    def run(pattern, n, gs, xl, words, iters, ls, ss, reps_=1, wide=0):
        cfg = M.moe_xchg_cfg(pattern, n, gs, xl, words, iters, ls, ss, 0, reps_, wide)
        ws = torch.zeros(M.moe_exchange_probe_workspace_size(cfg), dtype=torch.uint8, device=dev)
        out = torch.zeros(1 + 3 * n, dtype=torch.int32, device=dev)
        vals, errs = [], 0
        for _ in range(3):
            epoch[0] += 1
            cfg.epoch = epoch[0]
            out.zero_()
            M.moe_exchange_probe(cfg, ws, out)
            torch.cuda.synchronize()
            o = out.cpu().numpy().view("uint32").astype("int64")
            errs += int(o[0])
            ticks = o[1::3] | (o[2::3] << 32)
            if pattern == M.MOE_XCHG_RING:
                first = [b for b in range(n) if (b // (n // gs) if xl else b % gs) == 0]
                vals.append(float(ticks[first].max()) / 100.0 / (iters * gs))
            else:
                vals.append(float(ticks.max()) / 100.0 / iters)
        return round(sorted(vals)[1], 3), errs

    R, A = M.MOE_XCHG_RING, M.MOE_XCHG_ALL
    for label, gs, xl, ss in (("ring, hops across XCDs, device-coherent stores", 8, 0, Dv),
                              ("ring, hops inside one XCD, device-coherent stores", 32, 1, Dv),
                              ("ring, hops inside one XCD, stores to the XCD's L2", 32, 1, Xv)):
        us, err = run(R, cus, gs, xl, 0, 100, Dv, ss)
        rows.append({"pattern": "ring", "what": label, "us_per_hop": us, "timeouts": err})
    for words in (256, 512, 1024, 2048):
        for wide in (0, 1, 2):
            if wide == 2 and words > 1024:
                continue
            us, err = run(A, cus, cus, 0, words, 200, Dv, Dv, 1, wide)
            rows.append({"pattern": "all", "workgroups": cus, "group": cus, "words": words, "loads": forms[wide],
                         "us_per_exchange": us, "timeouts": err})
    for words, wide, reps_ in ((1024, 2, 8), (1024, 1, 8)):
        us, err = run(A, cus, cus, 0, words, 200, Dv, Dv, reps_, wide)
        rows.append({"pattern": "all", "workgroups": cus, "group": cus, "words": words, "loads": forms[wide],
                     "copies": reps_, "us_per_exchange": us, "timeouts": err})
    for words, wide, ss in ((1024, 2, Dv), (1024, 1, Dv), (512, 0, Xv)):
        us, err = run(A, cus, 32, 1, words, 200, Dv, ss, 1, wide)
        rows.append({"pattern": "all", "workgroups": cus, "group": "32 on one XCD (8 groups)", "words": words,
                     "loads": forms[wide], "stores": "device" if ss == Dv else "XCD L2",
                     "us_per_exchange": us, "timeouts": err})
    return {"metric": "tagged-word exchange latency between resident workgroups (measurement aid)",
            "unit": "us", "higher_is_better": False, "n_gpus": 1, "data": "synthetic", "rows": rows,
            "note": "one workgroup of one wave per compute unit; all: per phase, every workgroup publishes its "
                    "slice and polls the whole vector (the period of such a loop); ring: one word passed on"}


def phase_breakdown(layers, cfg, syn, torch, dev, M, tokens=12, warm=20):
    """Per-layer time split of the persistent kernel from its phase stamps (moe_decode_step_stamped,
    the global 100 MHz counter): medians over workgroups and over the inner layers of the last
    `tokens` tokens.  h_exchange / act_exchange: from the last workgroup's store of the vector to
    the median workgroup having all of it; gate_up: h seen -> SwiGLU outputs stored (median);
    store_spread: median -> last workgroup storing; act_to_down: all SwiGLU outputs in -> down
    phase starts; down: down phase -> layer output stored.  On a stack whose layers route
    themselves, the router phase too: router_dot (h seen -> the workgroup's logit stored),
    logit_exchange (last logit stored -> the median polling wave has all E), topk (-> the compute
    waves know the routing), to_gate_up_dots (routing known -> gate/up dot products done)."""
    import numpy as np
    from int4_expert_ffn_amd.chain import DecodeStack
    stack = DecodeStack(layers, cfg.K, dev)
    G = stack.grid()
    st = torch.zeros((G, cfg.L, 16), dtype=torch.int64, device=dev)
    hs = syn.hidden(17, warm + tokens, dev)
    self_routed = not cfg.head_hidden
    rows, tok_us = [], []
    for t in range(warm + tokens):
        stack.step(t, hs[t], stamps=st if t >= warm else None)
        if t >= warm:
            torch.cuda.synchronize()
            a = st.cpu().numpy().astype(np.float64) / 100.0
            tok_us.append(float(a[:, -1, 6].max() - a[:, 0, 0].min()))
            for l in range(1, cfg.L - 1):
                s, pv, nx = a[:, l, :], a[:, l - 1, :], a[:, l + 1, :]
                med = lambda v: float(np.median(v))
                rows.append({
                    "h_exchange": med(s[:, 1]) - pv[:, 6].max(),
                    "gate_up": med(s[:, 4]) - med(s[:, 3]),
                    "act_store_spread": s[:, 4].max() - med(s[:, 4]),
                    "act_exchange": med(s[:, 2]) - s[:, 4].max(),
                    "act_to_down": med(s[:, 5]) - med(s[:, 2]),
                    "down": med(s[:, 6]) - med(s[:, 5]),
                    "h_store_spread": s[:, 6].max() - med(s[:, 6]),
                    "layer": med(nx[:, 1]) - med(s[:, 1]),
                })
                if self_routed:
                    rows[-1].update({
                        "router_dot": med(s[:, 10]) - med(s[:, 3]),
                        "logit_exchange": med(s[:, 15]) - s[:, 10].max(),
                        "topk": med(s[:, 11]) - med(s[:, 15]),
                        "to_gate_up_dots": med(s[:, 8]) - med(s[:, 11]),
                    })
    assert stack.step_error_word() == 0, "a wait inside the decode kernel ran out of time (stamped)"
    out = {k: round(float(np.median([r[k] for r in rows])), 3) for k in rows[0]}
    out["token_us"] = round(float(np.median(tok_us)), 1)
    out["layers_used"] = f"1..{cfg.L - 2} (inner layers), {tokens} tokens"
    return out


def bench_stack(args, cfg, torch, M, S, dev):
    """A resident L-layer stack at batch 1: the timed step is one moe_decode_step launch per token
    (the persistent kernel running every layer); the expert FFN steps alone and the per-layer
    C-ABI calls are timed beside it."""
    from int4_expert_ffn_amd.chain import DecodeStack
    syn = S.Synth(cfg)
    t0 = time.time()
    layers = build_stack(cfg, syn, dev, M, norm_gain=args.norm_gain)
    torch.cuda.synchronize()
    log(f"stack resident: {cfg.L} layers, {torch.cuda.memory_allocated() / 2**30:.1f} GiB, {time.time() - t0:.1f} s")
    tm = Timer(torch, dev, syn.hidden(7, 3 * 64, dev))

    stack = DecodeStack(layers, cfg.K, dev)
    graphs = tm.capture(lambda t, h: stack.step(t, h))
    if args.eager:                               # same tokens, direct launches (graphs captured but unused)
        graphs = lambda t: stack.step(t, tm.ring[t % 3])
    runs = [tm.timed(graphs, args.steps, args.warmup)]
    args.warmup = runs[0][2]
    assert stack.step_error_word() == 0, "a wait inside the decode kernel ran out of time"
    h_out = stack.h[cfg.L].float()
    assert torch.isfinite(h_out).all(), "non-finite decode output"
    # the same timed loop again (no further warm-up): `value` is the median run of the repeats
    runs += [tm.timed(graphs, args.steps, 0) for _ in range(args.repeats - 1)]
    assert stack.step_error_word() == 0, "a wait inside the decode kernel ran out of time (repeats)"
    del graphs
    reps = [args.steps / r[0] for r in runs]
    wall, ev_ms, _ = sorted(runs, key=lambda r: r[0])[len(runs) // 2]
    total_bytes, eo_bytes = algorithmic_bytes(cfg)
    step_us = ev_ms * 1e3 / args.steps               # HIP-event time per token on the stream (median run)

    # the expert FFN steps alone (gate/up + SwiGLU, down + combine + residual through all layers, the
    # RMS-norm chain included) on the routing the full path chose for the same tokens, recorded
    # per token and written into the routing slots between tokens
    expert_only = None
    if not args.no_expert_only:
        n_pool = tm.n_pool
        rec_i = torch.empty((n_pool, cfg.L, cfg.K), dtype=torch.int32, device=dev)
        rec_w = torch.empty((n_pool, cfg.L, cfg.K), dtype=torch.float32, device=dev)
        if cfg.head_hidden:
            # prerouted: the routing the full path chose for the same tokens
            routing_note = "the routing the full path chose for the same tokens"
            src = DecodeStack(layers, cfg.K, dev)
            with torch.cuda.stream(tm.stream):
                for t in range(n_pool):
                    src.step(t, tm.pool[t])
                    rec_i[t].copy_(src.route_idx[t % 3])
                    rec_w[t].copy_(src.route_w[t % 3])
            torch.cuda.synchronize()
            assert src.step_error_word() == 0, "a wait inside the decode kernel ran out of time (recording)"
            del src
        else:
            # self-routed: per (token, layer) K distinct experts drawn uniformly, as the top-K of
            # seeded N(0, 1) logits, with their renormalised softmax weights
            routing_note = "seeded routing drawn uniformly per (token, layer): top-K of N(0,1) logits, renormalised"
            lg = syn.logits(13, n_pool * cfg.L, dev)
            M.moe_route_topk(n_pool * cfg.L, cfg.d, cfg.E, cfg.K, M.MOE_TOPK_RENORM, None, None, lg,
                             rec_i.view(-1, cfg.K), rec_w.view(-1, cfg.K))
            torch.cuda.synchronize()
        stack3 = DecodeStack(layers, cfg.K, dev)
        stack3.route_idx.copy_(rec_i[0:3])
        stack3.route_w.copy_(rec_w[0:3])

        def refill(p):
            stack3.route_idx.copy_(rec_i[p:p + 3])
            stack3.route_w.copy_(rec_w[p:p + 3])

        graphs3 = tm.capture(lambda t, h: stack3.step(t, h, given_routing=True))
        wall3, ev3, _ = tm.timed(graphs3, args.steps, args.warmup, refill)
        assert stack3.step_error_word() == 0, "a wait inside the decode kernel ran out of time (expert only)"
        del graphs3
        eo_us = ev3 * 1e3 / args.steps
        expert_only = {
            "tokens_per_s": round(args.steps / wall3, 2), "avg_us": round(eo_us, 2),
            "algorithmic_bytes_per_token": eo_bytes,
            "achieved_GBps": round(eo_bytes / (eo_us * 1e-6) / 1e9, 1),
            "frac_of_peak": round(eo_bytes / (eo_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "note": "S3-S6 alone (moe_decode_step with MOE_DECODE_GIVEN_ROUTING) on " + routing_note +
                    "; HIP-event time per token includes the routing refill copies",
        }

    # context: the same schedule as per-layer C-ABI calls
    per_layer_tok_s = None
    if not args.no_per_layer:
        stack2 = DecodeStack(layers, cfg.K, dev)
        graphs2 = tm.capture(lambda t, h: stack2.token(t, h))
        n2 = max(30, args.steps // 4)
        wall2, _, _ = tm.timed(graphs2, n2, 30)
        per_layer_tok_s = round(n2 / wall2, 2)
        del graphs2
    launches = (5 * cfg.L - 2) if cfg.head_hidden else 4 * cfg.L

    # cold tokens: a 1 GiB streaming read before each token evicts L2 and the memory-side cache, and
    # HIP events time the token's launch alone
    cold = None
    if not args.no_cold:
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        fold = torch.empty(M.MOE_READ_PROBE_BLOCKS, dtype=torch.int32, device=dev)
        stack_c = DecodeStack(layers, cfg.K, dev)
        graphs_c = tm.capture(lambda t, h: stack_c.step(t, h))
        n_cold = max(30, args.steps // 4) // 3 * 3
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_cold)]
        with torch.cuda.stream(tm.stream):
            tm.run(graphs_c, 30, 1)
            for i in range(n_cold):
                t = 31 + i
                if t % 3 == 1:
                    p = (t // 3 * 3) % tm.n_pool
                    tm.ring.copy_(tm.pool[p:p + 3])
                M.moe_read_probe(flush, fold)
                evs[i][0].record(tm.stream)
                graphs_c[(t - 1) % 3].replay()
                evs[i][1].record(tm.stream)
        torch.cuda.synchronize()
        assert stack_c.step_error_word() == 0, "a wait inside the decode kernel ran out of time (cold)"
        cold_us = sum(a.elapsed_time(b) for a, b in evs) * 1e3 / n_cold
        cold = {"tokens": n_cold, "avg_us": round(cold_us, 2), "tokens_per_s": round(1e6 / cold_us, 2),
                "achieved_GBps": round(total_bytes / (cold_us * 1e-6) / 1e9, 1),
                "frac_of_peak": round(total_bytes / (cold_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                "note": "a 1 GiB streaming read before each token; the token's launch timed alone"}
        del graphs_c, stack_c, flush
    # warm experts (the bound on prefetching a token's experts into the memory-side cache at token
    # start): before each token, every expert the token will use in layers 1..L-1 (their routing
    # is known then: the previous token's heads wrote it) is read once with the streaming probe,
    # deepest layer first so that the first layers are the most recently touched; HIP events then
    # time the token's launch alone.  Prerouted stacks only (a self-routed layer's experts are not
    # known before the layer runs).
    warm = None
    if cfg.head_hidden and not args.no_cold:
        fold = torch.empty(M.MOE_READ_PROBE_BLOCKS, dtype=torch.int32, device=dev)
        stack_w = DecodeStack(layers, cfg.K, dev)
        graphs_w = tm.capture(lambda t, h: stack_w.step(t, h))
        n_warm = max(30, args.steps // 10) // 3 * 3
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_warm)]
        touched = 0
        with torch.cuda.stream(tm.stream):
            tm.run(graphs_w, 30, 1)
            for i in range(n_warm):
                t = 31 + i
                if t % 3 == 1:
                    p = (t // 3 * 3) % tm.n_pool
                    tm.ring.copy_(tm.pool[p:p + 3])
                idx = stack_w.route_idx[t % 3].cpu()          # this token's routing (written by token t-1)
                for l in range(cfg.L - 1, 0, -1):
                    for e in idx[l].tolist():
                        for mat in layers[l].experts.tensors:
                            for arr in mat:
                                M.moe_read_probe(arr[e], fold)
                                touched += arr[e].numel() * arr[e].element_size()
                evs[i][0].record(tm.stream)
                graphs_w[(t - 1) % 3].replay()
                evs[i][1].record(tm.stream)
        torch.cuda.synchronize()
        assert stack_w.step_error_word() == 0, "a wait inside the decode kernel ran out of time (warm)"
        warm_us = sum(a.elapsed_time(b) for a, b in evs) * 1e3 / n_warm
        warm = {"tokens": n_warm, "avg_us": round(warm_us, 2), "tokens_per_s": round(1e6 / warm_us, 2),
                "expert_bytes_touched_per_token": touched // n_warm,
                "note": "each token's experts of layers 1..L-1 read into the caches just before the token "
                        "(deepest layer first); the token's launch timed alone"}
        del graphs_w, stack_w
    # measured HBM read ceiling: a plain 16-byte streaming read over 8 GiB
    buf = torch.empty(8 << 30, dtype=torch.uint8, device=dev)
    fold = torch.empty(M.MOE_READ_PROBE_BLOCKS, dtype=torch.int32, device=dev)
    for _ in range(2):
        M.moe_read_probe(buf, fold)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        M.moe_read_probe(buf, fold)
    e1.record()
    torch.cuda.synchronize()
    read_ceiling = 5 * buf.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del buf

    hist = routing_histogram(cfg, layers, syn, torch, dev) if not args.no_histogram else None
    phases = xprobe = None
    if not args.no_phases:
        phases = phase_breakdown(layers, cfg, syn, torch, dev, M)
        xprobe = exchange_probe(M, torch, dev, cfg.d // 2)

    tok_s = args.steps / wall
    rec = base_record(args, cfg, tok_s, wall, args.steps)
    if args.norm_gain:
        rec["config"]["workload"] += ", layer inputs RMS-normalised with a per-layer float16 gain"
        total_bytes += cfg.L * cfg.d * 2          # the gains
    rec["hbm"] = {"algorithmic_bytes_per_token": total_bytes,
                  "achieved_GBps": round(total_bytes * tok_s / 1e9, 1),
                  "frac_of_peak": round(total_bytes * tok_s / 1e9 / HBM_PEAK_GBPS, 4)}
    rec["hbm"]["measured_read_ceiling_GBps"] = round(read_ceiling, 1)
    rec["hbm"]["frac_of_measured_ceiling"] = round(total_bytes * tok_s / 1e9 / read_ceiling, 4)
    rec["roofline"] = roofline(f"k_decode_step (moe_decode_step: all {cfg.L} layers of one token in one launch)",
                               total_bytes, step_us,
                               stored_traffic() if cfg.name == "decode35b" and not args.norm_gain else None)
    rec["roofline"]["measured_read_ceiling_GBps"] = round(read_ceiling, 1)
    rec["roofline"]["frac_of_measured_ceiling"] = round(rec["roofline"]["achieved"] / read_ceiling, 4)
    rec["cold"] = cold
    rec["warm_experts"] = warm
    if phases is not None:
        floor = xprobe["ring_hop_us"]
        rec["roofline"]["exchange_floor_us"] = floor
        rec["roofline"]["latency_roof_us"] = round(cfg.L * 2 * floor, 1)
        rec["roofline"]["exchange_bound_us"] = round(cfg.L * (phases["h_exchange"] + phases["act_exchange"]), 1)
        rec["latency"] = {
            "phases_per_layer_us": phases, "exchange_probe": xprobe,
            "note": "exchange_floor_us: one dependent hand-off of a tagged word across XCDs (the probe's ring); "
                    "latency_roof_us = layers x 2 exchanges x that floor; exchange_bound_us = layers x (h + act "
                    "exchange as measured inside the kernel), the token time the two exchanges per layer take at "
                    "zero compute",
        }
    rec["repeats"] = {"tokens_per_s": [round(v, 2) for v in reps], "median": round(sorted(reps)[len(reps) // 2], 2),
                      "note": f"{len(reps)} runs of the same {args.steps} timed tokens; `value`, `ms_per_step` and the "
                              f"roofline's avg_us are those of the median run"}
    rec["routing_histogram"] = hist
    rec["expert_only"] = expert_only
    rec["per_layer_calls"] = {"tokens_per_s": per_layer_tok_s, "launches_per_token": launches,
                              "note": "same schedule issued as per-layer C-ABI calls in a HIP graph"}
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        rec["cpu_baseline"] = cpu_baseline(cfg, layers, syn, tokens=5 if cfg.d <= 2048 else 2)
        log("timing the CPU oracle on every core ...")
        rec["cpu_baseline_all_cores"] = cpu_baseline(cfg, layers, syn, tokens=1, streams=host_cores())
    return rec


def bench_tiny(args, cfg, torch, M, S, dev):
    """The small single-layer case (d 256, 16 experts): router + top-K, then the expert FFN with
    the fused weighted combine, four kernel launches per token, replayed as a graph.  Everything fits in
    cache, so this is a latency figure, not a bandwidth one."""
    from int4_expert_ffn_amd.chain import DecodeStack, LayerWeights
    syn = S.Synth(cfg)
    mats = S.fill_experts(syn, 0, dev)
    ex = M.Experts(mats["gate"], mats["up"], mats["down"], cfg.bits, cfg.group)
    stack = DecodeStack([LayerWeights(ex, syn.router(0, dev), None)], cfg.K, dev)
    tm = Timer(torch, dev, syn.hidden(7, 3 * 64, dev))
    graphs = tm.capture(lambda t, h: stack.token(t, h))
    wall, ev_ms, args.warmup = tm.timed(graphs, args.steps, args.warmup)
    total, _ = algorithmic_bytes(cfg)
    us = ev_ms * 1e3 / args.steps
    rec = base_record(args, cfg, args.steps / wall, wall, args.steps)
    rec["roofline"] = roofline("router + top-K + expert FFN with fused combine (4 launches per token)", total, us, None)
    rec["roofline"]["note"] = "the whole layer (132 KB) stays in cache: latency-bound, the fraction is not meaningful"
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        rec["cpu_baseline"] = cpu_baseline(cfg, stack.layers, syn, tokens=64)
    return rec


def bench_batched(args, cfg, torch, M, S, dev):
    """The batched layer (T tokens per call): router GEMM + top-K, routed experts as MFMA grouped
    GEMMs over the tokens sorted by expert, the shared expert with its unmerged LoRA, and the
    combine with the residual.  Four weight copies are rotated so that consecutive batches do
    not find the previous batch's weights in the memory-side cache."""
    T, K, d, E = cfg.T, cfg.K, cfg.d, cfg.E
    copies = []
    for c in range(4):
        syn = S.Synth(cfg, seed=c)
        mats = S.fill_experts(syn, 0, dev)
        se = syn.shared_expert_id()
        sh = M.Experts(*[syn.expert_mat(0, [se], m, dev) for m in S.MATS], cfg.bits, cfg.group)
        lw = syn.lora(0, dev)
        copies.append({"ex": M.Experts(mats["gate"], mats["up"], mats["down"], cfg.bits, cfg.group),
                       "sh": sh, "lora": M.Lora3([lw[m] for m in S.MATS], cfg.lora_alpha),
                       "router": syn.router(0, dev)})
    torch.cuda.synchronize()
    from int4_expert_ffn_amd.batched import BatchedLayer
    syn = S.Synth(cfg)
    n_in = 8
    hs = syn.hidden(11, n_in * T, dev).view(n_in, T, d)
    y = torch.empty((T, d), dtype=torch.float16, device=dev)
    for cp in copies:
        cp["layer"] = BatchedLayer(cp["ex"], cp["router"], T, K, dev, shared=cp["sh"], lora3=cp["lora"],
                                   two_streams=not args.one_stream, separate=args.separate_shared)

    def layer(cp, h):
        cp["layer"](h, y)

    # experts each (copy, input) pair touches, for the algorithmic bytes
    used = []
    for c, cp in enumerate(copies):
        for i in range(n_in):
            layer(cp, hs[i])
            used.append(int(torch.unique(cp["layer"].idx).numel()))
    torch.cuda.synchronize()
    stream = torch.cuda.Stream(device=dev)
    graphs = []
    with torch.cuda.stream(stream):
        for c, cp in enumerate(copies):
            for i in range(2):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    layer(cp, hs[(2 * c + i) % n_in])
                graphs.append(g)
    torch.cuda.synchronize()
    steps = args.steps
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        w0 = time.perf_counter()
        e0.record(stream)
        for i in range(steps):
            graphs[i % len(graphs)].replay()
        e1.record(stream)
        torch.cuda.synchronize()
        w1 = time.perf_counter()
    wall = w1 - w0
    us = e0.elapsed_time(e1) * 1e3 / steps
    assert torch.isfinite(y.float()).all(), "non-finite batched output"
    mean_used = sum(used) / len(used)
    eb = cfg.expert_bytes()
    lora_b = sum(2 * (r.numel() + b.numel()) for r, b in [syn.lora(0, "cpu")[m] for m in S.MATS])
    nbytes = int(round(mean_used * eb + eb + E * d * 2 + lora_b + 2 * T * d * 2))
    rec = base_record(args, cfg, steps * T / wall, wall, steps)
    sched = ("shared expert + LoRA as its own call, " + ("after the routed experts" if args.one_stream else
             "on a second stream")) if args.separate_shared else "shared expert + LoRA sorted in with the routed pairs"
    rec["roofline"] = roofline("the batched layer: router GEMM + top-K, sort, grouped MFMA gate/up and down, "
                               f"{sched}, combine (one graph per batch)", nbytes, us, None)
    rec["roofline"]["used_experts_mean"] = round(mean_used, 2)
    rec["batch_us"] = round(us, 2)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        rec["cpu_baseline"] = cpu_baseline_batched(cfg, S, tokens=32)
    return rec


def bench_relu_sparse(args, cfg, torch, M, S, dev):
    """The ReLU activation-sparse expert FFN through a resident 40-layer stack at batch 1: per layer
    one moe_expert_ffn_sparse call (gate/up with ReLU on the gate branch, then the down projection
    over the active neurons' neuron-major rows with the fused combine + residual), RMS-normalised
    layer inputs, routing given (top-K of seeded logits, drawn before the timed region).  The same
    schedule with the dense SwiGLU expert FFN (moe_expert_ffn_q4, row-major down) is timed beside it."""
    L, K, d, E, I = cfg.L, cfg.K, cfg.d, cfg.E, cfg.I
    syn = S.Synth(cfg)
    t0 = time.time()
    sparse, dense = [], []
    for l in range(L):
        mats = S.fill_experts(syn, l, dev, relu=True)
        sparse.append(M.Experts(mats["gate"], mats["up"], mats["down"], cfg.bits, cfg.group, neuron_major_down=True))
        dn = S.fill_experts(syn, l, dev)["down"]
        dense.append(M.Experts(mats["gate"], mats["up"], dn, cfg.bits, cfg.group))
    torch.cuda.synchronize()
    log(f"stacks resident: 2 x {L} layers, {torch.cuda.memory_allocated() / 2**30:.1f} GiB, {time.time() - t0:.1f} s")
    tm = Timer(torch, dev, syn.hidden(7, 3 * 64, dev))
    n_pool = tm.n_pool
    lg = syn.logits(9, n_pool * L, dev)
    idx_pool = torch.empty((n_pool, L, K), dtype=torch.int32, device=dev)
    w_pool = torch.empty((n_pool, L, K), dtype=torch.float32, device=dev)
    M.moe_route_topk(n_pool * L, d, E, K, M.MOE_TOPK_RENORM, None, None, lg, idx_pool.view(-1, K), w_pool.view(-1, K))
    ring_i = idx_pool[0:3].clone()
    ring_w = w_pool[0:3].clone()
    hs = torch.empty((L + 1, d), dtype=torch.float16, device=dev)
    n_act = torch.zeros((3, L, K), dtype=torch.int32, device=dev)
    ws = torch.empty(max(M.moe_expert_ffn_sparse_workspace_size(1, K, sparse[0]),
                         M.moe_expert_ffn_workspace_size(1, K, dense[0])), dtype=torch.uint8, device=dev)

    def token(t, h, layers, relu):
        s = t % 3
        hs[0].copy_(h.view(d))
        for l in range(L):
            x, y = hs[l].view(1, d), hs[l + 1].view(1, d)
            if relu:
                M.moe_expert_ffn_sparse(1, K, M.MOE_INPUT_RMSNORM, x, ring_i[s, l].view(1, K), layers[l], None,
                                        ring_w[s, l].view(1, K), x, y, n_act[s, l].view(1, K), ws)
            else:
                M.moe_expert_ffn_q4(1, K, M.MOE_INPUT_RMSNORM, x, ring_i[s, l].view(1, K), layers[l], None, None,
                                    ring_w[s, l].view(1, K), x, y, ws)

    def refill(p):
        ring_i.copy_(idx_pool[p:p + 3])
        ring_w.copy_(w_pool[p:p + 3])

    # active neurons of every pool token (inputs and routing fixed per token, so the timed pass reads the same rows)
    counts = []
    with torch.cuda.stream(tm.stream):
        for p in range(0, n_pool, 3):
            refill(p)
            for j in range(3):
                token(p + j + 3, tm.pool[p + j], sparse, True)     # slot (p + j) % 3 = j
                counts.append(n_act[(p + j) % 3].clone())
    torch.cuda.synchronize()
    cnt = torch.stack(counts).double()
    assert (cnt >= 0).all(), "an index outside [0, E) reached the sparse path"
    mean_active = float(cnt.mean())
    refill(0)

    res = {}
    for name, layers, relu in (("sparse", sparse, True), ("dense", dense, False)):
        graphs = tm.capture(lambda t, h: token(t, h, layers, relu))
        if args.eager:                           # same tokens, direct launches (graphs captured but unused)
            graphs = lambda t, layers=layers, relu=relu: token(t, tm.ring[t % 3], layers, relu)
        wall, ev_ms, warm = tm.timed(graphs, args.steps, args.warmup, refill)
        del graphs
        res[name] = (wall, ev_ms)
        assert torch.isfinite(hs[L].float()).all(), f"non-finite {name} output"
    args.warmup = warm
    row = d * cfg.bits // 8 + (d // cfg.group) * 4                  # one neuron-major down row
    gu = 2 * cfg.qmat_bytes("gate")
    vec = 3 * d * 2                                                 # x read, residual read, y written
    sparse_call = int(round(K * gu + K * mean_active * row + vec))
    dense_call = K * cfg.expert_bytes() + vec
    wall, ev_ms = res["sparse"]
    call_us = ev_ms * 1e3 / (args.steps * L)
    cfg_name = f"{cfg.name} shapes, ReLU activation-sparse experts (neuron-major down)"
    rec = base_record(args, cfg, args.steps / wall, wall, args.steps)
    rec["metric"] = "ReLU activation-sparse expert FFN decode tokens/s at batch 1 (40 layers) + achieved HBM GB/s"
    rec["config"]["workload"] = (f"{cfg_name}: d_model {d}, {E} experts, top-{K}, expert I {I}, int{cfg.bits} "
                                 f"affine g{cfg.group}, {L} layers resident, one moe_expert_ffn_sparse call per "
                                 f"layer, routing given, batch 1")
    rec["roofline"] = roofline("moe_expert_ffn_sparse per layer: k_gateup (ReLU) + k_down_sparse (+ fused combine)",
                               sparse_call, call_us, None)
    rec["roofline"]["bytes_note"] = (f"K dense gate/up matrices + the active neurons' down rows "
                                     f"({mean_active:.1f} of {I} per expert on average, measured) + the vectors")
    wall_d, ev_d = res["dense"]
    dense_us = ev_d * 1e3 / (args.steps * L)
    rec["active_fraction"] = round(mean_active / I, 4)
    rec["dense_swiglu_same_schedule"] = {
        "tokens_per_s": round(args.steps / wall_d, 2), "call_us": round(dense_us, 2),
        "bytes_per_call": dense_call, "achieved_GBps": round(dense_call / (dense_us * 1e-6) / 1e9, 1),
        "note": "moe_expert_ffn_q4 (SwiGLU, row-major down) on the same gate/up weights, inputs and routing"}
    rec["down_bytes_saved"] = round(1 - mean_active / I, 4)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        rec["cpu_baseline"] = cpu_baseline_relu(cfg, S, syn, tokens=5)
    return rec


def bench_stream(args, cfg, torch, M, S, dev):
    """Expert streaming (the pages' storage tier, here pinned host memory read over the host link):
    the 40-layer prerouted decode35b stack with every expert in host memory and an HBM pool of
    `--pool-slots` experts per layer.  Prefetch mode streams each layer's predicted experts for the
    next token on a copy stream as soon as the head of the layer before has predicted them; reactive
    mode streams each layer's experts in just before its expert FFN.  Each token is one HIP-graph
    replay; the resident stack's per-layer calls, replayed the same way, are timed for context."""
    from int4_expert_ffn_amd.chain import DecodeStack, LayerWeights
    from int4_expert_ffn_amd.stream import StreamedStack
    syn = S.Synth(cfg)
    t0 = time.time()
    routers = [syn.router(l, dev) for l in range(cfg.L + 1)]
    host_layers, dev_layers = [], []
    for l in range(cfg.L):
        mats = S.fill_experts(syn, l, dev)
        hmats = {m: tuple(torch.empty(a.shape, dtype=a.dtype, pin_memory=True).copy_(a) for a in arrs)
                 for m, arrs in mats.items()}
        head = None
        if l < cfg.L - 1:
            hw = syn.head(l, dev)
            hw["lin_x"] = routers[l + 1]
            head = M.PrerouterWeights(hw)
        dev_layers.append(LayerWeights(M.Experts(mats["gate"], mats["up"], mats["down"], cfg.bits, cfg.group),
                                       routers[l], head))
        host_layers.append(LayerWeights(M.Experts(hmats["gate"], hmats["up"], hmats["down"], cfg.bits, cfg.group,
                                                  host=True), routers[l], head))
    torch.cuda.synchronize()
    log(f"stack in pinned host memory and resident: {cfg.L} layers, {time.time() - t0:.1f} s")
    X = cfg.expert_bytes()
    tm = Timer(torch, dev, syn.hidden(7, 3 * 64, dev))

    # host link bandwidth of the pool copy: misses forced by resetting a pool before each call
    n_cal = 24
    pool = M.Pool(host_layers[1].experts, args.pool_slots, dev)
    cal_idx = (torch.arange((n_cal + 2) * cfg.K, dtype=torch.int32, device=dev) % cfg.E).view(n_cal + 2, cfg.K)
    cal_slot = torch.empty(cfg.K, dtype=torch.int32, device=dev)
    cal_ws = torch.empty(M.moe_stream_workspace_size(cfg.K), dtype=torch.uint8, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(tm.stream):
        for i in range(n_cal + 2):
            pool.reset()                     # every call copies all K experts
            if i == 2:
                e0.record(tm.stream)
            M.moe_stream_in(cfg.K, cal_idx[i], host_layers[1].experts, pool, cal_slot, None, cal_ws)
        e1.record(tm.stream)
    torch.cuda.synchronize()
    del pool
    cal_us = e0.elapsed_time(e1) * 1e3 / n_cal
    link_gbps = cfg.K * X / (cal_us * 1e-6) / 1e9
    log(f"pool copy: {cfg.K} experts in {cal_us:.1f} us = {link_gbps:.1f} GB/s")

    res = {}
    for mode in ("prefetch", "reactive"):
        stm = StreamedStack(host_layers, cfg.K, dev, n_slots=args.pool_slots, prefetch=(mode == "prefetch"),
                            fork_every=args.fork_every)
        run = tm.capture(lambda t, h, stm=stm: stm.token(t, h))
        # fill the pools first (about n_slots / misses-per-layer tokens), then count over the timed tokens
        n_fill = -(-max(args.warmup, 2 * args.pool_slots) // 3) * 3
        with torch.cuda.stream(tm.stream):
            tm.run(run, n_fill, 1)
        torch.cuda.synchronize()
        h_a, m_a = stm.hits_misses()
        wall, ev_ms, _ = tm.timed(run, args.steps, 0, start=1 + n_fill)
        del run
        h_b, m_b = stm.hits_misses()
        assert torch.isfinite(stm.h[cfg.L].float()).all(), f"non-finite {mode} output"
        res[mode] = dict(wall=wall, us=ev_ms * 1e3 / args.steps, hits=h_b - h_a, misses=m_b - m_a, tokens=args.steps)
    args.warmup = n_fill
    stack = DecodeStack(dev_layers, cfg.K, dev)
    graphs = tm.capture(lambda t, h: stack.token(t, h))
    n2 = max(30, args.steps // 4)
    wall_r, ev_r, _ = tm.timed(graphs, n2, 30)
    del graphs
    res_us = ev_r * 1e3 / n2

    p = res["prefetch"]
    miss_tok = p["misses"] / p["tokens"]
    hit_rate = p["hits"] / max(1, p["hits"] + p["misses"])
    bytes_tok = miss_tok * X
    # the pages' window model: in a window of w seconds the link brings floor(w * BW / X) experts;
    # the rest load after it ("Las matemáticas que importan")
    window_s = res_us * 1e-6
    n_window = math.floor(window_s * link_gbps * 1e9 / X)
    predicted_us = res_us + max(0.0, miss_tok - n_window) * X / (link_gbps * 1e9) * 1e6
    rec = base_record(args, cfg, args.steps / p["wall"], p["wall"], args.steps)
    rec["metric"] = "Streamed-expert decode tokens/s at batch 1 (experts in pinned host memory, HBM pool per layer)"
    rec["config"]["workload"] = (describe(cfg) + f"; every expert in pinned host memory, an HBM pool of "
                                 f"{args.pool_slots} experts per layer ({args.pool_slots * X * cfg.L / 2**30:.2f} GiB), "
                                 f"prerouter prefetch one token ahead on a copy stream")
    rec["roofline"] = {"kernel": "k_pool_copy (host memory -> HBM pool)", "bound": "host link",
                       "achieved": round(link_gbps, 1), "peak": 64.0, "unit": "GB/s",
                       "frac": round(link_gbps / 64.0, 4), "traffic": None, "bytes_per_launch": cfg.K * X,
                       "avg_us": round(cal_us, 2),
                       "note": "peak = PCIe 5.0 x16, one direction; the copy reads host memory over the host link"}
    rec["streaming"] = {
        "experts_streamed_per_token": round(miss_tok, 2), "hit_rate": round(hit_rate, 4),
        "bytes_streamed_per_token": int(round(bytes_tok)), "expert_bytes": X,
        "prefetch_us_per_token": round(p["us"], 1),
        "reactive_tokens_per_s": round(args.steps / res["reactive"]["wall"], 2),
        "reactive_us_per_token": round(res["reactive"]["us"], 1),
        "resident_per_layer_tokens_per_s": round(n2 / wall_r, 2), "resident_us_per_token": round(res_us, 1),
        "window_model": {"window_us": round(res_us, 1), "link_GBps": round(link_gbps, 1),
                         "experts_per_window": n_window, "experts_needed": round(miss_tok, 2),
                         "predicted_us_per_token": round(predicted_us, 1),
                         "hidden": bool(miss_tok <= n_window)},
        "note": "every path replays one HIP graph per token (the streamed ones on two streams, joined at the "
                "token's end); the resident per-layer path runs the same schedule with every expert in HBM",
    }
    if not args.no_cpu_baseline:   # streaming moves bytes and changes no result: the oracle is the resident chain's
        log("timing the CPU oracle ...")
        rec["cpu_baseline"] = cpu_baseline(cfg, dev_layers, syn, tokens=5)
    return rec


def cpu_baseline_relu(cfg, S, syn, tokens):
    """The fp64 oracle of the ReLU sparse expert FFN through all layers for `tokens` tokens (1 BLAS
    thread), with the same routing recipe; weights of the selected experts drawn beforehand."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(1)
    except Exception:  # pragma: no cover
        limiter = None
    L, K = cfg.L, cfg.K
    lg = syn.logits(9, tokens * L).numpy().reshape(tokens, L, cfg.E)
    route = [[O.route_topk(lg[t, l][None], K) for l in range(L)] for t in range(tokens)]
    packed = {}
    for t in range(tokens):
        for l in range(L):
            for e in route[t][l][0][0]:
                key = (l, int(e))
                if key not in packed:
                    packed[key] = [tuple(a[0].numpy() for a in syn.expert_mat(l, [int(e)], m))
                                   for m in ("gate", "up", "down_nm")]
    t0 = time.perf_counter()
    for t in range(tokens):
        h = O.f64(syn.hidden(7, 1)[0].numpy())
        for l in range(L):
            idx, w = route[t][l]
            x = O.rmsnorm(h)
            o = np.stack([O.expert_ffn_relu_packed(x, *packed[(l, int(e))], cfg.bits, cfg.group)[0] for e in idx[0]])
            h = O.to_f16_f64(O.combine(o, w[0], h))
    elapsed = time.perf_counter() - t0
    if limiter is not None:
        limiter.restore_original_limits()
    return {"value": round(tokens / elapsed, 5), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{tokens} token(s) through all {L} layers of the ReLU sparse expert FFN (fp64, explicit "
                      f"dequant, 1 BLAS thread; weights drawn beforehand)"}


def cpu_baseline_batched(cfg, S, tokens):
    """Time the fp64 oracle (single thread) on the first `tokens` tokens of a batch: router, top-K,
    the routed experts each token selects, the shared expert with its LoRA, combine.  The packed
    weights are drawn beforehand (untimed)."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(1)
    except Exception:  # pragma: no cover
        limiter = None
    syn = S.Synth(cfg)
    h = O.f64(syn.hidden(11, tokens).numpy())
    wr = syn.router(0).numpy()
    idx0, _ = O.route_topk(O.router_logits(wr, h), cfg.K)
    packed = {int(e): tuple(tuple(a[0].numpy() for a in syn.expert_mat(0, [int(e)], m)) for m in S.MATS)
              for e in np.unique(idx0)}
    se = syn.shared_expert_id()
    shared = tuple(tuple(a[0].numpy() for a in syn.expert_mat(0, [se], m)) for m in S.MATS)
    lw = syn.lora(0, "cpu")
    lora = {m: (lw[m][0].numpy(), lw[m][1].numpy()) for m in S.MATS}
    lora["alpha"] = cfg.lora_alpha
    t0 = time.perf_counter()
    idx, w = O.route_topk(O.router_logits(wr, h), cfg.K)
    o = np.zeros((tokens, cfg.K, cfg.d))
    for t in range(tokens):
        for k in range(cfg.K):
            o[t, k] = O.expert_ffn_packed(h[t], *packed[int(idx[t, k])], bits=cfg.bits, group=cfg.group)
    sh = O.expert_ffn_packed(h, *shared, cfg.bits, cfg.group, lora)
    O.combine(o, w, h, sh)
    elapsed = time.perf_counter() - t0
    if limiter is not None:
        limiter.restore_original_limits()
    return {"value": round(tokens / elapsed, 4), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"the first {tokens} tokens of a {cfg.T}-token batch (fp64, explicit dequant per expert "
                      f"and token, 1 BLAS thread; weights drawn beforehand)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=600)
    ap.add_argument("--warmup", type=int, default=60)
    ap.add_argument("--workload", choices=WORKLOADS, default="decode35b",
                    help="decode35b (default, the headline line), widek8, large-int4, large-int2 (resident stacks "
                         "through the persistent kernel), tiny (d 256, one layer), batched (256 tokens per call), "
                         "relu-sparse (decode35b shapes, ReLU activation-sparse experts, per-layer calls), "
                         "stream (decode35b with every expert in pinned host memory, HBM pools), exchange (the "
                         "exchange-latency probe's table)")
    ap.add_argument("--pool-slots", type=int, default=32, help="stream workload: HBM pool slots per layer")
    ap.add_argument("--separate-shared", action="store_true",
                    help="batched workload: the shared expert as its own call (on a second stream unless --one-stream)")
    ap.add_argument("--one-stream", action="store_true",
                    help="batched workload with --separate-shared: the shared expert on the main stream")
    ap.add_argument("--fork-every", type=int, default=8, help="stream workload: layers per prefetch fork")
    ap.add_argument("--no-cold", action="store_true", help="stack workloads: skip the cold-token timing")
    ap.add_argument("--no-histogram", action="store_true", help="stack workloads: skip the routing histogram")
    ap.add_argument("--repeats", type=int, default=5, help="stack workloads: runs of the timed loop (the first is value)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-layer", action="store_true", help="skip the per-layer-calls context timing")
    ap.add_argument("--no-expert-only", action="store_true", help="skip the expert-FFN-only timing")
    ap.add_argument("--no-phases", action="store_true",
                    help="stack workloads: skip the stamped phase breakdown and the exchange probe")
    ap.add_argument("--norm-gain", action="store_true",
                    help="stack workloads: every layer input normalised with a per-layer gain (x = g * h / rms(h))")
    ap.add_argument("--eager", action="store_true",
                    help="launch each timed token directly instead of replaying a HIP graph (for counter profiling)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (the reference for HBM byte counters)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: there is no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import int4_expert_ffn_amd as M
    import moe_synth as S

    dev = torch.device("cuda:0")
    if args.workload == "exchange":
        print(json.dumps(bench_exchange(args, torch, M, dev)), flush=True)
        return
    cfg = S.CONFIGS["decode35b" if args.workload in ("relu-sparse", "stream") else args.workload]
    if args.workload == "stream":
        rec = bench_stream(args, cfg, torch, M, S, dev)
    elif args.workload == "relu-sparse":
        rec = bench_relu_sparse(args, cfg, torch, M, S, dev)
    elif args.workload in STACK_WORKLOADS:
        rec = bench_stack(args, cfg, torch, M, S, dev)
    elif args.workload == "tiny":
        rec = bench_tiny(args, cfg, torch, M, S, dev)
    else:
        rec = bench_batched(args, cfg, torch, M, S, dev)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
