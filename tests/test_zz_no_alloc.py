"""GPU: moe_expert_ffn_q4_noalloc (the expert FFN on the library's own scratch, for callers that
cannot allocate) against moe_expert_ffn_q4 with a caller workspace, through the C ABI.  Two calls
in a row on one GPU, the second with a smaller input, each equal to the workspace entry point's
result; the same kernels run on the same inputs, so the outputs are compared bit for bit."""
import numpy as np
import pytest
import torch

import moe_synth as S
from parity_util import device_layer, log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def M():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int4_expert_ffn_amd as m
    return m


def _inputs(syn, cfg, T, seed):
    h = syn.hidden(seed, T).to(DEV)
    rng = np.random.default_rng(seed)
    idx = torch.tensor(np.array([rng.choice(cfg.E, cfg.K, replace=False) for _ in range(T)]), dtype=torch.int32,
                       device=DEV)
    w = torch.softmax(torch.tensor(rng.normal(size=(T, cfg.K)), dtype=torch.float32), -1).to(DEV)
    return h, idx, w


def _both(M, ex, cfg, T, h, idx, w):
    """(out, y) of the workspace entry point and of the allocation-free one."""
    K, d = cfg.K, cfg.d
    ws = torch.empty(M.moe_expert_ffn_workspace_size(T, K, ex), dtype=torch.uint8, device=DEV)
    o1 = torch.full((T, K, d), float("nan"), device=DEV)
    y1 = torch.empty((T, d), dtype=torch.float16, device=DEV)
    M.moe_expert_ffn_q4(T, K, M.MOE_INPUT_RMSNORM, h, idx, ex, None, o1, w, h, y1, ws)
    o2 = torch.full((T, K, d), float("nan"), device=DEV)
    y2 = torch.empty((T, d), dtype=torch.float16, device=DEV)
    M.moe_expert_ffn_q4_noalloc(T, K, M.MOE_INPUT_RMSNORM, h, idx, ex, None, o2, w, h, y2)
    torch.cuda.synchronize()
    return (o1, y1), (o2, y2)


@pytest.mark.parametrize("name,T1,T2", [("decode35b", 48, 3), ("decode35b", 4, 1), ("large-int2", 2, 1)])
def test_noalloc_equals_workspace_entry(M, name, T1, T2):
    cfg = S.CONFIGS[name]
    syn = S.Synth(cfg)
    ex = device_layer(syn, 0, DEV)
    for T, seed in ((T1, 900), (T2, 901)):   # the second call is smaller and reuses the scratch
        log(f"no-alloc expert FFN: {name} T={T}")
        h, idx, w = _inputs(syn, cfg, T, seed)
        (o1, y1), (o2, y2) = _both(M, ex, cfg, T, h, idx, w)
        assert torch.isfinite(o1).all() and torch.isfinite(y1.float()).all()
        assert torch.equal(o1, o2), f"T={T}: per-expert outputs differ"
        assert torch.equal(y1, y2), f"T={T}: fused combine differs"


def test_noalloc_rejects_oversize_without_enqueueing(M):
    cfg = S.CONFIGS["decode35b"]
    syn = S.Synth(cfg)
    ex = device_layer(syn, 0, DEV)
    T = 1024          # the grouped path's scratch at this size exceeds MOE_NOALLOC_SCRATCH_BYTES
    assert M.moe_expert_ffn_workspace_size(T, cfg.K, ex) > M.MOE_NOALLOC_SCRATCH_BYTES
    h = torch.zeros((T, cfg.d), dtype=torch.float16, device=DEV)
    idx = torch.zeros((T, cfg.K), dtype=torch.int32, device=DEV)
    out = torch.zeros((T, cfg.K, cfg.d), device=DEV)
    with pytest.raises(M.MoEError) as e:
        M.moe_expert_ffn_q4_noalloc(T, cfg.K, 0, h, idx, ex, None, out, None, None, None)
    assert e.value.status == M.MOE_ERR_TOO_LARGE
    torch.cuda.synchronize()
    assert bool((out == 0).all())
