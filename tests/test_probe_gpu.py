"""The HBM read-ceiling probe (moe_read_probe) reads every byte it is given: the xor of the words
it writes, one per block, equals the xor of every 32-bit word of the buffer, computed on the host.
Sizes cover a ragged tail (not a multiple of one grid step) and a buffer smaller than one grid step."""
import numpy as np
import pytest
import torch

from parity_util import log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def M():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int4_expert_ffn_amd as m
    return m


@pytest.mark.parametrize("nbytes", [16, 4096 * 256 * 16 * 8 * 3 + 16 * 37, 1 << 20, 64 << 20])
def test_read_probe_folds_every_word(M, nbytes):
    log(f"read probe: {nbytes} bytes")
    rng = np.random.default_rng(nbytes % 1000003)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to(DEV)
    out = torch.full((M.MOE_READ_PROBE_BLOCKS,), -1, dtype=torch.int32, device=DEV)
    M.moe_read_probe(buf, out)
    torch.cuda.synchronize()
    folded = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert int(folded) == int(np.bitwise_xor.reduce(host))


def _xchg(M, **k):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    base = dict(pattern=M.MOE_XCHG_ALL, n_wg=cus, group_size=cus, xcd_local=0, words=1024, iters=50,
                load_scope=M.MOE_XCHG_SCOPE_DEVICE, store_scope=M.MOE_XCHG_SCOPE_DEVICE, epoch=1, replicas=1, wide_loads=0)
    base.update(k)
    cfg = M.moe_xchg_cfg(**base)
    ws = torch.zeros(M.moe_exchange_probe_workspace_size(cfg), dtype=torch.uint8, device=DEV)
    out = torch.zeros(1 + 3 * cfg.n_wg, dtype=torch.int32, device=DEV)
    log(f"exchange probe: {base}")
    M.moe_exchange_probe(cfg, ws, out)
    cfg.epoch = 2  # a second call on the same workspace
    M.moe_exchange_probe(cfg, ws, out)
    torch.cuda.synchronize()
    o = out.cpu().numpy().view(np.uint32).astype(np.int64)
    ticks = o[1::3] | (o[2::3] << 32)
    return cfg, int(o[0]), ticks, o[3::3]


@pytest.mark.parametrize("pattern", ["all", "ring"])
def test_exchange_probe_device_scope_completes(M, pattern):
    """Device-coherent hand-offs across every compute unit complete with no wait running out, in
    a time that is a plausible handful of microseconds per phase; every XCD reports itself."""
    if pattern == "all":
        cfg, err, ticks, xcc = _xchg(M)
        per_phase_us = ticks.max() / 100.0 / cfg.iters
    else:
        cfg, err, ticks, xcc = _xchg(M, pattern=M.MOE_XCHG_RING, group_size=16, iters=20)
        per_phase_us = ticks[::cfg.n_wg // cfg.group_size].max() / 100.0 / (cfg.iters * cfg.group_size)
    assert err == 0
    assert 0.05 < per_phase_us < 100.0, per_phase_us
    assert set(np.unique(xcc).tolist()) <= set(range(8))


def test_exchange_probe_xcd_groups(M):
    """Groups formed as b % (n_wg / group_size) run on one XCD each (the round-robin dealing of
    workgroups over the XCDs), and device-scope exchanges inside them complete."""
    cfg, err, ticks, xcc = _xchg(M, group_size=32, xcd_local=1, words=256)
    ng = cfg.n_wg // cfg.group_size
    groups = [set(xcc[g::ng].tolist()) for g in range(ng)]
    assert all(len(s) == 1 for s in groups), groups
    assert len(set().union(*groups)) == min(8, ng)
    assert err == 0
