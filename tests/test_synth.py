"""The seeded input generator: SplitMix64 against its big-integer definition, slice
independence, and the value distributions of the workloads."""
import math

import numpy as np
import torch

import moe_synth as S


def test_hash_block_matches_python_definition():
    for key in (0, 1, S.stream_key(0, 1, 2, 3, 4), (1 << 64) - 1):
        h = S.hash_block([key], 5, 40).view(-1)
        for i in range(40):
            assert int(h[i].item()) & S.MASK64 == S.splitmix64_py(key, 5 + i)


def test_splitmix64_reference_values():
    # SplitMix64 with state 0: the first output is mix64(GAMMA)
    assert S.splitmix64_py(0, 0) == 0xE220A8397B1DCDAF
    assert S.splitmix64_py(0, 1) == 0x6E789E6AA1B965F4


def test_slices_are_independent_of_batching():
    syn = S.Synth(S.CONFIGS["tiny"])
    q_all, s_all, b_all = syn.expert_mat(0, list(range(16)), "down")
    q5, s5, b5 = syn.expert_mat(0, [5], "down")
    assert torch.equal(q_all[5], q5[0]) and torch.equal(s_all[5], s5[0]) and torch.equal(b_all[5], b5[0])
    assert not torch.equal(q_all[4], q_all[5])


def test_expert_value_recipe():
    for name in ("decode35b", "large-int2"):
        cfg = S.CONFIGS[name]
        q, s, b = S.Synth(cfg).expert_mat(1, [0, 3], "gate")
        sf = s.double()
        assert sf.min() >= 0.005 - 1e-5 and sf.max() <= 0.02 + 1e-5
        noise = b.double() + (1 << (cfg.bits - 1)) * sf
        assert abs(noise.mean().item()) < 2e-4 and 0.7e-3 < noise.std().item() < 1.3e-3
        codes = ((q.view(-1).numpy().view(np.uint32)[:, None] >> np.arange(0, 32, cfg.bits)) & ((1 << cfg.bits) - 1))
        counts = np.bincount(codes.reshape(-1), minlength=1 << cfg.bits)
        assert counts.min() / counts.max() > 0.97


def test_normal_moments():
    z = S.normal_f16([S.stream_key(0, 9, 9, 9, 9)], 200_000, 1.0).double()
    assert abs(z.mean().item()) < 0.01 and abs(z.std().item() - 1) < 0.01
    assert z.abs().max().item() <= 6.0


def test_router_scale_and_orthonormal_rows():
    cfg = S.CONFIGS["decode35b"]
    w = S.Synth(cfg).router(0).double()
    assert abs(w.std().item() * math.sqrt(cfg.d) - 1) < 0.02
    w2 = S.Synth(S.CONFIGS["widek8"]).router(3).double()
    gram = w2 @ w2.t()
    assert torch.allclose(gram, torch.eye(gram.shape[0], dtype=torch.float64), atol=5e-3)
    # and orthogonal to the all-ones direction (up to the float16 rounding of the rows)
    assert (w2.sum(dim=1).abs() / math.sqrt(w2.shape[1])).max().item() < 2e-3


def test_head_uses_next_router_for_linear_path():
    syn = S.Synth(S.CONFIGS["decode35b"])
    hd = syn.head(4)
    assert torch.equal(hd["lin_x"], syn.router(5))
    assert hd["fc1_r"].shape == (2 * 256, 1024) and hd["lin_r"].shape == (512, 256)
