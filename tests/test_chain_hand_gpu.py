"""GPU: the per-layer decode schedule on the hand-worked prerouted stack (prerouted_chain_hand.txt).

The expected routing is the fixture's, worked by hand from the pages' statement of the head (page
"La otra mitad del muro de la memoria ...", sections "Arquitectura del cabezal Prerouter" and
"Ideas clave"), not the oracle's: which layers route themselves, which take the previous token's
prediction, the two K-hot inputs of each head and where its prediction lands.  Every logit here is
an exact sum of small integers (heads) or h / rms(h) with integer h (routers), so indices are
compared exactly and weights to float32 rounding."""
import numpy as np
import pytest
import torch

import golden_io

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def M():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int4_expert_ffn_amd as m
    return m


def test_prerouted_chain_hand_worked_per_layer_path(M):
    from int4_expert_ffn_amd.chain import DecodeStack, LayerWeights

    fx = golden_io.hand_chain()
    d, E, K, I, H, L, g = fx["d"], fx["E"], fx["K"], fx["d_ff"], fx["H"], fx["L"], fx["group"]
    words = lambda cols: cols * fx["bits"] // 32
    z = lambda *s: torch.zeros(s, dtype=torch.float16, device=DEV)
    zq = lambda *s: torch.zeros(s, dtype=torch.int32, device=DEV)
    gu = (zq(E, I, words(d)), z(E, I, d // g), z(E, I, d // g))
    dn = (zq(E, d, words(I)), z(E, d, I // g), z(E, d, I // g))
    ex = M.Experts(gu, gu, dn, fx["bits"], g)
    layers = []
    for l in range(L):
        head = None
        if l in fx["heads"]:
            head = M.PrerouterWeights({"fc1_x": z(H, d), "fc1_r": z(2 * E, H), "fc2": z(E, H), "lin_x": z(E, d),
                                       "lin_r": torch.from_numpy(fx["lin_r"][l]).to(DEV)})
        layers.append(LayerWeights(ex, torch.from_numpy(fx["router"][l]).to(DEV), head))
    stack = DecodeStack(layers, K, DEV)
    for t in range(fx["h"].shape[0]):
        h = torch.from_numpy(fx["h"][t]).to(DEV)
        print(f"hand chain: token {t}", flush=True)
        out = stack.token(t, h)
        torch.cuda.synchronize()
        idx = stack.route_idx[t % 3].cpu().numpy()
        w = stack.route_w[t % 3].cpu().numpy()
        nxt_i = stack.route_idx[(t + 1) % 3].cpu().numpy()
        nxt_w = stack.route_w[(t + 1) % 3].cpu().numpy()
        hlog = stack.head_logits.cpu().numpy()
        for l in range(L):
            _, e_ref, w_ref = fx["route"][(t, l)]
            assert idx[l].tolist() == e_ref, (t, l, idx[l])
            np.testing.assert_allclose(w[l], w_ref, rtol=0, atol=1e-6)
            if l in fx["heads"]:
                np.testing.assert_array_equal(hlog[l], np.array(fx["head_logits"][(t, l)], dtype=np.float32))
                p_ref, pw_ref = fx["pred"][(t, l + 1)]
                assert nxt_i[l + 1].tolist() == p_ref, (t, l, nxt_i[l + 1])
                np.testing.assert_allclose(nxt_w[l + 1], pw_ref, rtol=0, atol=1e-6)
        # the experts output zero: every layer passes its input through unchanged
        assert torch.equal(out, h) and torch.equal(stack.h[1:L + 1], h.expand(L, d))
