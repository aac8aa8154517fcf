"""Reader for the small text fixtures under tests/golden/."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_fixture(name):
    """key -> list of tokens, for 'key v1 v2 ...' lines; '#' lines are comments."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, *v = line.split()
            out.setdefault(k, []).append(v)
    return out


def hand_chain():
    """The hand-worked prerouted chain (prerouted_chain_hand.txt) as plain numpy arrays.

    Returns a dict: shapes (d, E, K, I, bits, group, L, H), heads (layers carrying one),
    router [L][E][d] float16, lin_r {l: [2E][E] float16}, h [T][d] float16, and the expected
    values keyed by (t, l): route -> (source, idx, w), router_num -> [E], head_in -> (cur, prev or
    None), head_logits -> [E], pred (keyed by (t, l+1)) -> (idx, w)."""
    import numpy as np

    fx = read_fixture("prerouted_chain_hand.txt")
    one = {k: int(fx[k][0][0]) for k in ("d", "E", "K", "d_ff", "bits", "group", "L", "H")}
    d, E, L = one["d"], one["E"], one["L"]
    out = dict(one)
    out["heads"] = [int(v) for v in fx["heads"][0]]
    router = np.zeros((L, E, d), dtype=np.float16)
    for l, e, j, v in fx["router"]:
        router[int(l), int(e), int(j)] = float(v)
    lin_r = {l: np.zeros((2 * E, E), dtype=np.float16) for l in out["heads"]}
    for l, row, e, v in fx["lin_r"]:
        lin_r[int(l)][int(row), int(e)] = float(v)
    hs = sorted(fx["h"], key=lambda r: int(r[0]))
    h = np.zeros((len(hs), d), dtype=np.float16)
    for t, *v in hs:
        h[int(t), : len(v)] = [float(x) for x in v]
    out.update(router=router, lin_r=lin_r, h=h)
    out["route"] = {(int(t), int(l)): (src, [int(a), int(b)], [float(c), float(e)])
                    for t, l, src, a, b, c, e in fx["route"]}
    out["router_num"] = {(int(t), int(l)): [float(x) for x in v] for t, l, *v in fx["router_num"]}
    out["head_in"] = {(int(t), int(l)): ([int(v[0]), int(v[1])], None if v[2] == "none" else [int(v[2]), int(v[3])])
                      for t, l, *v in fx["head_in"]}
    out["head_logits"] = {(int(t), int(l)): [float(x) for x in v] for t, l, *v in fx["head_logits"]}
    out["pred"] = {(int(t), int(l)): ([int(a), int(b)], [float(c), float(e)]) for t, l, a, b, c, e in fx["pred"]}
    return out
