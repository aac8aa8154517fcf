"""C-ABI checks that need no GPU: the library loads, exports every function include/moe.h declares,
and rejects bad arguments on the host before anything is enqueued (so no call here reaches the
HIP runtime)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

lib_mod = pytest.importorskip("int4_expert_ffn_amd._lib", reason="libmoe.so not built")
torch = pytest.importorskip("torch")
if torch.cuda.device_count() > 0:   # the fake addresses below must never reach a real device
    pytest.skip("host-only argument checks; skipped where a GPU is visible", allow_module_level=True)
L = lib_mod._lib
OK, INVALID, UNSUP = 0, 1, 2

FAKE = 0x7F0000000000   # 16-byte aligned, never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_function():
    names = declared_functions()
    assert len(names) == 26
    assert sorted(lib_mod.EXPORTS) == names
    for n in names:
        assert hasattr(L, n)
    assert L.moe_version() == 100
    for s in (0, 1, 2, 3, 4):
        assert L.moe_status_string(s).startswith(b"MOE_")


def _ex(E=16, d=256, I=128, bits=4, group=32, q=FAKE):
    m = lambda: lib_mod.moe_qmat(q, FAKE, FAKE)
    return lib_mod.moe_experts(E, d, I, bits, group, m(), m(), m())


def _ffn(ex, T=1, K=2, flags=0, x=FAKE, idx=FAKE, lora=None, out=FAKE, wf=None, rf=None, yf=None,
         ws=FAKE, wsb=1 << 40):
    st = L.moe_expert_ffn_q4(None, T, K, flags, x, idx, ctypes.byref(ex), lora, out, wf, rf, yf, ws, wsb)
    assert st in (INVALID, UNSUP), "a call with fake pointers must never pass validation"
    return st


def test_route_topk_rejects():
    r = lambda *a: L.moe_route_topk(None, *a)
    assert r(0, 256, 16, 2, 0, FAKE, FAKE, FAKE, FAKE, FAKE) == INVALID       # T < 1
    assert r(1, 256, 16, 17, 0, FAKE, FAKE, FAKE, FAKE, FAKE) == INVALID      # K > E
    assert r(1, 256, 64, 17, 0, FAKE, FAKE, FAKE, FAKE, FAKE) == INVALID      # K > 16
    assert r(1, 256, 1025, 2, 0, FAKE, FAKE, FAKE, FAKE, FAKE) == INVALID     # E > 1024
    assert r(1, 256, 16, 2, 0, FAKE, FAKE, FAKE, None, FAKE) == INVALID       # idx NULL
    assert r(1, 256, 16, 2, 0x8, FAKE, FAKE, FAKE, FAKE, FAKE) == INVALID     # unknown flag
    assert r(1, 250, 16, 2, 0, FAKE, FAKE, FAKE, FAKE, FAKE) == INVALID       # d % 8
    assert r(1, 16384, 16, 2, 0, FAKE, FAKE, FAKE, FAKE, FAKE) == INVALID     # d > 8192
    assert r(1, 256, 16, 2, 0, FAKE + 2, FAKE, FAKE, FAKE, FAKE) == INVALID   # misaligned x
    assert r(1, 256, 16, 2, 0, None, FAKE, FAKE, FAKE, FAKE) == INVALID       # router without x


def test_expert_ffn_rejects():
    assert _ffn(_ex(bits=3)) == UNSUP
    assert _ffn(_ex(bits=8)) == UNSUP
    assert _ffn(_ex(group=16)) == UNSUP
    assert _ffn(_ex(group=256)) == UNSUP
    assert _ffn(_ex(d=240)) == INVALID                        # d % group
    assert _ffn(_ex(d=16384, group=64)) == INVALID            # d > 8192
    assert _ffn(_ex(bits=2, d=288, group=32)) == INVALID      # 2-bit row not whole 16-byte segments
    assert _ffn(_ex(q=FAKE + 4)) == INVALID                   # misaligned q
    assert _ffn(_ex(E=0)) == INVALID
    assert _ffn(_ex(E=2), K=3) == INVALID                     # K > E
    assert _ffn(_ex(), T=0) == INVALID
    assert _ffn(_ex(), x=None) == INVALID
    assert _ffn(_ex(), out=None) == INVALID                   # no output at all
    assert _ffn(_ex(), out=None, wf=FAKE, rf=FAKE) == INVALID  # partial fuse triple
    assert _ffn(_ex(), wsb=16) == INVALID                     # workspace too small
    assert _ffn(_ex(), ws=FAKE + 8) == INVALID                # misaligned workspace
    lora = (lib_mod.moe_lora * 3)(*[lib_mod.moe_lora(FAKE, FAKE, 16, 32.0)] * 3)
    assert _ffn(_ex(E=16), lora=lora) == INVALID              # LoRA only on a single shared expert
    bad_rank = (lib_mod.moe_lora * 3)(*[lib_mod.moe_lora(FAKE, FAKE, 65, 32.0)] * 3)
    assert _ffn(_ex(E=1), K=1, lora=bad_rank) == INVALID


def test_sparse_ffn_rejects():
    def sp(ex, T=1, K=2, flags=0, x=FAKE, out=FAKE, wf=None, rf=None, yf=None, n=None, ws=FAKE, wsb=1 << 40):
        st = L.moe_expert_ffn_sparse(None, T, K, flags, x, FAKE, ctypes.byref(ex), out, wf, rf, yf, n, ws, wsb)
        assert st in (INVALID, UNSUP), "a call with fake pointers must never pass validation"
        return st

    assert sp(_ex(bits=3)) == UNSUP
    assert sp(_ex(d=288, group=32)) == UNSUP                 # d not a multiple of the 64-column slab
    assert sp(_ex(bits=2, d=320, I=128, group=64)) == UNSUP    # d not a multiple of the 128-column 2-bit slab
    assert sp(_ex(d=240, group=32)) == INVALID                # d not a multiple of the group
    assert sp(_ex(d=256, I=8192, group=64)) == UNSUP          # d_ff above 4096
    assert sp(_ex(), flags=1) == INVALID                      # only MOE_INPUT_RMSNORM
    assert sp(_ex(), T=0) == INVALID
    assert sp(_ex(), x=None) == INVALID
    assert sp(_ex(), out=None) == INVALID                     # no output at all
    assert sp(_ex(), wf=FAKE) == INVALID                      # partial fuse triple
    assert sp(_ex(), wsb=16) == INVALID                       # workspace too small
    assert sp(_ex(), ws=FAKE + 8) == INVALID
    ex = _ex(E=256, d=2048, I=512, group=64)
    al = lambda v: (v + 255) // 256 * 256
    want = al(4 * 512 * 4) + al(4 * 2048 * 4) + al(32 * 4)
    assert L.moe_expert_ffn_sparse_workspace_size(1, 4, ctypes.byref(ex)) == want


def test_stream_in_rejects():
    src = _ex(E=256, d=2048, I=512, group=64)
    pool_ex = _ex(E=8, d=2048, I=512, group=64)
    pool = lib_mod.moe_pool(8, FAKE, FAKE, FAKE)
    ws = L.moe_stream_workspace_size(4)
    assert ws == 256 and L.moe_stream_workspace_size(0) == 0 and L.moe_stream_workspace_size(17) == 0

    def si(K=4, src=src, pex=pool_ex, pool=pool, idx=FAKE, out=FAKE, w=FAKE, wsb=ws):
        st = L.moe_stream_in(None, K, idx, ctypes.byref(src), ctypes.byref(pex), ctypes.byref(pool), out,
                             None, w, wsb)
        assert st in (INVALID, UNSUP), "a call with fake pointers must never pass validation"
        return st

    assert si(K=0) == INVALID
    assert si(K=17) == INVALID
    assert si(pool=lib_mod.moe_pool(8, FAKE, FAKE, None)) == INVALID    # no clock
    assert si(idx=None) == INVALID
    assert si(out=None) == INVALID
    assert si(w=None) == INVALID
    assert si(wsb=8) == INVALID                                     # workspace too small
    assert si(w=FAKE + 8) == INVALID                                # misaligned workspace
    assert si(K=9) == INVALID                                       # K above n_slots
    assert si(pool=lib_mod.moe_pool(4097, FAKE, FAKE, FAKE)) == INVALID   # above MOE_POOL_MAX_SLOTS
    assert si(pool=lib_mod.moe_pool(8, None, FAKE, FAKE)) == INVALID
    assert si(pex=_ex(E=9, d=2048, I=512, group=64)) == INVALID     # pool descriptor of another size
    assert si(pex=_ex(E=8, d=2048, I=512, group=32)) == INVALID     # shapes differ
    assert si(src=_ex(E=256, d=2048, I=512, group=64, q=FAKE + 4), pex=pool_ex) == INVALID  # misaligned codes
    assert si(src=_ex(E=256, d=2048, I=512, bits=3, group=64), pex=_ex(E=8, d=2048, I=512, bits=3, group=64)) == UNSUP


def test_stream_in_many_rejects():
    src = _ex(E=256, d=2048, I=512, group=64)
    pex = _ex(E=8, d=2048, I=512, group=64)
    pools = [lib_mod.moe_pool(8, FAKE + 256 * i, FAKE, FAKE) for i in range(10)]
    J = lib_mod.moe_stream_job

    def jobs(n, same_pool=False, other=None):
        arr = (J * max(1, n))()
        for i in range(n):
            s = other if (other is not None and i == n - 1) else src
            arr[i] = J(FAKE, ctypes.pointer(s), ctypes.pointer(pex), ctypes.pointer(pools[0 if same_pool else i]),
                       FAKE, None)
        return arr

    def many(n, arr, wsb=1 << 20, ws=FAKE):
        st = L.moe_stream_in_many(None, n, 4, arr, ws, wsb)
        assert st in (INVALID, UNSUP), "a call with fake pointers must never pass validation"
        return st

    assert many(0, jobs(1)) == INVALID
    assert many(9, jobs(9)) == INVALID                          # above MOE_POOL_MAX_JOBS
    assert many(3, jobs(3), wsb=512) == INVALID                 # workspace for 2 jobs only
    assert many(2, jobs(2, same_pool=True)) == INVALID          # one pool twice
    other = _ex(E=256, d=2048, I=1024, group=64)
    assert many(2, jobs(2, other=other)) == INVALID             # jobs of different shapes
    assert L.moe_stream_in_many(None, 1, 4, None, FAKE, 1 << 20) == INVALID


def test_read_probe_rejects():
    assert L.moe_read_probe(None, None, 1024, FAKE) == INVALID
    assert L.moe_read_probe(None, FAKE, 1024, None) == INVALID
    assert L.moe_read_probe(None, FAKE, 1000, FAKE) == INVALID     # not whole 16-byte units
    assert L.moe_read_probe(None, FAKE + 8, 1024, FAKE) == INVALID  # misaligned


def test_prerouter_and_combine_reject():
    pw = lib_mod.moe_prerouter_w(1024, FAKE, FAKE, None, FAKE, None, FAKE, FAKE, None)
    p = lambda *a, **k: L.moe_prerouter(None, *a)
    assert p(1, 2048, 256, 4, 0, FAKE, FAKE, None, ctypes.byref(pw), FAKE, FAKE, 16) == INVALID   # workspace
    assert p(1, 2048, 256, 4, 0, FAKE, None, None, ctypes.byref(pw), FAKE, FAKE, 1 << 30) == INVALID  # idx_cur
    pw0 = lib_mod.moe_prerouter_w(1020, FAKE, FAKE, None, FAKE, None, FAKE, FAKE, None)
    assert p(1, 2048, 256, 4, 0, FAKE, FAKE, None, ctypes.byref(pw0), FAKE, FAKE, 1 << 30) == INVALID  # H % 8
    pw1 = lib_mod.moe_prerouter_w(1024, FAKE, None, None, FAKE, None, FAKE, FAKE, None)
    assert p(1, 2048, 256, 4, 0, FAKE, FAKE, None, ctypes.byref(pw1), FAKE, FAKE, 1 << 30) == INVALID  # fc1_r
    so = lambda *a: L.moe_sort_by_expert(None, *a)
    assert so(0, 4, 256, FAKE, FAKE, FAKE, FAKE) == INVALID
    assert so(1, 4, 2000, FAKE, FAKE, FAKE, FAKE) == INVALID
    assert so(1 << 22, 16, 256, FAKE, FAKE, FAKE, FAKE) == INVALID
    assert so(4, 4, 256, FAKE, None, FAKE, FAKE) == INVALID
    st = lib_mod.moe_decode_stack(40, 256, 4, 2048, 512, 4, 64, 1024, FAKE, FAKE, FAKE)
    ds = lambda stk, tok=1, flags=1, ws=FAKE, wsb=1 << 40, hl=None: L.moe_decode_step(
        None, ctypes.byref(stk), tok, flags, FAKE, FAKE, hl, ws, wsb)
    assert ds(st, tok=-1) == INVALID
    assert ds(st, flags=2) == INVALID
    assert ds(st, flags=8) == INVALID           # unknown flag bit
    assert ds(st, flags=5, wsb=64) == INVALID   # given routing passes the flag check, the size check still applies
    assert ds(st, wsb=64) == INVALID
    assert ds(st, ws=FAKE + 16) == INVALID
    assert ds(st, hl=FAKE + 2) == INVALID      # per-layer copies must be 4-byte aligned
    bad = lib_mod.moe_decode_stack(40, 256, 9, 2048, 512, 4, 64, 1024, FAKE, FAKE, FAKE)
    assert ds(bad) == UNSUP                     # K > 8 is not a persistent-kernel shape
    tiny = lib_mod.moe_decode_stack(1, 16, 2, 256, 128, 4, 32, 0, FAKE, FAKE, FAKE)
    assert ds(tiny) == UNSUP                    # d_model 256: per-layer calls only
    nolayers = lib_mod.moe_decode_stack(40, 256, 4, 2048, 512, 4, 64, 1024, None, FAKE, FAKE)
    assert ds(nolayers) == INVALID
    assert L.moe_decode_workspace_size(ctypes.byref(st)) > 40 * 1024 * 8
    g2 = lib_mod.moe_decode_stack(40, 256, 4, 2048, 512, 4, 64, 1024, FAKE, FAKE, FAKE, 2)
    assert ds(g2) == INVALID                    # norm_gains is 0 or 1
    n = lambda *a: L.moe_rmsnorm(None, *a)
    assert n(0, 2048, FAKE, None, FAKE) == INVALID          # T < 1
    assert n(1, 2044, FAKE, None, FAKE) == INVALID          # d % 8
    assert n(1, 16384, FAKE, None, FAKE) == INVALID         # d > MOE_MAX_D
    assert n(1, 2048, None, None, FAKE) == INVALID          # h NULL
    assert n(1, 2048, FAKE + 8, None, FAKE) == INVALID      # h not 16-byte aligned
    assert n(1, 2048, FAKE, FAKE + 2, FAKE) == INVALID      # gain not 16-byte aligned
    c = lambda *a: L.moe_combine(None, *a)
    assert c(0, 4, 2048, FAKE, FAKE, FAKE, None, FAKE) == INVALID
    assert c(1, 17, 2048, FAKE, FAKE, FAKE, None, FAKE) == INVALID
    assert c(1, 4, 2048, None, FAKE, FAKE, None, FAKE) == INVALID
    assert c(1, 4, 2048, FAKE, FAKE, FAKE, None, None) == INVALID


def test_decode_step_grid_for_other_cu_counts():
    """The persistent kernel's plan on devices with other compute-unit counts (host-only): the four
    stacks it is built for take one workgroup per compute unit on a 256-CU device; elsewhere a plan
    is either refused (0: the call returns MOE_ERR_UNSUPPORTED there) or uses at most one workgroup
    per compute unit, so a plan that passes never needs more workgroups than can be resident."""
    gf = lambda stk, n: L.moe_decode_step_grid_for(ctypes.byref(stk), n)
    shapes = {  # L, E, K, d_model, d_ff, bits, group, d_hidden
        "decode35b": (40, 256, 4, 2048, 512, 4, 64, 1024),
        "widek8": (24, 256, 8, 2048, 512, 4, 64, 0),
        "large-int4": (15, 512, 4, 4096, 1024, 4, 64, 0),
        "large-int2": (15, 512, 4, 4096, 1024, 2, 64, 0),
    }
    for name, shp in shapes.items():
        st = lib_mod.moe_decode_stack(*shp, FAKE, FAKE, FAKE)
        assert gf(st, 256) == 256, name
        assert gf(st, 0) == 0 and gf(st, -8) == 0
        for n in (1, 8, 64, 80, 104, 120, 128, 160, 200, 228, 240, 255, 257, 304, 512, 1024, 4096, 1 << 20):
            g = gf(st, n)
            assert g == 0 or 1 <= g <= min(n, 1024), (name, n, g)
        # no device here: the current-device query and the call itself both refuse the stack
        assert L.moe_decode_step_grid(ctypes.byref(st)) == 0
        assert L.moe_decode_step(None, ctypes.byref(st), 1, 1, FAKE, FAKE, None, FAKE, 1 << 40) == UNSUP
    assert L.moe_decode_step_grid_for(None, 256) == 0
    tiny = lib_mod.moe_decode_stack(1, 16, 2, 256, 128, 4, 32, 0, FAKE, FAKE, FAKE)
    assert gf(tiny, 256) == 0                   # d_model 256: per-layer calls only
    bad = lib_mod.moe_decode_stack(40, 256, 9, 2048, 512, 4, 64, 1024, FAKE, FAKE, FAKE)
    assert gf(bad, 256) == 0                    # K > 8


def test_expert_ffn_shared_rejects():
    ex = _ex(E=256, d=2048, I=512, group=64)
    sh = _ex(E=1, d=2048, I=512, group=64)
    ws_need = L.moe_expert_ffn_shared_workspace_size(256, 4, ctypes.byref(ex))
    assert ws_need > L.moe_expert_ffn_workspace_size(256, 4, ctypes.byref(ex)) > 0
    assert L.moe_expert_ffn_shared_workspace_size(31, 4, ctypes.byref(ex)) == 0

    def call(T=256, K=4, flags=0, shared=sh, lora=None, w=FAKE, r=FAKE, y=FAKE, ws=FAKE, wsb=ws_need, e=ex):
        return L.moe_expert_ffn_q4_shared(None, T, K, flags, FAKE, FAKE, ctypes.byref(e),
                                          ctypes.byref(shared) if shared is not None else None, lora, w, r, y, ws, wsb)
    assert call(shared=None) == INVALID
    assert call(shared=_ex(E=2, d=2048, I=512, group=64)) == INVALID        # one shared expert
    assert call(shared=_ex(E=1, d=2048, I=1024, group=64)) == INVALID       # shapes must match
    assert call(shared=_ex(E=1, d=2048, I=512, group=32)) == INVALID
    assert call(w=None) == INVALID and call(r=None) == INVALID and call(y=None) == INVALID
    assert call(wsb=ws_need - 1) == INVALID
    assert call(ws=FAKE + 8) == INVALID
    assert call(flags=0x8) == INVALID
    assert call(T=31, wsb=1 << 40) == UNSUP                                 # the batched path only
    bad_lora = (lib_mod.moe_lora * 3)(*[lib_mod.moe_lora(FAKE, FAKE, 0, 32.0) for _ in range(3)])
    assert call(lora=ctypes.cast(bad_lora, ctypes.POINTER(lib_mod.moe_lora))) == INVALID  # rank 0


def test_workspace_sizes_closed_form():
    al = lambda v: (v + 255) // 256 * 256
    assert L.moe_prerouter_workspace_size(1, 256, 1024) == al(4096) + al(1024)
    assert L.moe_prerouter_workspace_size(0, 256, 1024) == 0
    ex = _ex(E=256, d=2048, I=512, group=64)
    want = al(1 * 4 * 512 * 4) + 3 * al(64 * 4)
    assert L.moe_expert_ffn_workspace_size(1, 4, ctypes.byref(ex)) == want
    assert L.moe_expert_ffn_workspace_size(256, 4, ctypes.byref(ex)) > want


def test_binding_checks_tensors_on_host():
    with pytest.raises(ValueError):
        lib_mod._ptr(torch.zeros(4), None, "x")      # a host tensor is refused before any call


def test_binding_rejects_short_tensors():
    """The Python binding checks every tensor against the call's sizes before the library sees it."""
    f16, f32, i32 = torch.float16, torch.float32, torch.int32
    T, K, d, E = 2, 4, 8, 16
    with pytest.raises(ValueError, match="o holds"):
        lib_mod.moe_combine(T, K, d, torch.zeros(T * K * d - 1, dtype=f32), torch.zeros(T * K, dtype=f32),
                            torch.zeros(T * d, dtype=f16), None, torch.zeros(T * d, dtype=f16))
    with pytest.raises(ValueError, match="y holds"):
        lib_mod.moe_combine(T, K, d, torch.zeros(T * K * d, dtype=f32), torch.zeros(T * K, dtype=f32),
                            torch.zeros(T * d, dtype=f16), None, torch.zeros(T * d - 2, dtype=f16))
    with pytest.raises(ValueError, match="idx holds"):
        lib_mod.moe_route_topk(T, d, E, K, 0, None, None, torch.zeros(T * E, dtype=f32),
                               torch.zeros(T * K - 1, dtype=i32), torch.zeros(T * K, dtype=f32))
    with pytest.raises(ValueError, match="offsets holds"):
        lib_mod.moe_sort_by_expert(T, K, E, torch.zeros(T * K, dtype=i32), torch.zeros(E + 1, dtype=i32),
                                   torch.zeros(E + 1, dtype=i32), torch.zeros(T * K, dtype=i32))
    with pytest.raises(ValueError, match="gain holds"):
        lib_mod.moe_rmsnorm(T, d, torch.zeros(T * d, dtype=f16), torch.zeros(d - 1, dtype=f16),
                            torch.zeros(T * d, dtype=f16))


def test_exchange_probe_rejects():
    """Every configuration outside the header's limits is refused before anything is enqueued."""
    good = dict(pattern=0, n_wg=256, group_size=256, xcd_local=0, words=1024, iters=100, load_scope=0,
                store_scope=0, epoch=1, replicas=1, wide_loads=0)
    cfg = lambda **k: lib_mod.moe_xchg_cfg(**{**good, **k})
    assert L.moe_exchange_probe_workspace_size(ctypes.byref(cfg())) > 0
    bad = [dict(pattern=2), dict(n_wg=0), dict(group_size=3), dict(words=1000), dict(words=256 * 65),
           dict(iters=0), dict(iters=40000), dict(load_scope=2), dict(store_scope=-1), dict(xcd_local=2),
           dict(pattern=1, group_size=8, iters=9000), dict(replicas=0), dict(replicas=9), dict(wide_loads=3), dict(wide_loads=2, words=2048, group_size=256)]
    for b in bad:
        c = cfg(**b)
        assert L.moe_exchange_probe_workspace_size(ctypes.byref(c)) == 0, b
        assert L.moe_exchange_probe(None, ctypes.byref(c), FAKE, 1 << 30, FAKE) == INVALID, b
    c = cfg()
    assert L.moe_exchange_probe(None, ctypes.byref(c), None, 1 << 30, FAKE) == INVALID
    assert L.moe_exchange_probe(None, ctypes.byref(c), FAKE, 16, FAKE) == INVALID       # workspace too small
    assert L.moe_exchange_probe(None, ctypes.byref(c), FAKE + 8, 1 << 30, FAKE) == INVALID  # not 256-aligned
    assert L.moe_exchange_probe(None, None, FAKE, 1 << 30, FAKE) == INVALID


def test_expert_ffn_noalloc_rejects():
    """The allocation-free entry point checks its arguments as moe_expert_ffn_q4 does (nothing is
    enqueued), and refuses a call whose scratch would exceed MOE_NOALLOC_SCRATCH_BYTES."""
    ex = _ex()
    f = lambda *a: L.moe_expert_ffn_q4_noalloc(None, *a)
    assert f(0, 2, 0, FAKE, FAKE, ctypes.byref(ex), None, FAKE, None, None, None) == INVALID   # T < 1
    assert f(1, 2, 0, None, FAKE, ctypes.byref(ex), None, FAKE, None, None, None) == INVALID   # no x
    assert f(1, 2, 0, FAKE, FAKE, ctypes.byref(ex), None, None, None, None, None) == INVALID   # no output
    assert f(1, 2, 0, FAKE, FAKE, ctypes.byref(ex), None, FAKE, FAKE, None, None) == INVALID   # half a fuse
    bad = _ex(bits=3)
    assert f(1, 2, 0, FAKE, FAKE, ctypes.byref(bad), None, FAKE, None, None, None) == UNSUP
    big = _ex(E=16, d=8192, I=8192)
    need = L.moe_expert_ffn_workspace_size(40, 16, ctypes.byref(big))
    assert need > lib_mod.MOE_NOALLOC_SCRATCH_BYTES
    assert f(40, 16, 0, FAKE, FAKE, ctypes.byref(big), None, FAKE, None, None, None) == lib_mod.MOE_ERR_TOO_LARGE
