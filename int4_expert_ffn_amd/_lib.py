"""ctypes binding of libmoe.so (include/moe.h).  Argument marshalling only: every step of the
layer runs in the library's HIP kernels.  Functions take torch tensors (device memory) or raw
integer device addresses, check dtype / device / contiguity, and raise MoEError on a non-OK
status.  The stream defaults to torch's current stream on the tensors' device.

Loading fails loudly (ImportError) when the library has not been built; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_HIP, MOE_ERR_TOO_LARGE = 0, 1, 2, 3, 4
MOE_NOALLOC_SCRATCH_BYTES = 16 << 20
MOE_TOPK_RENORM = 0x1
MOE_INPUT_RMSNORM = 0x2
MOE_DECODE_GIVEN_ROUTING = 0x4
MOE_MAX_E, MOE_MAX_K, MOE_MAX_D = 1024, 16, 8192

# every symbol include/moe.h declares
EXPORTS = (
    "moe_route_topk", "moe_prerouter_workspace_size", "moe_prerouter",
    "moe_expert_ffn_workspace_size", "moe_expert_ffn_q4", "moe_combine", "moe_rmsnorm", "moe_sort_by_expert",
    "moe_status_string", "moe_version", "moe_decode_workspace_size", "moe_decode_step",
    "moe_expert_ffn_sparse_workspace_size", "moe_expert_ffn_sparse", "moe_stream_workspace_size", "moe_stream_in",
    "moe_stream_in_many", "moe_read_probe", "moe_exchange_probe_workspace_size", "moe_exchange_probe",
    "moe_decode_step_grid", "moe_decode_step_stamped", "moe_expert_ffn_q4_noalloc", "moe_decode_step_grid_for",
    "moe_expert_ffn_shared_workspace_size", "moe_expert_ffn_q4_shared",
)


class MoEError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call}: {_lib.moe_status_string(status).decode()}")


class moe_qmat(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("biases", ctypes.c_void_p)]


class moe_experts(ctypes.Structure):
    _fields_ = [("n_experts", ctypes.c_int32), ("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("bits", ctypes.c_int32), ("group", ctypes.c_int32),
                ("gate", moe_qmat), ("up", moe_qmat), ("down", moe_qmat)]


class moe_lora(ctypes.Structure):
    _fields_ = [("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("rank", ctypes.c_int32), ("alpha", ctypes.c_float)]


class moe_prerouter_w(ctypes.Structure):
    _fields_ = [("d_hidden", ctypes.c_int32),
                ("fc1_x", ctypes.c_void_p), ("fc1_r", ctypes.c_void_p), ("fc1_b", ctypes.c_void_p),
                ("fc2", ctypes.c_void_p), ("fc2_b", ctypes.c_void_p),
                ("lin_x", ctypes.c_void_p), ("lin_r", ctypes.c_void_p), ("lin_b", ctypes.c_void_p)]


class moe_decode_layer(ctypes.Structure):
    _fields_ = [("experts", moe_experts), ("router", ctypes.c_void_p), ("head", moe_prerouter_w),
                ("norm_gain", ctypes.c_void_p)]


class moe_pool(ctypes.Structure):
    _fields_ = [("n_slots", ctypes.c_int32), ("slot_expert", ctypes.c_void_p), ("slot_stamp", ctypes.c_void_p),
                ("clock", ctypes.c_void_p)]


class moe_stream_job(ctypes.Structure):
    _fields_ = [("idx", ctypes.c_void_p), ("src", ctypes.POINTER(moe_experts)), ("pool_experts", ctypes.POINTER(moe_experts)),
                ("pool", ctypes.POINTER(moe_pool)), ("idx_slot", ctypes.c_void_p), ("counters", ctypes.c_void_p)]


class moe_xchg_cfg(ctypes.Structure):
    _fields_ = [("pattern", ctypes.c_int32), ("n_wg", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("xcd_local", ctypes.c_int32), ("words", ctypes.c_int32), ("iters", ctypes.c_int32),
                ("load_scope", ctypes.c_int32), ("store_scope", ctypes.c_int32), ("epoch", ctypes.c_uint32),
                ("replicas", ctypes.c_int32), ("wide_loads", ctypes.c_int32)]


class moe_decode_stack(ctypes.Structure):
    _fields_ = [("L", ctypes.c_int32), ("E", ctypes.c_int32), ("K", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("d_ff", ctypes.c_int32), ("bits", ctypes.c_int32), ("group", ctypes.c_int32),
                ("d_hidden", ctypes.c_int32), ("layers", ctypes.c_void_p), ("route_idx", ctypes.c_void_p),
                ("route_w", ctypes.c_void_p), ("norm_gains", ctypes.c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m int4_expert_ffn_amd.build`")
    # torch first: its HIP runtime must be the one libmoe.so binds to.  Loaded the other way round,
    # the process ends up with two runtimes and torch's streams are foreign to the library's.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, u32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
    st = ctypes.c_int
    sig = {
        "moe_route_topk": (st, [vp, i32, i32, i32, i32, u32, vp, vp, vp, vp, vp]),
        "moe_prerouter_workspace_size": (sz, [i32, i32, i32]),
        "moe_prerouter": (st, [vp, i32, i32, i32, i32, u32, vp, vp, vp, ctypes.POINTER(moe_prerouter_w), vp, vp, sz]),
        "moe_expert_ffn_workspace_size": (sz, [i32, i32, ctypes.POINTER(moe_experts)]),
        "moe_expert_ffn_q4": (st, [vp, i32, i32, u32, vp, vp, ctypes.POINTER(moe_experts), ctypes.POINTER(moe_lora),
                                   vp, vp, vp, vp, vp, sz]),
        "moe_expert_ffn_q4_noalloc": (st, [vp, i32, i32, u32, vp, vp, ctypes.POINTER(moe_experts),
                                           ctypes.POINTER(moe_lora), vp, vp, vp, vp]),
        "moe_expert_ffn_shared_workspace_size": (sz, [i32, i32, ctypes.POINTER(moe_experts)]),
        "moe_expert_ffn_q4_shared": (st, [vp, i32, i32, u32, vp, vp, ctypes.POINTER(moe_experts),
                                          ctypes.POINTER(moe_experts), ctypes.POINTER(moe_lora), vp, vp, vp, vp, sz]),
        "moe_expert_ffn_sparse_workspace_size": (sz, [i32, i32, ctypes.POINTER(moe_experts)]),
        "moe_expert_ffn_sparse": (st, [vp, i32, i32, u32, vp, vp, ctypes.POINTER(moe_experts), vp, vp, vp, vp, vp,
                                       vp, sz]),
        "moe_stream_workspace_size": (sz, [i32]),
        "moe_stream_in": (st, [vp, i32, vp, ctypes.POINTER(moe_experts), ctypes.POINTER(moe_experts),
                               ctypes.POINTER(moe_pool), vp, vp, vp, sz]),
        "moe_stream_in_many": (st, [vp, i32, i32, ctypes.POINTER(moe_stream_job), vp, sz]),
        "moe_read_probe": (st, [vp, vp, sz, vp]),
        "moe_exchange_probe_workspace_size": (sz, [ctypes.POINTER(moe_xchg_cfg)]),
        "moe_exchange_probe": (st, [vp, ctypes.POINTER(moe_xchg_cfg), vp, sz, vp]),
        "moe_combine": (st, [vp, i32, i32, i32, vp, vp, vp, vp, vp]),
        "moe_rmsnorm": (st, [vp, i32, i32, vp, vp, vp]),
        "moe_sort_by_expert": (st, [vp, i32, i32, i32, vp, vp, vp, vp]),
        "moe_status_string": (ctypes.c_char_p, [st]),
        "moe_decode_workspace_size": (sz, [ctypes.POINTER(moe_decode_stack)]),
        "moe_decode_step": (st, [vp, ctypes.POINTER(moe_decode_stack), i32, u32, vp, vp, vp, vp, sz]),
        "moe_decode_step_grid": (i32, [ctypes.POINTER(moe_decode_stack)]),
        "moe_decode_step_grid_for": (i32, [ctypes.POINTER(moe_decode_stack), i32]),
        "moe_decode_step_stamped": (st, [vp, ctypes.POINTER(moe_decode_stack), i32, u32, vp, vp, vp, vp, sz, vp, sz]),
        "moe_version": (i32, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


# ----------------------------------------------------------------------------------------------
def _ptr(t, dtype=None, name="tensor", pinned_ok=False) -> Optional[int]:
    """Device address of a tensor (checked), a raw int address, or None.  pinned_ok: a pinned host
    tensor is accepted too (its address is valid on the device)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    import torch
    if not t.is_cuda and not (pinned_ok and t.is_pinned()):
        raise ValueError(f"{name} must be a device tensor" + (" or pinned host memory" if pinned_ok else ""))
    if not t.is_cuda:
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        return _host_device_ptr(t, name)
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return t.data_ptr()


def _need(t, n, name):
    """A tensor argument must hold at least n elements (the kernels index it by the call's sizes;
    raw addresses and None pass through unchecked)."""
    if t is None or isinstance(t, int):
        return
    if t.numel() < n:
        raise ValueError(f"{name} holds {t.numel()} elements, the call needs {n}")


_hip = None


def _host_device_ptr(t, name) -> int:
    """The device address of pinned host memory, as the HIP runtime maps it (refused, before any
    launch, when the runtime reports the memory is not mapped for the device)."""
    global _hip
    if _hip is None:
        for cand in ("libamdhip64.so", "/opt/rocm/lib/libamdhip64.so"):
            try:
                _hip = ctypes.CDLL(cand)
                break
            except OSError:
                continue
        if _hip is None:
            raise ValueError("the HIP runtime library is not loadable")
        _hip.hipHostGetDevicePointer.restype = ctypes.c_int
        _hip.hipHostGetDevicePointer.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p, ctypes.c_uint]
    dptr = ctypes.c_void_p()
    err = _hip.hipHostGetDevicePointer(ctypes.byref(dptr), ctypes.c_void_p(t.data_ptr()), 0)
    if err != 0 or not dptr.value:
        raise ValueError(f"{name}: pinned host memory has no device mapping (hipHostGetDevicePointer error {err})")
    return dptr.value


def _stream(stream, *tensors) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    for t in tensors:
        if t is not None and not isinstance(t, int):
            return torch.cuda.current_stream(t.device).cuda_stream
    return None


def _check(status: int, call: str):
    if status != MOE_OK:
        raise MoEError(status, call)


def _f16():
    import torch
    return torch.float16


def _i32():
    import torch
    return torch.int32


def _f32():
    import torch
    return torch.float32


def _qw():
    import torch
    return (torch.int32, torch.uint32) if hasattr(torch, "uint32") else (torch.int32,)


class Experts:
    """A stack of E quantised experts (tensors kept alive here) and its C descriptor."""

    def __init__(self, gate, up, down, bits: int, group: int, neuron_major_down: bool = False,
                 host: bool = False):
        """neuron_major_down: down codes [E][d_ff][d_model] with group-major scales / biases
        [E][d_model/group][d_ff] (the layout of moe_expert_ffn_sparse), else codes [E][d_model][d_ff]
        with scales / biases [E][d_model][d_ff/group].  host: the tensors may be pinned host memory
        (a streaming source for moe_stream_in)."""
        self.tensors = (gate, up, down)
        q = gate[0]
        E, I, words = q.shape
        d = words * 32 // bits
        want = (E, I, d * bits // 32) if neuron_major_down else (E, d, I * bits // 32)
        if tuple(down[0].shape) != want:
            raise ValueError(f"down codes have shape {tuple(down[0].shape)}, expected {want}")
        want = (E, d // group, I) if neuron_major_down else (E, d, I // group)
        if tuple(down[1].shape) != want or tuple(down[2].shape) != want:
            raise ValueError(f"down scales/biases have shape {tuple(down[1].shape)}, expected {want}")
        self.neuron_major_down = neuron_major_down
        mats = [moe_qmat(_ptr(m[0], _qw(), "q", host), _ptr(m[1], _f16(), "scales", host),
                         _ptr(m[2], _f16(), "biases", host)) for m in (gate, up, down)]
        self.desc = moe_experts(E, d, I, bits, group, *mats)
        self.E, self.d, self.I, self.bits, self.group = E, d, I, bits, group


class Lora3:
    """Adapters of gate, up and down: sequence of three (A, B) float16 tensor pairs."""

    def __init__(self, pairs: Sequence, alpha: float):
        self.tensors = tuple(pairs)
        arr = (moe_lora * 3)()
        for i, (A, B) in enumerate(pairs):
            arr[i] = moe_lora(_ptr(A, _f16(), "lora A"), _ptr(B, _f16(), "lora B"), A.shape[0], float(alpha))
        self.desc = arr


class PrerouterWeights:
    def __init__(self, w: dict):
        self.tensors = dict(w)
        g = lambda k: _ptr(w.get(k), _f16(), k)
        self.desc = moe_prerouter_w(w["fc1_x"].shape[0], g("fc1_x"), g("fc1_r"), g("fc1_b"), g("fc2"), g("fc2_b"),
                                    g("lin_x"), g("lin_r"), g("lin_b"))
        self.H = w["fc1_x"].shape[0]


# ---------------------------------------------------------------------------------------------- calls
def moe_route_topk(T, d, E, K, flags, x, w_router, logits, idx, w, stream=None):
    if w_router is not None:
        _need(x, T * d, "x")
        _need(w_router, E * d, "w_router")
    _need(logits, T * E, "logits")
    _need(idx, T * K, "idx")
    _need(w, T * K, "w")
    st = _lib.moe_route_topk(_stream(stream, logits, idx), T, d, E, K, flags,
                             _ptr(x, _f16(), "x"), _ptr(w_router, _f16(), "w_router"),
                             _ptr(logits, _f32(), "logits"), _ptr(idx, _i32(), "idx"), _ptr(w, _f32(), "w"))
    _check(st, "moe_route_topk")


def moe_prerouter_workspace_size(T, E, d_hidden) -> int:
    return _lib.moe_prerouter_workspace_size(T, E, d_hidden)


def moe_prerouter(T, d, E, K, flags, x, idx_cur, idx_prev, pw: PrerouterWeights, logits, workspace,
                  workspace_bytes=None, stream=None):
    _need(x, T * d, "x")
    _need(idx_cur, T * K, "idx_cur")
    _need(idx_prev, T * K, "idx_prev")
    _need(logits, T * E, "logits")
    nbytes = workspace_bytes if workspace_bytes is not None else workspace.numel() * workspace.element_size()
    st = _lib.moe_prerouter(_stream(stream, logits), T, d, E, K, flags, _ptr(x, _f16(), "x"),
                            _ptr(idx_cur, _i32(), "idx_cur"), _ptr(idx_prev, _i32(), "idx_prev"),
                            ctypes.byref(pw.desc), _ptr(logits, _f32(), "logits"), _ptr(workspace, None, "workspace"),
                            nbytes)
    _check(st, "moe_prerouter")


def moe_expert_ffn_workspace_size(T, K, ex: Experts) -> int:
    return _lib.moe_expert_ffn_workspace_size(T, K, ctypes.byref(ex.desc))


def moe_expert_ffn_q4(T, K, flags, x, idx, ex: Experts, lora3: Optional[Lora3], out, w_fuse, r_fuse, y_fuse,
                      workspace, workspace_bytes=None, stream=None):
    d = ex.d
    _need(x, T * d, "x")
    _need(idx, T * K, "idx")
    _need(out, T * K * d, "out")
    _need(w_fuse, T * K, "w_fuse")
    _need(r_fuse, T * d, "r_fuse")
    _need(y_fuse, T * d, "y_fuse")
    nbytes = workspace_bytes if workspace_bytes is not None else workspace.numel() * workspace.element_size()
    st = _lib.moe_expert_ffn_q4(_stream(stream, x, idx), T, K, flags, _ptr(x, _f16(), "x"), _ptr(idx, _i32(), "idx"),
                                ctypes.byref(ex.desc), ctypes.cast(lora3.desc, ctypes.POINTER(moe_lora)) if lora3 is not None else None,
                                _ptr(out, _f32(), "out"), _ptr(w_fuse, _f32(), "w_fuse"), _ptr(r_fuse, _f16(), "r_fuse"),
                                _ptr(y_fuse, _f16(), "y_fuse"), _ptr(workspace, None, "workspace"), nbytes)
    _check(st, "moe_expert_ffn_q4")


def moe_expert_ffn_q4_noalloc(T, K, flags, x, idx, ex: Experts, lora3: Optional[Lora3], out, w_fuse, r_fuse, y_fuse,
                              stream=None):
    """moe_expert_ffn_q4 on the library's own scratch (no workspace argument, nothing allocated)."""
    d = ex.d
    _need(x, T * d, "x")
    _need(idx, T * K, "idx")
    _need(out, T * K * d, "out")
    _need(w_fuse, T * K, "w_fuse")
    _need(r_fuse, T * d, "r_fuse")
    _need(y_fuse, T * d, "y_fuse")
    st = _lib.moe_expert_ffn_q4_noalloc(_stream(stream, x, idx), T, K, flags, _ptr(x, _f16(), "x"),
                                        _ptr(idx, _i32(), "idx"), ctypes.byref(ex.desc),
                                        ctypes.cast(lora3.desc, ctypes.POINTER(moe_lora)) if lora3 is not None else None,
                                        _ptr(out, _f32(), "out"), _ptr(w_fuse, _f32(), "w_fuse"),
                                        _ptr(r_fuse, _f16(), "r_fuse"), _ptr(y_fuse, _f16(), "y_fuse"))
    _check(st, "moe_expert_ffn_q4_noalloc")


def moe_expert_ffn_shared_workspace_size(T, K, ex: Experts) -> int:
    return _lib.moe_expert_ffn_shared_workspace_size(T, K, ctypes.byref(ex.desc))


def moe_expert_ffn_q4_shared(T, K, flags, x, idx, ex: Experts, shared: Experts, lora3: Optional[Lora3], w, r, y,
                             workspace, workspace_bytes=None, stream=None):
    """Routed experts + a shared expert (with its LoRA) + the combine in one call: y = r + sum_k w_k o_k
    + shared."""
    d = ex.d
    _need(x, T * d, "x")
    _need(idx, T * K, "idx")
    _need(w, T * K, "w")
    _need(r, T * d, "r")
    _need(y, T * d, "y")
    nbytes = workspace_bytes if workspace_bytes is not None else workspace.numel() * workspace.element_size()
    st = _lib.moe_expert_ffn_q4_shared(_stream(stream, x, idx), T, K, flags, _ptr(x, _f16(), "x"),
                                       _ptr(idx, _i32(), "idx"), ctypes.byref(ex.desc), ctypes.byref(shared.desc),
                                       ctypes.cast(lora3.desc, ctypes.POINTER(moe_lora)) if lora3 is not None else None,
                                       _ptr(w, _f32(), "w"), _ptr(r, _f16(), "r"), _ptr(y, _f16(), "y"),
                                       _ptr(workspace, None, "workspace"), nbytes)
    _check(st, "moe_expert_ffn_q4_shared")


def moe_expert_ffn_sparse_workspace_size(T, K, ex: Experts) -> int:
    return _lib.moe_expert_ffn_sparse_workspace_size(T, K, ctypes.byref(ex.desc))


def moe_expert_ffn_sparse(T, K, flags, x, idx, ex: Experts, out, w_fuse, r_fuse, y_fuse, n_active, workspace,
                          workspace_bytes=None, stream=None):
    """ReLU activation-sparse expert FFN; ex.down is neuron-major ([E][d_ff][d_model] packed)."""
    d = ex.d
    _need(x, T * d, "x")
    _need(idx, T * K, "idx")
    _need(out, T * K * d, "out")
    _need(w_fuse, T * K, "w_fuse")
    _need(r_fuse, T * d, "r_fuse")
    _need(y_fuse, T * d, "y_fuse")
    _need(n_active, T * K, "n_active")
    nbytes = workspace_bytes if workspace_bytes is not None else workspace.numel() * workspace.element_size()
    st = _lib.moe_expert_ffn_sparse(_stream(stream, x, idx), T, K, flags, _ptr(x, _f16(), "x"),
                                    _ptr(idx, _i32(), "idx"), ctypes.byref(ex.desc), _ptr(out, _f32(), "out"),
                                    _ptr(w_fuse, _f32(), "w_fuse"), _ptr(r_fuse, _f16(), "r_fuse"),
                                    _ptr(y_fuse, _f16(), "y_fuse"), _ptr(n_active, _i32(), "n_active"),
                                    _ptr(workspace, None, "workspace"), nbytes)
    _check(st, "moe_expert_ffn_sparse")


class Pool:
    """An HBM pool of n_slots experts shaped like `like` (an Experts), its slot state, and its
    descriptors for moe_stream_in and the expert FFN calls."""

    def __init__(self, like: Experts, n_slots: int, device):
        import torch
        dev = torch.device(device)
        mats = []
        for m in like.tensors:
            mats.append(tuple(torch.empty((n_slots,) + tuple(a.shape[1:]), dtype=a.dtype, device=dev) for a in m))
        self.experts = Experts(*mats, like.bits, like.group, neuron_major_down=like.neuron_major_down)
        self.slot_expert = torch.full((n_slots,), -1, dtype=torch.int32, device=dev)
        self.slot_stamp = torch.full((n_slots,), -1, dtype=torch.int32, device=dev)
        self.clock = torch.zeros(1, dtype=torch.int32, device=dev)
        self.desc = moe_pool(n_slots, self.slot_expert.data_ptr(), self.slot_stamp.data_ptr(), self.clock.data_ptr())
        self.n_slots = n_slots

    def reset(self):
        self.slot_expert.fill_(-1)
        self.slot_stamp.fill_(-1)
        self.clock.zero_()


def moe_stream_workspace_size(K) -> int:
    return _lib.moe_stream_workspace_size(K)


def moe_stream_in(K, idx, src: Experts, pool: Pool, idx_slot, counters, workspace, workspace_bytes=None,
                  stream=None):
    nbytes = workspace_bytes if workspace_bytes is not None else workspace.numel() * workspace.element_size()
    st = _lib.moe_stream_in(_stream(stream, idx, idx_slot), K, _ptr(idx, _i32(), "idx"), ctypes.byref(src.desc),
                            ctypes.byref(pool.experts.desc), ctypes.byref(pool.desc), _ptr(idx_slot, _i32(), "idx_slot"),
                            _ptr(counters, _i32(), "counters"), _ptr(workspace, None, "workspace"), nbytes)
    _check(st, "moe_stream_in")


MOE_POOL_MAX_JOBS = 8
MOE_READ_PROBE_BLOCKS = 4096


def moe_read_probe(buf, out, stream=None):
    """Streaming read of the device tensor `buf` (measurement aid); out: int32 [MOE_READ_PROBE_BLOCKS]."""
    nbytes = buf.numel() * buf.element_size()
    if out.numel() < MOE_READ_PROBE_BLOCKS:
        raise ValueError(f"moe_read_probe: out needs {MOE_READ_PROBE_BLOCKS} int32 words")
    st = _lib.moe_read_probe(_stream(stream, buf, out), _ptr(buf, None, "buf"), nbytes, _ptr(out, _i32(), "out"))
    _check(st, "moe_read_probe")


MOE_XCHG_ALL, MOE_XCHG_RING = 0, 1
MOE_XCHG_SCOPE_DEVICE, MOE_XCHG_SCOPE_XCD = 0, 1


def moe_exchange_probe_workspace_size(cfg: moe_xchg_cfg) -> int:
    return _lib.moe_exchange_probe_workspace_size(ctypes.byref(cfg))


def moe_exchange_probe(cfg: moe_xchg_cfg, workspace, out, stream=None):
    """Tagged-word hand-off probe (measurement aid).  workspace: uint8 device tensor of
    moe_exchange_probe_workspace_size(cfg) bytes, zeroed once; out: int32 [1 + 3 n_wg] device tensor
    with out[0] zeroed (waits that ran out are added there)."""
    if out.numel() < 1 + 3 * cfg.n_wg:
        raise ValueError(f"moe_exchange_probe: out needs {1 + 3 * cfg.n_wg} int32 words")
    nbytes = workspace.numel() * workspace.element_size()
    st = _lib.moe_exchange_probe(_stream(stream, workspace, out), ctypes.byref(cfg), _ptr(workspace, None, "workspace"),
                                 nbytes, _ptr(out, _i32(), "out"))
    _check(st, "moe_exchange_probe")


def moe_stream_in_many(K, jobs, workspace, workspace_bytes=None, stream=None):
    """jobs: sequence of (idx, src Experts, Pool, idx_slot, counters or None), at most MOE_POOL_MAX_JOBS,
    distinct pools of one shape; workspace of len(jobs) * moe_stream_workspace_size(K) bytes."""
    n = len(jobs)
    arr = (moe_stream_job * max(1, n))()
    for i, (idx, src, pool, idx_slot, counters) in enumerate(jobs):
        arr[i] = moe_stream_job(_ptr(idx, _i32(), "idx"), ctypes.pointer(src.desc), ctypes.pointer(pool.experts.desc),
                                ctypes.pointer(pool.desc), _ptr(idx_slot, _i32(), "idx_slot"),
                                _ptr(counters, _i32(), "counters"))
    nbytes = workspace_bytes if workspace_bytes is not None else workspace.numel() * workspace.element_size()
    first = jobs[0] if n else (None,) * 5
    st = _lib.moe_stream_in_many(_stream(stream, first[0], first[3]), n, K, arr, _ptr(workspace, None, "workspace"),
                                 nbytes)
    _check(st, "moe_stream_in_many")


def moe_combine(T, K, d, o, w, r, shared, y, stream=None):
    _need(o, T * K * d, "o")
    _need(w, T * K, "w")
    _need(r, T * d, "r")
    _need(shared, T * d, "shared")
    _need(y, T * d, "y")
    st = _lib.moe_combine(_stream(stream, o, y), T, K, d, _ptr(o, _f32(), "o"), _ptr(w, _f32(), "w"),
                          _ptr(r, _f16(), "r"), _ptr(shared, _f32(), "shared"), _ptr(y, _f16(), "y"))
    _check(st, "moe_combine")


def moe_rmsnorm(T, d, h, gain, x, stream=None):
    _need(h, T * d, "h")
    _need(gain, d, "gain")
    _need(x, T * d, "x")
    st = _lib.moe_rmsnorm(_stream(stream, h, x), T, d, _ptr(h, _f16(), "h"), _ptr(gain, _f16(), "gain"),
                          _ptr(x, _f16(), "x"))
    _check(st, "moe_rmsnorm")


def moe_sort_by_expert(T, K, E, idx, counts, offsets, perm, stream=None):
    _need(idx, T * K, "idx")
    _need(counts, E + 1, "counts")
    _need(offsets, E + 2, "offsets")
    _need(perm, T * K, "perm")
    st = _lib.moe_sort_by_expert(_stream(stream, idx), T, K, E, _ptr(idx, _i32(), "idx"), _ptr(counts, _i32(), "counts"),
                                 _ptr(offsets, _i32(), "offsets"), _ptr(perm, _i32(), "perm"))
    _check(st, "moe_sort_by_expert")


def moe_decode_workspace_size(stack: "moe_decode_stack") -> int:
    return _lib.moe_decode_workspace_size(ctypes.byref(stack))


def moe_decode_step(stack: "moe_decode_stack", token, flags, h_in, h_out, workspace, workspace_bytes=None,
                    stream=None, h_layers=None):
    nbytes = workspace_bytes if workspace_bytes is not None else workspace.numel() * workspace.element_size()
    st = _lib.moe_decode_step(_stream(stream, h_in, h_out), ctypes.byref(stack), token, flags, _ptr(h_in, _f16(), "h_in"),
                              _ptr(h_out, _f16(), "h_out"), _ptr(h_layers, _f16(), "h_layers"),
                              _ptr(workspace, None, "workspace"), nbytes)
    _check(st, "moe_decode_step")


def moe_decode_step_grid(stack: "moe_decode_stack") -> int:
    return _lib.moe_decode_step_grid(ctypes.byref(stack))


def moe_decode_step_grid_for(stack: "moe_decode_stack", compute_units: int) -> int:
    return _lib.moe_decode_step_grid_for(ctypes.byref(stack), int(compute_units))


def moe_decode_step_stamped(stack: "moe_decode_stack", token, flags, h_in, h_out, stamps, workspace,
                            workspace_bytes=None, stream=None, h_layers=None):
    """moe_decode_step writing phase stamps into `stamps` (int64 device tensor, [G][L][16])."""
    nbytes = workspace_bytes if workspace_bytes is not None else workspace.numel() * workspace.element_size()
    st = _lib.moe_decode_step_stamped(_stream(stream, h_in, h_out), ctypes.byref(stack), token, flags,
                                      _ptr(h_in, _f16(), "h_in"), _ptr(h_out, _f16(), "h_out"),
                                      _ptr(h_layers, _f16(), "h_layers"), _ptr(stamps, None, "stamps"),
                                      stamps.numel() * stamps.element_size(), _ptr(workspace, None, "workspace"), nbytes)
    _check(st, "moe_decode_step_stamped")


def moe_version() -> int:
    return _lib.moe_version()


def moe_status_string(status: int) -> str:
    return _lib.moe_status_string(status).decode()
