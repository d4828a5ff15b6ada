"""ctypes binding of libmoe.so (the C ABI declared in include/moe.h).

Argument marshalling only: every step of the MoE path runs in the library's
HIP kernels. torch is used for device memory and streams; numpy for host
buffers. The library must have been built (routed_expert_int4_router_amd.build);
loading fails loudly otherwise, and there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_ENOMEM, MOE_EHIP, MOE_ESTATE = 0, -1, -2, -3, -4
STORE_DEVICE, STORE_HOST, STORE_FILE = 0, 1, 2
KERNELS_FAST, KERNELS_SCALAR = 0, 1
FILE_DIRECT = 1
_STATUS_NAMES = {MOE_EINVAL: "MOE_EINVAL", MOE_ENOMEM: "MOE_ENOMEM", MOE_EHIP: "MOE_EHIP", MOE_ESTATE: "MOE_ESTATE"}

# every symbol moe.h declares
EXPORTS = [
    "moe_expert_bytes", "moe_expert_stride", "moe_blob_offset", "moe_pack", "moe_unpack",
    "moe_model_create", "moe_model_set_layer", "moe_model_set_experts", "moe_model_host_blob", "moe_model_open_blob",
    "moe_model_destroy", "moe_layer_forward", "moe_layer_decode", "moe_stack_decode",
    "moe_layer_forward_noalloc", "moe_debug_routing",
    "moe_pool_create", "moe_pool_reset", "moe_pool_stats", "moe_pool_trace", "moe_pool_destroy",
    "moe_pool_simulate", "moe_model_set_kernels", "moe_profile_enable", "moe_profile_read", "moe_last_error",
    "moe_gdn_create", "moe_gdn_set_layer", "moe_gdn_reset", "moe_gdn_decode", "moe_gdn_profile", "moe_gdn_read_state",
    "moe_gdn_destroy",
    "moe_attn_create", "moe_attn_set_layer", "moe_attn_write_cache", "moe_attn_read_cache", "moe_attn_decode",
    "moe_attn_profile", "moe_attn_destroy",
]


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("hidden", "n_experts", "top_k", "inter", "shared_inter", "bits", "group", "n_layers", "norm_topk")]


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_uint64), ("total_ms", ctypes.c_double)]


class GdnConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("n_layers", "n_k_heads", "n_v_heads", "d_k", "d_v")]


class AttnConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("n_layers", "n_q_heads", "n_kv_heads", "head_dim", "rot_dim", "max_pos")]


class PoolStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in
                ("accesses", "hits", "misses", "evictions", "h2d_bytes", "requested_bytes",
                 "storage_reads", "storage_bytes", "direct_io")]

    def as_dict(self):
        return {n: int(getattr(self, n)) for n, _ in self._fields_}


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m routed_expert_int4_router_amd.build`")
        # torch ships its own HIP runtime (libamdhip64.so.7). Loading torch first
        # makes libmoe's libamdhip64.so.7 dependency resolve to that same copy, so
        # torch's device pointers and streams and libmoe's kernels share one runtime.
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        maps = open("/proc/self/maps").read()
        runtimes = {ln.split()[-1] for ln in maps.splitlines() if "libamdhip64" in ln}
        if len(runtimes) > 1:
            raise ImportError(f"two HIP runtimes loaded in one process: {sorted(runtimes)}")
        P, I32, I64, SZ, U64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_uint64
        CP = ctypes.POINTER(Config)
        sig = {
            "moe_expert_bytes": (SZ, [CP, I32]),
            "moe_expert_stride": (SZ, [CP, I32]),
            "moe_blob_offset": (U64, [U64, U64, U64]),
            "moe_pack": (I32, [CP, I32, P, P, P, I64, P, SZ]),
            "moe_unpack": (I32, [CP, I32, P, P, P]),
            "moe_model_create": (I32, [CP, I32, ctypes.POINTER(P)]),
            "moe_model_set_layer": (I32, [P, I32, P, P, P, P]),
            "moe_model_set_experts": (I32, [P, I64, I64, P]),
            "moe_model_host_blob": (I32, [P, ctypes.POINTER(P), ctypes.POINTER(SZ)]),
            "moe_model_open_blob": (I32, [P, ctypes.c_char_p, U64, I32]),
            "moe_model_destroy": (None, [P]),
            "moe_layer_forward": (I32, [P, I32, P, I32, P, P]),
            "moe_layer_decode": (I32, [P, I32, P, I32, P, P]),
            "moe_stack_decode": (I32, [P, P, P, I32, P, P]),
            "moe_layer_forward_noalloc": (I32, [P, I32, P, I32, P, P]),
            "moe_debug_routing": (I32, [P, P, P, SZ, ctypes.POINTER(SZ)]),
            "moe_pool_create": (I32, [P, SZ, ctypes.POINTER(P)]),
            "moe_pool_reset": (I32, [P]),
            "moe_pool_stats": (I32, [P, ctypes.POINTER(PoolStats)]),
            "moe_pool_trace": (I32, [P, P, P, SZ, ctypes.POINTER(SZ)]),
            "moe_pool_destroy": (None, [P]),
            "moe_pool_simulate": (I32, [I64, I32, I64, P, P, P]),
            "moe_model_set_kernels": (I32, [P, I32]),
            "moe_profile_enable": (I32, [P, I32]),
            "moe_profile_read": (I32, [P, ctypes.POINTER(KernelTime), SZ, ctypes.POINTER(SZ)]),
            "moe_last_error": (ctypes.c_char_p, []),
            "moe_gdn_create": (I32, [ctypes.POINTER(GdnConfig), ctypes.POINTER(P)]),
            "moe_gdn_set_layer": (I32, [P, I32, P, P, P, P]),
            "moe_gdn_reset": (I32, [P]),
            "moe_gdn_decode": (I32, [P, I32, I32, P, P, P, P, I32, P, P]),
            "moe_gdn_read_state": (I32, [P, I32, P, P]),
            "moe_gdn_profile": (I32, [P, I32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(U64)]),
            "moe_gdn_destroy": (None, [P]),
            "moe_attn_create": (I32, [ctypes.POINTER(AttnConfig), ctypes.POINTER(P)]),
            "moe_attn_set_layer": (I32, [P, I32, P, P]),
            "moe_attn_write_cache": (I32, [P, I32, I32, I32, P, P]),
            "moe_attn_read_cache": (I32, [P, I32, I32, I32, P, P]),
            "moe_attn_decode": (I32, [P, I32, I32, I32, P, P, P, P, I32, P, P]),
            "moe_attn_profile": (I32, [P, I32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(U64)]),
            "moe_attn_destroy": (None, [P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def last_error() -> str:
    return lib().moe_last_error().decode()


def _check(st: int) -> None:
    if st != MOE_OK:
        raise MoeError(st, last_error())


def make_config(hidden, n_experts, top_k, inter, shared_inter=None, bits=4, group=64, n_layers=1,
                norm_topk=1) -> Config:
    return Config(hidden, n_experts, top_k, inter, inter if shared_inter is None else shared_inter, bits, group,
                  n_layers, norm_topk)


def config_of(obj) -> Config:
    """Config from any object with the moe_config field names (a dataclass, a namespace)."""
    if isinstance(obj, Config):
        return obj
    return make_config(obj.hidden, obj.n_experts, obj.top_k, obj.inter, obj.shared_inter, obj.bits, obj.group,
                       obj.n_layers, getattr(obj, "norm_topk", 1))


def _ptr(a) -> int:
    """Address of a numpy array or torch tensor (contiguous)."""
    if a is None:
        return None
    if isinstance(a, np.ndarray):
        if not a.flags["C_CONTIGUOUS"]:
            raise ValueError("array must be C-contiguous")
        return a.ctypes.data
    if hasattr(a, "data_ptr"):
        if not a.is_contiguous():
            raise ValueError("tensor must be contiguous")
        return a.data_ptr()
    return int(a)


def _check_io(x, out, n: int, hidden: int) -> None:
    """Refuse buffers the kernels would read or write out of bounds: x and out
    must be device tensors of the right type holding at least n rows of
    ``hidden`` elements (no check for an empty call)."""
    if n < 0:
        raise ValueError("n_tok must be >= 0")
    if n == 0:
        return
    import torch
    for name, t, dtypes in (("x", x, (torch.int16, torch.bfloat16)), ("out", out, (torch.float32,))):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch tensor on the GPU")
        if not t.is_cuda:
            raise ValueError(f"{name} must be on the GPU")
        if t.dtype not in dtypes:
            raise TypeError(f"{name} must be of dtype {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
        if t.dim() < 1 or t.shape[-1] != hidden:
            raise ValueError(f"{name} must have rows of hidden = {hidden} elements, got shape {tuple(t.shape)}")
        if t.numel() < n * hidden:
            raise ValueError(f"{name} holds {t.numel() // hidden} rows, fewer than n_tok = {n}")


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if hasattr(stream, "cuda_stream"):
        return stream.cuda_stream
    return int(stream)


def expert_bytes(cfg, inter: Optional[int] = None) -> int:
    c = config_of(cfg)
    return int(lib().moe_expert_bytes(ctypes.byref(c), c.inter if inter is None else inter))


def expert_stride(cfg, inter: Optional[int] = None) -> int:
    c = config_of(cfg)
    return int(lib().moe_expert_stride(ctypes.byref(c), c.inter if inter is None else inter))


def blob_offset(base: int, gid: int, stride: int) -> int:
    return int(lib().moe_blob_offset(base, gid, stride))


def pack(cfg, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray, inter: Optional[int] = None,
         out: Optional[np.ndarray] = None) -> np.ndarray:
    """Pack n experts (fp32 [n][I][H], [n][I][H], [n][H][I], or one expert without the n axis)."""
    c = config_of(cfg)
    inter = c.inter if inter is None else inter
    wg = np.ascontiguousarray(w_gate, dtype=np.float32)
    wu = np.ascontiguousarray(w_up, dtype=np.float32)
    wd = np.ascontiguousarray(w_down, dtype=np.float32)
    n = 1 if wg.ndim == 2 else wg.shape[0]
    stride = expert_stride(c, inter)
    if out is None:
        out = np.empty(n * stride, dtype=np.uint8)
    _check(lib().moe_pack(ctypes.byref(c), inter, _ptr(wg), _ptr(wu), _ptr(wd), n, _ptr(out), out.nbytes))
    return out


def unpack(cfg, record: np.ndarray, inter: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    c = config_of(cfg)
    inter = c.inter if inter is None else inter
    rec = np.ascontiguousarray(record, dtype=np.uint8)
    q = np.empty(3 * c.hidden * inter, dtype=np.uint8)
    sc = np.empty(3 * c.hidden * inter // 64 * 2, dtype=np.uint16)
    _check(lib().moe_unpack(ctypes.byref(c), inter, _ptr(rec), _ptr(q), _ptr(sc)))
    return q, sc


def pool_simulate(n_slots: int, gids: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    g = np.ascontiguousarray(gids, dtype=np.int64)
    steps, k = g.shape
    hit = np.empty(steps * k, dtype=np.uint8)
    victim = np.empty(steps * k, dtype=np.int64)
    _check(lib().moe_pool_simulate(n_slots, k, steps, _ptr(g), _ptr(hit), _ptr(victim)))
    return hit, victim


class Model:
    """A model handle: resident dense weights + routed experts in HBM or pinned host memory."""

    def __init__(self, cfg, storage: int = STORE_DEVICE):
        self.cfg = config_of(cfg)
        self.storage = storage
        h = ctypes.c_void_p()
        _check(lib().moe_model_create(ctypes.byref(self.cfg), storage, ctypes.byref(h)))
        self._h = h

    @property
    def handle(self):
        return self._h

    def close(self):
        if self._h:
            lib().moe_model_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_layer(self, layer: int, router_w: np.ndarray, router_bias: Optional[np.ndarray], shared_record: np.ndarray,
                  shared_gate: np.ndarray):
        rw = np.ascontiguousarray(router_w, dtype=np.float32)
        rb = None if router_bias is None else np.ascontiguousarray(router_bias, dtype=np.float32)
        sr = np.ascontiguousarray(shared_record, dtype=np.uint8)
        sg = np.ascontiguousarray(shared_gate, dtype=np.float32)
        _check(lib().moe_model_set_layer(self._h, layer, _ptr(rw), _ptr(rb), _ptr(sr), _ptr(sg)))

    def set_experts(self, first_gid: int, records: np.ndarray):
        recs = np.ascontiguousarray(records, dtype=np.uint8)
        stride = expert_stride(self.cfg)
        n = recs.nbytes // stride
        _check(lib().moe_model_set_experts(self._h, first_gid, n, _ptr(recs)))

    def host_blob(self) -> np.ndarray:
        p = ctypes.c_void_p()
        n = ctypes.c_size_t()
        _check(lib().moe_model_host_blob(self._h, ctypes.byref(p), ctypes.byref(n)))
        return np.ctypeslib.as_array((ctypes.c_uint8 * n.value).from_address(p.value))

    def open_blob(self, path: str, base: int = 0, direct: bool = True):
        """File-backed model: read records from the blob file at `path` (O_DIRECT when allowed)."""
        _check(lib().moe_model_open_blob(self._h, os.fsencode(path), base, FILE_DIRECT if direct else 0))

    def layer_forward(self, layer: int, x, out, n_tok: Optional[int] = None, stream=None):
        n = x.shape[0] if n_tok is None else n_tok
        _check_io(x, out, n, self.cfg.hidden)
        _check(lib().moe_layer_forward(self._h, layer, _ptr(x), n, _ptr(out), _stream(stream)))

    def layer_decode(self, layer: int, x, out, n_tok: Optional[int] = None, stream=None):
        n = x.shape[0] if n_tok is None else n_tok
        _check_io(x, out, n, self.cfg.hidden)
        _check(lib().moe_layer_decode(self._h, layer, _ptr(x), n, _ptr(out), _stream(stream)))

    def layer_forward_noalloc(self, layer: int, x, out, n_tok: Optional[int] = None, stream=None):
        n = x.shape[0] if n_tok is None else n_tok
        _check_io(x, out, n, self.cfg.hidden)
        _check(lib().moe_layer_forward_noalloc(self._h, layer, _ptr(x), n, _ptr(out), _stream(stream)))

    def stack_decode(self, x0, out, pool: Optional["Pool"] = None, n_tok: Optional[int] = None, stream=None):
        n = x0.shape[0] if n_tok is None else n_tok
        _check_io(x0, out, n, self.cfg.hidden)
        _check(lib().moe_stack_decode(self._h, None if pool is None else pool.handle, _ptr(x0), n, _ptr(out),
                                      _stream(stream)))

    def set_kernels(self, kernels: int):
        """KERNELS_FAST, or KERNELS_SCALAR: the plainly written, bit-identical variants."""
        _check(lib().moe_model_set_kernels(self._h, kernels))

    def profile_enable(self, enable: bool = True):
        _check(lib().moe_profile_enable(self._h, 1 if enable else 0))

    def profile_read(self) -> dict:
        """{kernel family: (launches, total_ms)} since enable / the last read."""
        arr = (KernelTime * 32)()
        n = ctypes.c_size_t()
        _check(lib().moe_profile_read(self._h, arr, 32, ctypes.byref(n)))
        return {arr[i].name.decode(): (int(arr[i].launches), float(arr[i].total_ms)) for i in range(min(32, n.value))}

    def debug_routing(self, cap: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
        n = ctypes.c_size_t()
        _check(lib().moe_debug_routing(self._h, None, None, 0, ctypes.byref(n)))
        steps = n.value if cap is None else min(cap, n.value)
        k = self.cfg.top_k
        idx = np.empty((steps, k), dtype=np.int32)
        w = np.empty((steps, k), dtype=np.float32)
        _check(lib().moe_debug_routing(self._h, _ptr(idx), _ptr(w), steps, ctypes.byref(n)))
        return idx, w


class Pool:
    """Bounded HBM expert pool of a host-storage model."""

    def __init__(self, model: Model, budget_bytes: int):
        self.model = model
        h = ctypes.c_void_p()
        _check(lib().moe_pool_create(model.handle, budget_bytes, ctypes.byref(h)))
        self._h = h

    @property
    def handle(self):
        return self._h

    def close(self):
        if self._h:
            lib().moe_pool_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def reset(self):
        _check(lib().moe_pool_reset(self._h))

    def stats(self) -> dict:
        s = PoolStats()
        _check(lib().moe_pool_stats(self._h, ctypes.byref(s)))
        return s.as_dict()

    def trace(self) -> Tuple[np.ndarray, np.ndarray]:
        n = ctypes.c_size_t()
        _check(lib().moe_pool_trace(self._h, None, None, 0, ctypes.byref(n)))
        hit = np.empty(n.value, dtype=np.uint8)
        victim = np.empty(n.value, dtype=np.int64)
        _check(lib().moe_pool_trace(self._h, _ptr(hit), _ptr(victim), n.value, ctypes.byref(n)))
        return hit, victim


def _check_dev(name, t, dtypes, numel):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a torch tensor on the GPU")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must be of dtype {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, the call needs {numel}")


class GatedDeltaNet:
    """Gated DeltaNet decode layers (recurrent state in HBM)."""

    def __init__(self, n_layers: int, n_k_heads: int, n_v_heads: int, d_k: int, d_v: int):
        self.cfg = GdnConfig(n_layers, n_k_heads, n_v_heads, d_k, d_v)
        self.channels = 2 * n_k_heads * d_k + n_v_heads * d_v
        h = ctypes.c_void_p()
        _check(lib().moe_gdn_create(ctypes.byref(self.cfg), ctypes.byref(h)))
        self._h = h

    def close(self):
        if self._h:
            lib().moe_gdn_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_layer(self, layer: int, conv_w, a_log, dt_bias, norm_w):
        arrs = [np.ascontiguousarray(x, dtype=np.float32) for x in (conv_w, a_log, dt_bias, norm_w)]
        _check(lib().moe_gdn_set_layer(self._h, layer, *[_ptr(x) for x in arrs]))

    def reset(self):
        _check(lib().moe_gdn_reset(self._h))

    def decode(self, first_layer: int, n_layers: int, qkv, z, a, b, out, n_tok: Optional[int] = None, stream=None):
        import torch
        n = qkv.shape[0] if n_tok is None else n_tok
        if n > 0:
            c = self.cfg
            bf = (torch.int16, torch.bfloat16)
            _check_dev("qkv", qkv, bf, n * n_layers * self.channels)
            _check_dev("z", z, bf, n * n_layers * c.n_v_heads * c.d_v)
            _check_dev("a", a, bf, n * n_layers * c.n_v_heads)
            _check_dev("b", b, bf, n * n_layers * c.n_v_heads)
            _check_dev("out", out, (torch.float32,), n * n_layers * c.n_v_heads * c.d_v)
        _check(lib().moe_gdn_decode(self._h, first_layer, n_layers, _ptr(qkv), _ptr(z), _ptr(a), _ptr(b), n,
                                    _ptr(out), _stream(stream)))

    def profile(self, enable: bool):
        """(total_ms, launches) recorded since the previous call; then record (or not) from now on."""
        ms = ctypes.c_double()
        n = ctypes.c_uint64()
        _check(lib().moe_gdn_profile(self._h, 1 if enable else 0, ctypes.byref(ms), ctypes.byref(n)))
        return ms.value, n.value

    def read_state(self, layer: int):
        c = self.cfg
        s = np.empty((c.n_v_heads, c.d_v, c.d_k), np.float32)
        w = np.empty((self.channels, 3), np.float32)
        _check(lib().moe_gdn_read_state(self._h, layer, _ptr(s), _ptr(w)))
        return s, w


class GatedAttention:
    """Gated grouped-query attention decode layers with an fp16 KV cache in HBM."""

    def __init__(self, n_layers: int, n_q_heads: int, n_kv_heads: int, head_dim: int, rot_dim: int, max_pos: int):
        self.cfg = AttnConfig(n_layers, n_q_heads, n_kv_heads, head_dim, rot_dim, max_pos)
        h = ctypes.c_void_p()
        _check(lib().moe_attn_create(ctypes.byref(self.cfg), ctypes.byref(h)))
        self._h = h

    def close(self):
        if self._h:
            lib().moe_attn_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_layer(self, layer: int, q_norm_w, k_norm_w):
        arrs = [np.ascontiguousarray(x, dtype=np.float32) for x in (q_norm_w, k_norm_w)]
        for x in arrs:
            if x.size != self.cfg.head_dim:
                raise ValueError(f"norm weights must hold head_dim = {self.cfg.head_dim} values")
        _check(lib().moe_attn_set_layer(self._h, layer, _ptr(arrs[0]), _ptr(arrs[1])))

    def write_cache(self, layer: int, first_pos: int, k16, v16):
        """k16, v16: fp16 bit patterns [n_kv_heads][n][head_dim] (uint16)."""
        k16 = np.ascontiguousarray(k16, dtype=np.uint16)
        v16 = np.ascontiguousarray(v16, dtype=np.uint16)
        c = self.cfg
        if k16.shape != v16.shape or k16.ndim != 3 or k16.shape[0] != c.n_kv_heads or k16.shape[2] != c.head_dim:
            raise ValueError("k16, v16 must both be [n_kv_heads][n][head_dim]")
        _check(lib().moe_attn_write_cache(self._h, layer, first_pos, k16.shape[1], _ptr(k16), _ptr(v16)))

    def read_cache(self, layer: int, first_pos: int, n: int):
        c = self.cfg
        k = np.empty((c.n_kv_heads, n, c.head_dim), np.uint16)
        v = np.empty_like(k)
        _check(lib().moe_attn_read_cache(self._h, layer, first_pos, n, _ptr(k), _ptr(v)))
        return k, v

    def decode(self, first_layer: int, n_layers: int, pos0: int, q, gate, k, v, out, n_tok: Optional[int] = None,
               stream=None):
        import torch
        n = q.shape[0] if n_tok is None else n_tok
        if n > 0:
            c = self.cfg
            bf = (torch.int16, torch.bfloat16)
            qd, kd = c.n_q_heads * c.head_dim, c.n_kv_heads * c.head_dim
            _check_dev("q", q, bf, n * n_layers * qd)
            _check_dev("gate", gate, bf, n * n_layers * qd)
            _check_dev("k", k, bf, n * n_layers * kd)
            _check_dev("v", v, bf, n * n_layers * kd)
            _check_dev("out", out, (torch.float32,), n * n_layers * qd)
        _check(lib().moe_attn_decode(self._h, first_layer, n_layers, pos0, _ptr(q), _ptr(gate), _ptr(k), _ptr(v), n,
                                     _ptr(out), _stream(stream)))

    def profile(self, enable: bool):
        """(split_ms, combine_ms, steps) recorded since the previous call; then record (or not) from now on."""
        ms_s, ms_c = ctypes.c_double(), ctypes.c_double()
        n = ctypes.c_uint64()
        _check(lib().moe_attn_profile(self._h, 1 if enable else 0, ctypes.byref(ms_s), ctypes.byref(ms_c),
                                      ctypes.byref(n)))
        return ms_s.value, ms_c.value, n.value
