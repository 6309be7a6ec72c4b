"""Python binding of libexmoe, the fused grouped W4A16 MoE expert layer for MI355X.

Argument marshalling only: tensors are passed to the C ABI as device pointers with
torch's current HIP stream; every step of the layer runs in the library's HIP kernels
(host C++ for the offline packer and the slot-cache policy). PyTorch provides device
memory and streams. Importing this package fails loudly if libexmoe.so is not built.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libexmoe.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libexmoe.so is not built ({LIB_PATH}); run python w4a16_mixture_experts_amd/build_lib.py")
# torch ships its own HIP runtime under the SONAME libamdhip64.so.7 but links it by the
# name libamdhip64.so. Loading torch first makes this library bind to that same runtime;
# loaded the other way round, the process would hold two HIP runtimes, and a kernel
# launched from one does not see the device the other initialised.
try:
    import torch  # noqa: F401
except ImportError:
    pass
_lib = ctypes.CDLL(LIB_PATH)

# status codes (exmoe.h)
OK = 0
ERR_INVALID_ARGUMENT = -1
ERR_UNSUPPORTED = -2
ERR_WORKSPACE = -3
ERR_HIP = -4
ERR_OUT_OF_MEMORY = -5
ERR_CACHE = -6

PATH_AUTO, PATH_DECODE, PATH_PREFILL, PATH_SEQUENTIAL = 0, 1, 2, 3
WEIGHTS_BF16 = 0x100       # flag: the bank holds dense bf16 experts (bf16_pack)
DEBUG_COUNTERS = 0x200     # flag: expert kernels count the rows they ran per expert (workspace_rows)
CACHE_DRY_RUN = 1

_vp = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t


class ExpertBankC(ctypes.Structure):
    _fields_ = [("base", _vp), ("stride", _sz), ("expert_to_slot", _vp)]


class CacheStatsC(ctypes.Structure):
    _fields_ = [("lookups", ctypes.c_uint64), ("hits", ctypes.c_uint64), ("misses", ctypes.c_uint64),
                ("evictions", ctypes.c_uint64), ("h2d_bytes", ctypes.c_uint64), ("h2d_copies", ctypes.c_uint64),
                ("device_bytes", ctypes.c_uint64), ("pinned_host_bytes", ctypes.c_uint64), ("resident", _i)]


_SIGS = {
    "exmoe_status_string": (ctypes.c_char_p, [_i]),
    "exmoe_last_error": (ctypes.c_char_p, []),
    "exmoe_abi_version": (_i, []),
    "exmoe_packed_expert_bytes": (_sz, [_i, _i]),
    "exmoe_quantize_pack": (_i, [_vp, _vp, _vp, _i, _i, _i, _vp, _sz]),
    "exmoe_unpack_expert": (_i, [_vp, _sz, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp]),
    "exmoe_route_topk": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp]),
    "exmoe_topk_from_logits": (_i, [_vp, _i, _i, _i, _i, _vp, _vp, _vp]),
    "exmoe_route_weights": (_i, [_vp, _vp, _i, _i, _i, _i, _vp, _vp]),
    "exmoe_group_workspace_bytes": (_sz, [_i, _i, _i]),
    "exmoe_group_tokens": (_i, [_vp, _i, _i, _i, _vp, _vp, _vp, _vp, _sz, _vp]),
    "exmoe_active_experts": (_i, [_vp, _i, _vp, _vp, _vp]),
    "exmoe_moe_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "exmoe_bf16_expert_bytes": (_sz, [_i, _i]),
    "exmoe_workspace_flags": (_i, [_vp, _sz, _i, ctypes.POINTER(ctypes.c_uint32), _vp]),
    "exmoe_workspace_rows": (_i, [_vp, _sz, _i, _i, _vp, _vp]),
    "exmoe_bf16_pack": (_i, [_vp, _vp, _vp, _i, _i, _vp, _sz]),
    "exmoe_moe_forward": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, ctypes.POINTER(ExpertBankC), _i, _i, _i, _i, _i, _i,
                               _vp, _vp, _sz, _vp]),
    "exmoe_moe_forward_cached": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _i, _i, _i, _i, _i, _i, _i,
                                      _vp, _vp, _sz, _vp]),
    "exmoe_moe_layer_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "exmoe_moe_layer": (_i, [_vp, _vp, _vp, ctypes.POINTER(ExpertBankC), _i, _i, _i, _i, _i, _i, _i,
                             _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "exmoe_moe_layer_noalloc": (_i, [_vp, _vp, _vp, ctypes.POINTER(ExpertBankC), _i, _i, _i, _i, _i, _i, _i,
                                     _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "exmoe_slot_cache_create": (_i, [_i, _i, _i, _sz, _i, ctypes.POINTER(_vp)]),
    "exmoe_slot_cache_host_slot": (_i, [_vp, _i, _i, ctypes.POINTER(_vp)]),
    "exmoe_slot_cache_preload": (_i, [_vp, _vp]),
    "exmoe_slot_cache_acquire": (_i, [_vp, _i, _vp, _i, _vp, ctypes.POINTER(ExpertBankC)]),
    "exmoe_slot_cache_table": (_i, [_vp, _i, _vp]),
    "exmoe_slot_cache_waves": (_i, [_vp, _i, _vp, _i, _i, _vp, ctypes.POINTER(_i), ctypes.POINTER(_i)]),
    "exmoe_slot_cache_stats": (_i, [_vp, ctypes.POINTER(CacheStatsC)]),
    "exmoe_slot_cache_reset_stats": (_i, [_vp]),
    "exmoe_slot_cache_destroy": (_i, [_vp]),
    "exmoe_profile_enable": (_i, [_i]),
    "exmoe_profile_reset": (_i, []),
    "exmoe_profile_read": (_i, [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_uint64)]),
    "exmoe_span_enable": (_i, [_i]),
    "exmoe_span_clear": (_i, []),
    "exmoe_span_read": (_i, [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_uint64)]),
    "exmoe_device_copy": (_i, [_vp, _vp, _sz, _vp]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTED = tuple(_SIGS)


class ExmoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_lib.exmoe_status_string(status).decode()} ({status}): {msg}")
        self.status = status


def _check(status: int):
    if status != OK:
        raise ExmoeError(status, _lib.exmoe_last_error().decode())


def last_error() -> str:
    return _lib.exmoe_last_error().decode()


def abi_version() -> int:
    return _lib.exmoe_abi_version()


def packed_expert_bytes(H: int, I: int) -> int:
    return _lib.exmoe_packed_expert_bytes(H, I)


# ----------------------------------------------------------------------------- host packer
def bf16_expert_bytes(H: int, I: int) -> int:
    return _lib.exmoe_bf16_expert_bytes(H, I)


def bf16_pack(g_bits: np.ndarray, u_bits: np.ndarray, d_bits: np.ndarray) -> np.ndarray:
    """bf16 bits gate [I,H], up [I,H], down [H,I] (uint16) -> dense bf16 blob (uint8 numpy)."""
    g = np.ascontiguousarray(g_bits, dtype=np.uint16)
    u = np.ascontiguousarray(u_bits, dtype=np.uint16)
    d = np.ascontiguousarray(d_bits, dtype=np.uint16)
    I, H = g.shape
    if u.shape != (I, H) or d.shape != (H, I):
        raise ValueError("shape mismatch: gate/up [I,H], down [H,I]")
    nb = bf16_expert_bytes(H, I)
    out = np.empty(nb, dtype=np.uint8)
    _check(_lib.exmoe_bf16_pack(g.ctypes.data, u.ctypes.data, d.ctypes.data, H, I, out.ctypes.data, nb))
    return out


def quantize_pack(w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray, out: Optional[np.ndarray] = None,
                  out_ptr: Optional[int] = None) -> np.ndarray:
    """fp32 gate [I,H], up [I,H], down [H,I] -> packed blob (uint8 numpy, or written to out_ptr)."""
    g = np.ascontiguousarray(w_gate, dtype=np.float32)
    u = np.ascontiguousarray(w_up, dtype=np.float32)
    d = np.ascontiguousarray(w_down, dtype=np.float32)
    I, H = g.shape
    if u.shape != (I, H) or d.shape != (H, I):
        raise ValueError("shape mismatch: gate/up [I,H], down [H,I]")
    nb = packed_expert_bytes(H, I)
    if out_ptr is None:
        if out is None:
            out = np.empty(nb, dtype=np.uint8)
        ptr = out.ctypes.data
        size = out.nbytes
    else:
        ptr, size = out_ptr, nb
    _check(_lib.exmoe_quantize_pack(g.ctypes.data, u.ctypes.data, d.ctypes.data, H, I, 128, ptr, size))
    return out


def unpack_expert(blob: np.ndarray, H: int, I: int):
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    qg = np.empty((I, H), np.int8); qu = np.empty((I, H), np.int8); qd = np.empty((H, I), np.int8)
    sg = np.empty((I, H // 128), np.uint16); su = np.empty_like(sg); sd = np.empty((H, I // 128), np.uint16)
    _check(_lib.exmoe_unpack_expert(blob.ctypes.data, blob.nbytes, H, I, qg.ctypes.data, qu.ctypes.data,
                                    qd.ctypes.data, sg.ctypes.data, su.ctypes.data, sd.ctypes.data))
    return qg, sg, qu, su, qd, sd


# ----------------------------------------------------------------------------- device calls
def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return _torch().cuda.current_stream().cuda_stream


def route_topk(x, w_router, k: int, bias=None, renormalize: bool = True, logits=None, ids=None, weights=None):
    """x bf16 [T,H], w_router bf16 [E,H], bias fp32 [E] -> (logits bf16 [T,E], ids int32 [T,k], weights fp32 [T,k])."""
    torch = _torch()
    T, H = x.shape
    E = w_router.shape[0]
    dev = x.device
    logits = torch.empty((T, E), dtype=torch.bfloat16, device=dev) if logits is None else logits
    ids = torch.empty((T, k), dtype=torch.int32, device=dev) if ids is None else ids
    weights = torch.empty((T, k), dtype=torch.float32, device=dev) if weights is None else weights
    _check(_lib.exmoe_route_topk(_ptr(x), _ptr(w_router), _ptr(bias), T, H, E, k, int(renormalize), _ptr(logits),
                                 _ptr(ids), _ptr(weights), _stream()))
    return logits, ids, weights


def topk_from_logits(logits, k: int, renormalize: bool = True):
    torch = _torch()
    T, E = logits.shape
    ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    weights = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _check(_lib.exmoe_topk_from_logits(_ptr(logits), T, E, k, int(renormalize), _ptr(ids), _ptr(weights), _stream()))
    return ids, weights


def route_weights(logits, ids, renormalize: bool = True, weights=None):
    torch = _torch()
    T, E = logits.shape
    k = ids.shape[1]
    weights = torch.empty((T, k), dtype=torch.float32, device=logits.device) if weights is None else weights
    _check(_lib.exmoe_route_weights(_ptr(logits), _ptr(ids), T, E, k, int(renormalize), _ptr(weights), _stream()))
    return weights


def group_tokens(ids, E: int, offsets=None, sorted_flat=None, flat_to_sorted=None):
    torch = _torch()
    T, k = ids.shape
    dev = ids.device
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev) if offsets is None else offsets
    sorted_flat = torch.empty(T * k, dtype=torch.int32, device=dev) if sorted_flat is None else sorted_flat
    flat_to_sorted = torch.empty(T * k, dtype=torch.int32, device=dev) if flat_to_sorted is None else flat_to_sorted
    nws = _lib.exmoe_group_workspace_bytes(T, k, E)
    ws = torch.empty(max(nws, 4), dtype=torch.uint8, device=dev) if nws else None
    _check(_lib.exmoe_group_tokens(_ptr(ids), T, k, E, _ptr(offsets), _ptr(sorted_flat), _ptr(flat_to_sorted),
                                   _ptr(ws) if ws is not None else None, nws, _stream()))
    return offsets, sorted_flat, flat_to_sorted


def active_experts(offsets) -> list[int]:
    E = offsets.numel() - 1
    buf = (ctypes.c_int32 * E)()
    n = ctypes.c_int(0)
    _check(_lib.exmoe_active_experts(_ptr(offsets), E, ctypes.cast(buf, _vp), ctypes.byref(n), _stream()))
    return [buf[i] for i in range(n.value)]


@dataclass
class ExpertBank:
    """Packed experts in device memory: expert e's blob at base + stride * slot(e)."""
    base: object                 # torch uint8 tensor (kept alive) or raw int pointer
    stride: int
    expert_to_slot: object = None   # torch int32 [E] or None
    base_ptr: Optional[int] = None

    def c(self) -> ExpertBankC:
        base = self.base_ptr if self.base_ptr is not None else self.base.data_ptr()
        e2s = None if self.expert_to_slot is None else (
            self.expert_to_slot if isinstance(self.expert_to_slot, int) else self.expert_to_slot.data_ptr())
        return ExpertBankC(base, self.stride, e2s)


def bank_from_blobs(blobs, device="cuda") -> ExpertBank:
    """Upload a list of packed blobs (numpy uint8) into one device bank, stride rounded to 256 B."""
    torch = _torch()
    nb = blobs[0].nbytes
    stride = (nb + 255) // 256 * 256
    host = np.zeros((len(blobs), stride), dtype=np.uint8)
    for i, b in enumerate(blobs):
        host[i, :nb] = b
    dev = torch.from_numpy(host.reshape(-1)).to(device)
    return ExpertBank(base=dev, stride=stride)


def moe_workspace_bytes(T, H, I, E, k, flags=PATH_AUTO) -> int:
    return _lib.exmoe_moe_workspace_bytes(T, H, I, E, k, flags)


def alloc_workspace(nbytes: int, device="cuda"):
    """Zero-filled workspace: the layer call keeps arrival counters, zero between calls,
    in its first 4096 bytes."""
    torch = _torch()
    return torch.zeros(max(nbytes, 4096), dtype=torch.uint8, device=device)


FLAG_EXPERT_WITHOUT_SLOT = 1
FLAG_ROWS_UNGROUPED = 2


def workspace_flags(workspace, clear: bool = True) -> int:
    """Conditions the expert kernels recorded in a workspace (bit 0: a routed expert had no
    slot); synchronizes the current stream."""
    v = ctypes.c_uint32(0)
    _check(_lib.exmoe_workspace_flags(_ptr(workspace), workspace.numel(), int(clear), ctypes.byref(v), _stream()))
    return v.value


def workspace_rows(workspace, E: int, clear: bool = True) -> np.ndarray:
    """Per-expert counters of routed rows run since the last clear (DEBUG_COUNTERS calls);
    synchronizes the current stream."""
    out = np.empty(E, dtype=np.int32)
    _check(_lib.exmoe_workspace_rows(_ptr(workspace), workspace.numel(), E, int(clear), out.ctypes.data, _stream()))
    return out


def moe_forward(x, ids, weights, offsets, sorted_flat, flat_to_sorted, bank: ExpertBank, I: int,
                flags: int = PATH_AUTO, y=None, workspace=None):
    torch = _torch()
    T, H = x.shape
    k = ids.shape[1]
    E = offsets.numel() - 1
    y = torch.empty((T, H), dtype=torch.bfloat16, device=x.device) if y is None else y
    need = moe_workspace_bytes(T, H, I, E, k, flags)
    workspace = alloc_workspace(need, x.device) if workspace is None else workspace
    bc = bank.c()
    _check(_lib.exmoe_moe_forward(_ptr(x), _ptr(ids), _ptr(weights), _ptr(offsets), _ptr(sorted_flat),
                                  _ptr(flat_to_sorted), ctypes.byref(bc), T, H, I, E, k, flags, _ptr(y),
                                  _ptr(workspace), workspace.numel(), _stream()))
    return y


class LayerBuffers:
    """Preallocated outputs and workspace of one layer call (no allocation per call)."""

    def __init__(self, T, H, I, E, k, flags=PATH_AUTO, device="cuda"):
        torch = _torch()
        self.T, self.H, self.I, self.E, self.k, self.flags = T, H, I, E, k, flags
        self.logits = torch.empty((T, E), dtype=torch.bfloat16, device=device)
        self.ids = torch.empty((T, k), dtype=torch.int32, device=device)
        self.weights = torch.empty((T, k), dtype=torch.float32, device=device)
        self.offsets = torch.empty(E + 1, dtype=torch.int32, device=device)
        self.sorted_flat = torch.empty(max(T * k, 1), dtype=torch.int32, device=device)
        self.flat_to_sorted = torch.empty(max(T * k, 1), dtype=torch.int32, device=device)
        self.y = torch.empty((T, H), dtype=torch.bfloat16, device=device)
        self.workspace = alloc_workspace(_lib.exmoe_moe_layer_workspace_bytes(T, H, I, E, k, flags), device)


def moe_layer(x, w_router, bank: ExpertBank, I: int, k: int, bias=None, renormalize: bool = True,
              flags: int = PATH_AUTO, buffers: Optional[LayerBuffers] = None, stream: Optional[int] = None):
    """route + group + experts in one call; returns the LayerBuffers holding every output."""
    T, H = x.shape
    E = w_router.shape[0]
    b = buffers or LayerBuffers(T, H, I, E, k, flags, x.device)
    bc = bank.c()
    _check(_lib.exmoe_moe_layer(_ptr(x), _ptr(w_router), _ptr(bias), ctypes.byref(bc), T, H, I, E, k,
                                int(renormalize), flags, _ptr(b.logits), _ptr(b.ids), _ptr(b.weights), _ptr(b.offsets),
                                _ptr(b.sorted_flat), _ptr(b.flat_to_sorted), _ptr(b.y), _ptr(b.workspace),
                                b.workspace.numel(), _stream() if stream is None else stream))
    return b


def moe_layer_noalloc(x, w_router, bank: ExpertBank, I: int, k: int, buffers: LayerBuffers, bias=None,
                      renormalize: bool = True, flags: int = PATH_AUTO):
    """moe_layer without a workspace (the library's fixed per-GPU array serves as one):
    every output goes to the preallocated `buffers` (its workspace is not used)."""
    T, H = x.shape
    E = w_router.shape[0]
    b = buffers
    bc = bank.c()
    _check(_lib.exmoe_moe_layer_noalloc(_ptr(x), _ptr(w_router), _ptr(bias), ctypes.byref(bc), T, H, I, E, k,
                                        int(renormalize), flags, _ptr(b.logits), _ptr(b.ids), _ptr(b.weights),
                                        _ptr(b.offsets), _ptr(b.sorted_flat), _ptr(b.flat_to_sorted), _ptr(b.y),
                                        _stream()))
    return b


# ----------------------------------------------------------------------------- slot cache
def moe_forward_cached(x, ids, weights, offsets, sorted_flat, flat_to_sorted, cache: "SlotCache", layer: int,
                       active, I: int, flags: int = PATH_AUTO, y=None, workspace=None):
    """Expert layer through a slot cache in cache-sized waves (active: every routed expert id)."""
    torch = _torch()
    T, H = x.shape
    k = ids.shape[1]
    E = offsets.numel() - 1
    y = torch.empty((T, H), dtype=torch.bfloat16, device=x.device) if y is None else y
    need = moe_workspace_bytes(T, H, I, E, k, flags)
    workspace = alloc_workspace(need, x.device) if workspace is None else workspace
    arr = (ctypes.c_int32 * max(len(active), 1))(*[int(e) for e in active])
    _check(_lib.exmoe_moe_forward_cached(_ptr(x), _ptr(ids), _ptr(weights), _ptr(offsets), _ptr(sorted_flat),
                                         _ptr(flat_to_sorted), cache._h, layer, ctypes.cast(arr, _vp), len(active),
                                         T, H, I, E, k, flags, _ptr(y), _ptr(workspace), workspace.numel(),
                                         _stream()))
    return y


class SlotCache:
    """GPU slot cache over a pinned host pool (policy in C++, copies on a side stream)."""

    def __init__(self, layers: int, E: int, slots: int, expert_bytes: int, dry_run: bool = False):
        h = _vp()
        _check(_lib.exmoe_slot_cache_create(layers, E, slots, expert_bytes, CACHE_DRY_RUN if dry_run else 0,
                                            ctypes.byref(h)))
        self._h = h
        self.dry_run = dry_run
        self.layers, self.E, self.slots, self.expert_bytes = layers, E, slots, expert_bytes

    def host_slot(self, layer: int, expert: int) -> int:
        p = _vp()
        _check(_lib.exmoe_slot_cache_host_slot(self._h, layer, expert, ctypes.byref(p)))
        return p.value

    def fill(self, layer: int, expert: int, blob: np.ndarray):
        ctypes.memmove(self.host_slot(layer, expert), blob.ctypes.data, blob.nbytes)

    def preload(self):
        _check(_lib.exmoe_slot_cache_preload(self._h, _stream()))

    def acquire(self, layer: int, active) -> ExpertBank:
        arr = (ctypes.c_int32 * max(len(active), 1))(*[int(e) for e in active])
        bc = ExpertBankC()
        _check(_lib.exmoe_slot_cache_acquire(self._h, layer, ctypes.cast(arr, _vp), len(active),
                                             None if self.dry_run else _stream(), ctypes.byref(bc)))
        return ExpertBank(base=None, stride=bc.stride, expert_to_slot=bc.expert_to_slot, base_ptr=bc.base)

    def waves(self, layer: int, active, run: bool = False):
        """The cache-sized waves a cached forward on `layer` would run: list of id lists.
        run=True (dry-run caches only) also looks the waves up, as that forward does."""
        arr = (ctypes.c_int32 * max(len(active), 1))(*[int(e) for e in active])
        order = np.empty(max(len(active), 1), dtype=np.int32)
        n, w = _i(0), _i(0)
        _check(_lib.exmoe_slot_cache_waves(self._h, layer, ctypes.cast(arr, _vp), len(active), int(run),
                                           order.ctypes.data, ctypes.byref(n), ctypes.byref(w)))
        ids = order[:n.value].tolist()
        return [ids[i:i + w.value] for i in range(0, len(ids), w.value)] if ids else []

    def table(self, layer: int) -> np.ndarray:
        out = np.empty(self.E, dtype=np.int32)
        _check(_lib.exmoe_slot_cache_table(self._h, layer, out.ctypes.data))
        return out

    def stats(self) -> dict:
        s = CacheStatsC()
        _check(_lib.exmoe_slot_cache_stats(self._h, ctypes.byref(s)))
        return {f: getattr(s, f) for f, _ in CacheStatsC._fields_}

    def reset_stats(self):
        _check(_lib.exmoe_slot_cache_reset_stats(self._h))

    def close(self):
        if self._h:
            _check(_lib.exmoe_slot_cache_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ----------------------------------------------------------------------------- kernel timing
def profile_enable(on: bool = True):
    _check(_lib.exmoe_profile_enable(int(on)))


def profile_reset():
    _check(_lib.exmoe_profile_reset())


def profile_read(kernel: str):
    """(total milliseconds, launches) of one library kernel since the last reset."""
    ms = ctypes.c_double(0.0)
    n = ctypes.c_uint64(0)
    _check(_lib.exmoe_profile_read(kernel.encode(), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def span_enable(max_launches: int):
    """Launch span stamps for the next `max_launches` expert-layer kernel launches (0: off)."""
    _check(_lib.exmoe_span_enable(int(max_launches)))


def span_clear():
    """Reset the span stamps, keeping the slots' assignment (replay a graph, then read)."""
    _check(_lib.exmoe_span_clear())


def span_read(kernel: str):
    """(total microseconds, launches) of one kernel's spans since the last clear."""
    us = ctypes.c_double(0.0)
    n = ctypes.c_uint64(0)
    _check(_lib.exmoe_span_read(kernel.encode(), ctypes.byref(us), ctypes.byref(n)))
    return us.value, n.value


def device_copy(dst, src):
    """Plain device copy of src into dst (same byte size, multiple of 16) on the current stream."""
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n:
        raise ValueError("device_copy: size mismatch")
    _check(_lib.exmoe_device_copy(_vp(dst.data_ptr()), _vp(src.data_ptr()), n, _stream()))
