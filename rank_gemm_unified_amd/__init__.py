"""Python binding of liblorapool: the unmerged multi-LoRA projection over a unified page pool.

The functions below carry the C-ABI's names and only marshal arguments (torch tensors become their
device addresses, streams their hipStream_t handles); every step of the projection runs in the
library's HIP kernels.  Importing this package fails loudly when the library has not been built or
was built from sources other than the ones beside it.

``Pool`` is a convenience owner of the device buffers a pool needs (pages and page table),
allocated with torch; torch is used for device memory and streams only.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblorapool.so")

LORA_OK, LORA_EINVAL, LORA_ENOMEM, LORA_ENOENT = 0, -1, -2, -3
LORA_ERANK, LORA_EBUSY, LORA_EEXIST, LORA_EHIP, LORA_EDEVICE = -4, -5, -6, -7, -8
LORA_F32, LORA_BF16 = 0, 1
LORA_MAX_RANK, LORA_MAX_ADAPTERS, LORA_MAX_TOKENS = 64, 8192, 1 << 22
LORA_VICTIM_LOAD_ORDER, LORA_VICTIM_LRU, LORA_VICTIM_FARTHEST = 0, 1, 2
LORA_MAX_CALL_SLOTS = 4
LORA_NOALLOC_SCRATCH_MB = 32
STATUS_NAMES = {0: "ok", -1: "einval", -2: "enomem", -3: "enoent", -4: "erank", -5: "ebusy",
                -6: "eexist", -7: "ehip", -8: "edevice"}

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it first (python rank_gemm_unified_amd/build.py "
                      "or __graft_entry__.build()); there is no fallback path")
# torch ships its own HIP runtime under the same soname as /opt/rocm's.  Whichever is loaded first
# serves the whole process, and a process that loads this library before torch ends up with two
# halves of different runtimes that see no device.  Load torch's first.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_P64 = ctypes.POINTER(ctypes.c_int64)
_P32 = ctypes.POINTER(ctypes.c_int32)


class lora_pool_stats_t(ctypes.Structure):
    _fields_ = [("num_pages", _i64), ("free_pages", _i64), ("kv_pages", _i64), ("adapter_pages", _i64),
                ("resident_adapters", _i32), ("idle_adapters", _i32), ("kv_requests", _i64),
                ("loads", _i64), ("evictions", _i64), ("bytes_loaded", _i64)]


class lora_profile_t(ctypes.Structure):
    _fields_ = [("calls", _i64), ("ms_group", ctypes.c_double), ("ms_first", ctypes.c_double),
                ("ms_second", ctypes.c_double)]


_SIGS = {
    "lora_pool_create": (ctypes.c_int, [_vp, _i64, _i32, _i32, _i32, _i32, _i32, _vp, _vp, ctypes.POINTER(_vp)]),
    "lora_pool_free": (ctypes.c_int, [_vp]),
    "lora_pool_load_adapter": (ctypes.c_int, [_vp, _i32, _i32, _vp, _vp, _vp]),
    "lora_pool_release_adapter": (ctypes.c_int, [_vp, _i32]),
    "lora_pool_set_victim_rule": (ctypes.c_int, [_vp, _i32]),
    "lora_pool_set_lookahead": (ctypes.c_int, [_vp, _vp, _i64]),
    "lora_pool_evict_adapter": (ctypes.c_int, [_vp, _i32, _vp]),
    "lora_pool_grow_kv": (ctypes.c_int, [_vp, _i64, _i32, _vp]),
    "lora_pool_free_kv": (ctypes.c_int, [_vp, _i64]),
    "lora_pool_pages_for": (_i64, [_i32, _i32, _i32]),
    "lora_kv_pages_per_token": (_i64, [_i32]),
    "lora_pool_stats": (ctypes.c_int, [_vp, ctypes.POINTER(lora_pool_stats_t)]),
    "lora_pool_page_table": (ctypes.c_int, [_vp, _i32, ctypes.POINTER(_vp), _P32]),
    "lora_pool_adapter_pages": (ctypes.c_int, [_vp, _i32, _vp, _i64, _P64, _P32, _P32]),
    "lora_pool_kv_pages": (ctypes.c_int, [_vp, _i64, _vp, _i64, _P64]),
    "lora_pool_free_list": (ctypes.c_int, [_vp, _vp, _i64, _P64]),
    "lora_pool_resident": (ctypes.c_int, [_vp, _vp, _i32, _P32]),
    "lora_project_workspace_size": (_sz, [_vp, _i64]),
    "lora_project_slots_workspace_size": (_sz, [_vp, _i32, _i64]),
    "lora_project_slots": (ctypes.c_int, [_vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _sz, _vp]),
    "lora_project_slots_x": (ctypes.c_int, [_vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _sz, _vp]),
    "lora_project": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _sz, _vp]),
    "lora_debug_gather": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _vp, _vp]),
    "lora_debug_project": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _sz, _vp, _vp, _vp]),
    "lora_project_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp]),
    "lora_check_device_errors": (ctypes.c_int, [_vp]),
    "lora_profile_start": (ctypes.c_int, [_vp, _i32]),
    "lora_profile_stop": (ctypes.c_int, [_vp, ctypes.POINTER(lora_profile_t)]),
    "lora_last_error": (ctypes.c_char_p, []),
    "lora_version": (ctypes.c_char_p, []),
}
for _name, (_res, _args) in _SIGS.items():
    try:
        _f = getattr(_lib, _name)
    except AttributeError as _e:
        raise ImportError(f"{LIB_PATH} lacks {_name}: it is stale, rebuild it "
                          "(python rank_gemm_unified_amd/build.py)") from _e
    _f.restype, _f.argtypes = _res, _args

EXPORTED = tuple(_SIGS)

# The library carries the hash of the sources it was built from; refuse one built from other sources
# (a stale build whose exports happen to match would otherwise load silently).
from ._srchash import source_hash as _source_hash  # noqa: E402

SOURCE_HASH = _source_hash()
_built = _lib.lora_version().decode()
if SOURCE_HASH is not None and not _built.endswith(" src " + SOURCE_HASH):
    raise ImportError(f"{LIB_PATH} ({_built}) was not built from the sources beside it (hash {SOURCE_HASH}): "
                      "it is stale, rebuild it (python rank_gemm_unified_amd/build.py)")


class LoraError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        self.status = STATUS_NAMES.get(code, str(code))
        msg = _lib.lora_last_error().decode(errors="replace")
        super().__init__(f"{where}: {self.status} ({code}): {msg}")


def _check(rc: int, where: str) -> int:
    if rc != LORA_OK:
        raise LoraError(rc, where)
    return rc


def _ptr(t) -> int | None:
    """Device/host address of a tensor or array (None stays NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _stream(s) -> int | None:
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(s, int):
        return s
    return s.cuda_stream


# ---- C-ABI, one wrapper per entry point ----------------------------------------------------------

def lora_pool_create(pages, num_pages, hidden, dtype, max_rank, n_slots, max_adapters, page_table,
                     free_order=None):
    fo = None
    if free_order is not None:
        fo = np.ascontiguousarray(free_order, dtype=np.int64)
    out = _vp()
    _check(_lib.lora_pool_create(_ptr(pages), num_pages, hidden, dtype, max_rank, n_slots, max_adapters,
                                 _ptr(page_table), None if fo is None else fo.ctypes.data, ctypes.byref(out)),
           "lora_pool_create")
    return out.value


def lora_pool_free(pool):
    return _check(_lib.lora_pool_free(pool), "lora_pool_free")


def lora_pool_load_adapter(pool, adapter_id, rank, A_t, B, stream=None, check=True):
    rc = _lib.lora_pool_load_adapter(pool, adapter_id, rank, _ptr(A_t), _ptr(B), _stream(stream))
    return _check(rc, "lora_pool_load_adapter") if check else rc


def lora_pool_set_victim_rule(pool, rule, check=True):
    rc = _lib.lora_pool_set_victim_rule(pool, rule)
    return _check(rc, "lora_pool_set_victim_rule") if check else rc


def lora_pool_set_lookahead(pool, adapter_ids, check=True):
    ids = np.ascontiguousarray(adapter_ids, dtype=np.int32)
    rc = _lib.lora_pool_set_lookahead(pool, ids.ctypes.data if ids.size else None, ids.size)
    return _check(rc, "lora_pool_set_lookahead") if check else rc


def lora_pool_release_adapter(pool, adapter_id, check=True):
    rc = _lib.lora_pool_release_adapter(pool, adapter_id)
    return _check(rc, "lora_pool_release_adapter") if check else rc


def lora_pool_evict_adapter(pool, adapter_id, stream=None, check=True):
    rc = _lib.lora_pool_evict_adapter(pool, adapter_id, _stream(stream))
    return _check(rc, "lora_pool_evict_adapter") if check else rc


def lora_pool_grow_kv(pool, request_id, layers, check=True):
    """Returns the new KV page ids (list), or the status code when check=False and it failed."""
    out = np.zeros(max(2 * layers, 1), np.int64)
    rc = _lib.lora_pool_grow_kv(pool, request_id, layers, out.ctypes.data)
    if rc != LORA_OK:
        return _check(rc, "lora_pool_grow_kv") if check else rc
    return out[: 2 * layers].tolist()


def lora_pool_free_kv(pool, request_id, check=True):
    rc = _lib.lora_pool_free_kv(pool, request_id)
    return _check(rc, "lora_pool_free_kv") if check else rc


def lora_pool_pages_for(rank, projections, layers):
    return _lib.lora_pool_pages_for(rank, projections, layers)


def lora_kv_pages_per_token(layers):
    return _lib.lora_kv_pages_per_token(layers)


def lora_pool_stats(pool) -> dict:
    st = lora_pool_stats_t()
    _check(_lib.lora_pool_stats(pool, ctypes.byref(st)), "lora_pool_stats")
    return {name: getattr(st, name) for name, _ in st._fields_}


def lora_pool_page_table(pool, slot):
    ptr, stride = _vp(), _i32()
    _check(_lib.lora_pool_page_table(pool, slot, ctypes.byref(ptr), ctypes.byref(stride)), "lora_pool_page_table")
    return ptr.value, stride.value


def lora_pool_adapter_pages(pool, adapter_id):
    n, rank, users = _i64(), _i32(), _i32()
    rc = _lib.lora_pool_adapter_pages(pool, adapter_id, None, 0, ctypes.byref(n), ctypes.byref(rank),
                                      ctypes.byref(users))
    if rc == LORA_ENOENT:
        raise LoraError(rc, "lora_pool_adapter_pages")
    out = np.zeros(max(n.value, 1), np.int64)
    _check(_lib.lora_pool_adapter_pages(pool, adapter_id, out.ctypes.data, n.value, ctypes.byref(n),
                                        ctypes.byref(rank), ctypes.byref(users)), "lora_pool_adapter_pages")
    return out[: n.value].tolist(), rank.value, users.value


def lora_pool_kv_pages(pool, request_id):
    n = _i64()
    rc = _lib.lora_pool_kv_pages(pool, request_id, None, 0, ctypes.byref(n))
    if rc == LORA_ENOENT:
        raise LoraError(rc, "lora_pool_kv_pages")
    out = np.zeros(max(n.value, 1), np.int64)
    _check(_lib.lora_pool_kv_pages(pool, request_id, out.ctypes.data, n.value, ctypes.byref(n)), "lora_pool_kv_pages")
    return out[: n.value].tolist()


def lora_pool_free_list(pool):
    n = _i64()
    _lib.lora_pool_free_list(pool, None, 0, ctypes.byref(n))
    out = np.zeros(max(n.value, 1), np.int64)
    _check(_lib.lora_pool_free_list(pool, out.ctypes.data, n.value, ctypes.byref(n)), "lora_pool_free_list")
    return out[: n.value].tolist()


def lora_pool_resident(pool):
    n = _i32()
    _lib.lora_pool_resident(pool, None, 0, ctypes.byref(n))
    out = np.zeros(max(n.value, 1), np.int32)
    _check(_lib.lora_pool_resident(pool, out.ctypes.data, n.value, ctypes.byref(n)), "lora_pool_resident")
    return out[: n.value].tolist()


def lora_project_workspace_size(pool, T):
    return _lib.lora_project_workspace_size(pool, T)


def lora_project(pool, x, W, page_table, adapter_ids, ranks, scale, T, y, workspace, workspace_bytes=None,
                 stream=None, check=True):
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    rc = _lib.lora_project(pool, _ptr(x), _ptr(W), _ptr(page_table), _ptr(adapter_ids), _ptr(ranks), _ptr(scale),
                           T, _ptr(y), _ptr(workspace), workspace_bytes, _stream(stream))
    return _check(rc, "lora_project") if check else rc


def lora_project_slots_workspace_size(pool, n, T):
    return _lib.lora_project_slots_workspace_size(pool, n, T)


def lora_project_slots(pool, slots, x, Ws, adapter_ids, ranks, scale, T, ys, workspace, workspace_bytes=None,
                       stream=None, check=True):
    """slots: sequence of slot indices; Ws, ys: sequences of tensors (or addresses), one per slot."""
    n = len(slots)
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    sl = np.ascontiguousarray(slots, dtype=np.int32)
    wp = (ctypes.c_void_p * max(n, 1))(*[_ptr(w) for w in Ws])
    yp = (ctypes.c_void_p * max(n, 1))(*[_ptr(y) for y in ys])
    rc = _lib.lora_project_slots(pool, n, sl.ctypes.data, _ptr(x), ctypes.cast(wp, ctypes.c_void_p),
                                 _ptr(adapter_ids), _ptr(ranks), _ptr(scale), T, ctypes.cast(yp, ctypes.c_void_p),
                                 _ptr(workspace), workspace_bytes, _stream(stream))
    return _check(rc, "lora_project_slots") if check else rc


def lora_debug_gather(pool, page_table, adapter_ids, ranks, T, out, stream=None, check=True):
    rc = _lib.lora_debug_gather(pool, _ptr(page_table), _ptr(adapter_ids), _ptr(ranks), T, _ptr(out),
                                _stream(stream))
    return _check(rc, "lora_debug_gather") if check else rc


def lora_project_slots_x(pool, slots, xs, Ws, adapter_ids, ranks, scale, T, ys, workspace, workspace_bytes=None,
                         stream=None, check=True):
    """slots: sequence of slot indices; xs, Ws, ys: sequences of tensors (or addresses), one per slot."""
    n = len(slots)
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    sl = np.ascontiguousarray(slots, dtype=np.int32)
    xp = (ctypes.c_void_p * max(n, 1))(*[_ptr(x) for x in xs])
    wp = (ctypes.c_void_p * max(n, 1))(*[_ptr(w) for w in Ws])
    yp = (ctypes.c_void_p * max(n, 1))(*[_ptr(y) for y in ys])
    rc = _lib.lora_project_slots_x(pool, n, sl.ctypes.data, ctypes.cast(xp, ctypes.c_void_p),
                                   ctypes.cast(wp, ctypes.c_void_p), _ptr(adapter_ids), _ptr(ranks), _ptr(scale), T,
                                   ctypes.cast(yp, ctypes.c_void_p), _ptr(workspace), workspace_bytes, _stream(stream))
    return _check(rc, "lora_project_slots_x") if check else rc


def lora_debug_project(pool, x, W, page_table, adapter_ids, ranks, scale, T, y, workspace, gather_out, order_out,
                       workspace_bytes=None, stream=None, check=True):
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    rc = _lib.lora_debug_project(pool, _ptr(x), _ptr(W), _ptr(page_table), _ptr(adapter_ids), _ptr(ranks),
                                 _ptr(scale), T, _ptr(y), _ptr(workspace), workspace_bytes, _ptr(gather_out),
                                 _ptr(order_out), _stream(stream))
    return _check(rc, "lora_debug_project") if check else rc


def lora_project_noalloc(pool, x, W, page_table, adapter_ids, ranks, scale, T, y, stream=None, check=True):
    rc = _lib.lora_project_noalloc(pool, _ptr(x), _ptr(W), _ptr(page_table), _ptr(adapter_ids), _ptr(ranks),
                                   _ptr(scale), T, _ptr(y), _stream(stream))
    return _check(rc, "lora_project_noalloc") if check else rc


def lora_check_device_errors(pool, check=True):
    rc = _lib.lora_check_device_errors(pool)
    return _check(rc, "lora_check_device_errors") if check else rc


def lora_profile_start(pool, max_calls):
    return _check(_lib.lora_profile_start(pool, max_calls), "lora_profile_start")


def lora_profile_stop(pool) -> dict:
    pr = lora_profile_t()
    _check(_lib.lora_profile_stop(pool, ctypes.byref(pr)), "lora_profile_stop")
    return {name: getattr(pr, name) for name, _ in pr._fields_}


def lora_last_error() -> str:
    return _lib.lora_last_error().decode(errors="replace")


def lora_version() -> str:
    return _lib.lora_version().decode()


def run_pool_ops(pool, ops, ranks, adapter_weights, stream=None):
    """Apply a list of pool operations (as the workload generators emit them) to a pool handle.

    adapter_weights(aid) -> (A_t, B).  Returns each operation's status code.
    """
    out = []
    for op in ops:
        k = op[0]
        if k == "load":
            aid = op[1]
            at, b = adapter_weights(aid) if int(ranks[aid]) > 0 else (None, None)
            out.append(lora_pool_load_adapter(pool, aid, int(ranks[aid]), at, b, stream, check=False))
        elif k == "kv":
            r = lora_pool_grow_kv(pool, op[1], op[2], check=False)
            out.append(r if isinstance(r, int) else 0)
        elif k == "free_kv":
            out.append(lora_pool_free_kv(pool, op[1], check=False))
        elif k == "release":
            out.append(lora_pool_release_adapter(pool, op[1], check=False))
        elif k == "evict":
            out.append(lora_pool_evict_adapter(pool, op[1], stream, check=False))
        else:
            raise ValueError(k)
    return out


# ---- convenience owner of a pool's device buffers ----------------------------------------------------

class Pool:
    """A pool plus the torch-allocated device memory it runs on (pages, page table, workspace)."""

    def __init__(self, num_pages, hidden, dtype, n_slots=1, max_adapters=1, max_rank=LORA_MAX_RANK,
                 free_order=None, device="cuda"):
        import torch
        self.torch = torch
        self.hidden, self.dtype, self.n_slots = hidden, dtype, n_slots
        self.max_rank, self.max_adapters, self.num_pages = max_rank, max_adapters, num_pages
        self.tdtype = torch.float32 if dtype == LORA_F32 else torch.bfloat16
        if device is None:
            self.pages = self.table = None
        else:
            self.pages = torch.empty((num_pages, hidden), dtype=self.tdtype, device=device)
            self.table = torch.empty((n_slots, max_adapters, 2 * max_rank), dtype=torch.int32, device=device)
        self.handle = lora_pool_create(self.pages, num_pages, hidden, dtype, max_rank, n_slots, max_adapters,
                                       self.table, free_order)
        self._ws = None

    def close(self):
        if self.handle:
            lora_pool_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def slot_table(self, slot):
        return self.table[slot]

    def stats(self):
        return lora_pool_stats(self.handle)

    def workspace(self, T):
        need = lora_project_workspace_size(self.handle, T)
        if self._ws is None or self._ws.numel() < need:
            self._ws = self.torch.empty(max(need, 256), dtype=self.torch.uint8, device=self.pages.device)
        return self._ws

    def run_ops(self, ops, ranks, adapter_weights, stream=None):
        return run_pool_ops(self.handle, ops, ranks, adapter_weights, stream)

    def project_slots(self, slots, x, Ws, adapter_ids, ranks, scale, ys=None, stream=None):
        """x: one tensor every slot reads (lora_project_slots), or a list with one per slot
        (lora_project_slots_x)."""
        per_slot = isinstance(x, (list, tuple))
        x0 = x[0] if per_slot else x
        T = x0.shape[0]
        if ys is None:
            ys = [self.torch.empty_like(x0) for _ in slots]
        need = lora_project_slots_workspace_size(self.handle, len(slots), T)
        if self._ws is None or self._ws.numel() < need:
            self._ws = self.torch.empty(max(need, 256), dtype=self.torch.uint8, device=self.pages.device)
        if per_slot:
            lora_project_slots_x(self.handle, slots, x, Ws, adapter_ids, ranks, scale, T, ys, self._ws, stream=stream)
        else:
            lora_project_slots(self.handle, slots, x, Ws, adapter_ids, ranks, scale, T, ys, self._ws, stream=stream)
        return ys

    def project(self, slot, x, W, adapter_ids, ranks, scale, y=None, stream=None):
        T = x.shape[0]
        if y is None:
            y = self.torch.empty_like(x)
        ws = self.workspace(T)
        lora_project(self.handle, x, W, self.table[slot], adapter_ids, ranks, scale, T, y, ws, stream=stream)
        return y
