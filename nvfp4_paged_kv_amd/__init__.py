"""Python binding of the MI355X NVFP4 paged-KV library (libnvfp4kv.so).

Argument marshalling only: every step of the append and of the prefill runs
in the library's HIP kernels.  torch supplies device memory and the current
stream.  Importing this package does not need a GPU; calling the device
entry points does, and they raise if the built library is missing.

Entry points (same names as the C ABI in include/nvfp4kv.h):
  nvfp4_append_paged_kv(k, v, slot_mapping, k_scale, v_scale,
                        k_cache, v_cache, k_sf, v_sf, page_size)
  plan(qo_indptr, kv_lens, num_q_heads, num_kv_heads, head_dim, page_size)
  paged_prefill_causal(q, qo_indptr, kv_indptr, page_table, kv_lens, caches,
                       out, sm_scale, plan=None)
  read_device_error(device=None, clear=True)
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional, Union

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnvfp4kv.so")

OK, EINVAL, EUNSUPPORTED, ERANGE, EHIP, EWORKSPACE = 0, -1, -2, -3, -4, -5
DEV_BAD_K_SCALE, DEV_BAD_V_SCALE, DEV_SLOT_OOB, DEV_PAGE_OOB, DEV_BAD_SCALE_ATTN = 1, 2, 4, 8, 16
DEV_SPLIT_TIMEOUT = 32

ENTRY_POINTS = ("nvfp4_append_paged_kv", "nvfp4_prefill_plan", "paged_prefill_causal",
                "paged_prefill_causal_noalloc", "nvfp4_decode_plan", "paged_decode",
                "nvfp4kv_read_device_error", "nvfp4kv_status_string", "nvfp4kv_abi_version")


class NVFP4KVError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {lib().nvfp4kv_status_string(status).decode()} (status {status})")


class Cache(ctypes.Structure):
    _fields_ = [("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
                ("k_sf", ctypes.c_void_p), ("v_sf", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("num_pages", ctypes.c_int64), ("page_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32)]


class PlanStruct(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("batch", "num_q_heads", "num_kv_heads", "head_dim", "page_size",
                 "max_q_len", "max_kv_len")] + \
               [("total_q", ctypes.c_int64), ("total_kv", ctypes.c_int64)] + \
               [(n, ctypes.c_int32) for n in
                ("uniform_q", "uniform_kv", "head_first", "block_q", "block_n",
                 "q_tiles_per_head", "max_tile_cost", "num_xcd")] + \
               [(n, ctypes.c_int64) for n in
                ("num_tiles", "kv_bytes", "l2_bytes", "workspace_bytes")] + \
               [("split_len", ctypes.c_int32), ("max_chunks", ctypes.c_int32),
                ("num_items", ctypes.c_int64), ("num_split_tiles", ctypes.c_int64),
                ("dequant_mode", ctypes.c_int32), ("cu_count", ctypes.c_int32),
                ("schedule", ctypes.c_int32)]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class DecodePlanStruct(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("batch", "num_q_heads", "num_kv_heads", "head_dim", "page_size", "max_kv_len")] + \
               [("total_kv", ctypes.c_int64), ("chunk_len", ctypes.c_int32), ("max_chunks", ctypes.c_int32),
                ("num_items", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64),
                ("heads_per_wave", ctypes.c_int32)]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


_lib = None


def lib():
    """The loaded C library.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        path = os.environ.get("NVFP4KV_LIBRARY", LIB_PATH)
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with "
                               "`python nvfp4_paged_kv_amd/build.py` (hipcc, gfx950)")
        L = ctypes.CDLL(path)
        P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        L.nvfp4_append_paged_kv.argtypes = [P, P, P, I64, P, P, P, P, P, P, I64, I32, I32, I32, P, P]
        L.nvfp4_append_paged_kv.restype = ctypes.c_int
        L.nvfp4_prefill_plan.argtypes = [P, P, P, I32, I32, I32, I32, I32, I64, I32, I32, I32,
                                         ctypes.POINTER(PlanStruct)]
        L.nvfp4_prefill_plan.restype = ctypes.c_int
        L.paged_prefill_causal.argtypes = [P, P, P, P, P, ctypes.POINTER(Cache), P, ctypes.c_float,
                                           ctypes.POINTER(PlanStruct), P, I64, P, P]
        L.paged_prefill_causal.restype = ctypes.c_int
        L.paged_prefill_causal_noalloc.argtypes = [P, P, P, P, P, ctypes.POINTER(Cache), P, ctypes.c_float,
                                                   ctypes.POINTER(PlanStruct), P, P]
        L.paged_prefill_causal_noalloc.restype = ctypes.c_int
        L.nvfp4_decode_plan.argtypes = [P, I32, I32, I32, I32, I32, I32, ctypes.POINTER(DecodePlanStruct)]
        L.nvfp4_decode_plan.restype = ctypes.c_int
        L.paged_decode.argtypes = [P, P, P, P, ctypes.POINTER(Cache), P, ctypes.c_float,
                                   ctypes.POINTER(DecodePlanStruct), P, I64, P, P]
        L.paged_decode.restype = ctypes.c_int
        L.nvfp4kv_read_device_error.argtypes = [P, P, ctypes.POINTER(ctypes.c_uint32), ctypes.c_int]
        L.nvfp4kv_read_device_error.restype = ctypes.c_int
        L.nvfp4kv_status_string.argtypes = [ctypes.c_int]
        L.nvfp4kv_status_string.restype = ctypes.c_char_p
        L.nvfp4kv_abi_version.restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status: int, what: str):
    if status == EINVAL or status == ERANGE:
        raise ValueError(f"{what}: {lib().nvfp4kv_status_string(status).decode()}")
    if status != OK:
        raise NVFP4KVError(status, what)


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


# one device error word per device (int32 zeros; a torch fill, not a copy)
_err_words: dict = {}


def _norm_device(device) -> torch.device:
    """torch.device with the current GPU's index filled in, so that "cuda" and
    "cuda:N" name one workspace or error word."""
    device = torch.device(device)
    if device.type == "cuda" and device.index is None:
        device = torch.device("cuda", torch.cuda.current_device())
    return device


def device_error_word(device) -> torch.Tensor:
    """The library's default device error word for `device` (one per device)."""
    device = _norm_device(device)
    if device not in _err_words:
        _err_words[device] = torch.zeros(1, dtype=torch.int32, device=device)
    return _err_words[device]


def read_device_error(device=None, clear: bool = True, word: Optional[torch.Tensor] = None) -> int:
    """Synchronizing read of the device error bits (the only syncing call)."""
    if word is None:
        word = device_error_word(device if device is not None else "cuda")
    bits = ctypes.c_uint32(0)
    _check(lib().nvfp4kv_read_device_error(ctypes.c_void_p(word.data_ptr()), _stream(word.device),
                                           ctypes.byref(bits), int(clear)), "read_device_error")
    return int(bits.value)


def _scale_tensor(name: str, value, device: torch.device) -> torch.Tensor:
    """The global decode scale as an fp32 scalar on `device` (scale contract of
    the FlashInfer PR #6204 page, sections "code analysis" and "change in
    error handling").  A Python number or a CPU tensor is already on the host,
    so it is validated here and rejected with ValueError.  A GPU tensor is
    passed through unread: only its shape, dtype, device and layout are
    checked, and its value is validated by the kernels (a host read would
    wait for the stream)."""
    if isinstance(value, torch.Tensor) and value.device.type == "cuda":
        if value.numel() != 1 or value.dtype != torch.float32:
            raise ValueError(f"{name} must be a scalar torch.float32 tensor")
        if value.device != device:
            raise ValueError(f"{name} must be on {device}")
        if not value.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        return value
    if isinstance(value, torch.Tensor):
        if value.numel() != 1:
            raise ValueError(f"{name} must be a scalar")
        value = float(value.reshape(()).item())
    value = float(value)
    if not math.isfinite(value) or value <= 0.0:
        raise ValueError(f"{name}: a global decode scale has to be finite and greater than zero "
                         f"(got {value!r})")
    return torch.full((), value, dtype=torch.float32, device=device)


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(t.data_ptr() if t is not None else 0)


def nvfp4_append_paged_kv(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor, k_scale,
                          v_scale, k_cache: torch.Tensor, v_cache: torch.Tensor,
                          k_sf: torch.Tensor, v_sf: torch.Tensor, page_size: int,
                          dev_error: Optional[torch.Tensor] = None):
    """Quantize k/v (bf16 [T, H_kv, D]) to NVFP4 and write them at slot_mapping
    (int64 [T]) into the NHD caches (uint8 [P, page_size, H_kv, D/2]) and
    scale-factor pages (uint8 [P, page_size, H_kv, D/16]).  Never synchronizes."""
    if k.dim() != 3 or v.shape != k.shape:
        raise ValueError("k and v must be [num_tokens, num_kv_heads, head_dim] of equal shape")
    T, H, D = k.shape
    dev = k.device
    for name, t, dt in (("k", k, torch.bfloat16), ("v", v, torch.bfloat16),
                        ("slot_mapping", slot_mapping, torch.int64), ("k_cache", k_cache, torch.uint8),
                        ("v_cache", v_cache, torch.uint8), ("k_sf", k_sf, torch.uint8),
                        ("v_sf", v_sf, torch.uint8)):
        if t.dtype != dt:
            raise ValueError(f"{name} must be {dt}")
        if t.device != dev:
            raise ValueError(f"{name} must be on {dev}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be [num_tokens]")
    P = k_cache.shape[0]
    if k_cache.shape != (P, page_size, H, D // 2) or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache/v_cache must be [num_pages, page_size, num_kv_heads, head_dim/2]")
    if k_sf.shape != (P, page_size, H, D // 16) or v_sf.shape != k_sf.shape:
        raise ValueError("k_sf/v_sf must be [num_pages, page_size, num_kv_heads, head_dim/16]")
    ks = _scale_tensor("k_scale", k_scale, dev)
    vs = _scale_tensor("v_scale", v_scale, dev)
    err = dev_error if dev_error is not None else device_error_word(dev)
    _check(lib().nvfp4_append_paged_kv(
        _ptr(k), _ptr(v), _ptr(slot_mapping), T, _ptr(ks), _ptr(vs), _ptr(k_cache), _ptr(v_cache),
        _ptr(k_sf), _ptr(v_sf), P, page_size, H, D, _ptr(err), _stream(dev)), "nvfp4_append_paged_kv")


@dataclass
class PagedCache:
    """An NVFP4 paged KV cache (NHD pages) with its global decode scales."""
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    k_sf: torch.Tensor
    v_sf: torch.Tensor
    k_scale: torch.Tensor
    v_scale: torch.Tensor

    @classmethod
    def empty(cls, num_pages, page_size, num_kv_heads, head_dim, device, k_scale=1.0, v_scale=1.0,
              fill: Optional[int] = 0):
        def mk(last):
            t = torch.empty((num_pages, page_size, num_kv_heads, last), dtype=torch.uint8, device=device)
            if fill is not None:
                t.fill_(fill)
            return t
        return cls(mk(head_dim // 2), mk(head_dim // 2), mk(head_dim // 16), mk(head_dim // 16),
                   _scale_tensor("k_scale", k_scale, torch.device(device)),
                   _scale_tensor("v_scale", v_scale, torch.device(device)))

    @property
    def num_pages(self):
        return self.k_cache.shape[0]

    @property
    def page_size(self):
        return self.k_cache.shape[1]

    @property
    def num_kv_heads(self):
        return self.k_cache.shape[2]

    @property
    def head_dim(self):
        return self.k_cache.shape[3] * 2

    def append(self, k, v, slot_mapping, dev_error=None):
        nvfp4_append_paged_kv(k, v, slot_mapping, self.k_scale, self.v_scale, self.k_cache,
                              self.v_cache, self.k_sf, self.v_sf, self.page_size, dev_error)

    def _struct(self) -> Cache:
        return Cache(self.k_cache.data_ptr(), self.v_cache.data_ptr(), self.k_sf.data_ptr(),
                     self.v_sf.data_ptr(), self.k_scale.data_ptr(), self.v_scale.data_ptr(),
                     self.num_pages, self.page_size, self.num_kv_heads, self.head_dim)


class Plan:
    """Host-side plan of one prefill batch (FlashInfer PR #5043 page: plan()
    max lengths from tensor reductions, lengths cast to int32 at entry)."""

    def __init__(self, qo_indptr, kv_lens, num_q_heads, num_kv_heads, head_dim, page_size,
                 kv_indptr=None, l2_bytes: int = 0, split_len: int = 0, tile_waves: int = 0,
                 dequant_mode: Optional[int] = None, cu_count: int = 0, schedule: int = 0):
        qo = _host_int32(qo_indptr, "qo_indptr")
        kvl = _host_int32(kv_lens, "kv_lens")
        kvp = _host_int32(kv_indptr, "kv_indptr") if kv_indptr is not None else None
        if qo.numel() != kvl.numel() + 1:
            raise ValueError("qo_indptr must have batch + 1 entries")
        self.struct = PlanStruct()
        _check(lib().nvfp4_prefill_plan(
            _ptr(qo), _ptr(kvl), _ptr(kvp), kvl.numel(), num_q_heads, num_kv_heads, head_dim,
            page_size, l2_bytes, cu_count, split_len, tile_waves, ctypes.byref(self.struct)),
            "nvfp4_prefill_plan")
        if dequant_mode is not None:
            self.struct.dequant_mode = int(dequant_mode)
        if schedule:
            self.struct.schedule = int(schedule)
        self.qo_host, self.kv_lens_host, self.kv_indptr_host = qo, kvl, kvp
        # page-table entries the batch's requests own (checked against the
        # device page table's size at every call)
        if kvp is not None and kvp.numel() == kvl.numel() + 1:
            self.pages_needed = int(kvp[-1]) if kvp.numel() else 0
        else:
            self.pages_needed = int(((kvl.to(torch.int64) + page_size - 1) // page_size).sum()) \
                if kvl.numel() else 0
        self._workspace = {}

    def __getattr__(self, name):
        if name == "struct":
            raise AttributeError(name)
        return getattr(self.struct, name)

    def workspace(self, device) -> Optional[torch.Tensor]:
        n = self.struct.workspace_bytes
        if n == 0:
            return None
        device = _norm_device(device)
        if device not in self._workspace:
            # no initial contents needed: each call writes its work list and
            # zeroes its split counters before the prefill kernel reads them
            self._workspace[device] = torch.empty(n, dtype=torch.uint8, device=device)
        return self._workspace[device]


def _host_int32(t, name) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        t = torch.as_tensor(t)
    if t.device.type != "cpu":
        raise ValueError(f"{name} must be a host (CPU) tensor for the plan step")
    t = t.flatten()
    if t.dtype == torch.uint32:
        t = t.to(torch.int64)
    return t.to(torch.int32).contiguous()


SCHEDULE_HEAVIEST, SCHEDULE_STREAM, SCHEDULE_REQUEST, SCHEDULE_PAIRED = 1, 2, 3, 4


def plan(qo_indptr, kv_lens, num_q_heads, num_kv_heads, head_dim, page_size, kv_indptr=None,
         l2_bytes: int = 0, split_len: int = 0, tile_waves: int = 0, dequant_mode: Optional[int] = None,
         cu_count: int = 0, schedule: int = 0) -> Plan:
    """Host plan of one prefill batch.  l2_bytes / cu_count: device L2 and CU
    count to plan for (0: the current device's); split_len: KV tiles per chunk
    of a split Q tile (0 automatic, > 0 forced, < 0 never); tile_waves: waves
    of 32 query rows per workgroup (0 automatic, 4 or 8); dequant_mode: the
    staging form and dequant-placement ablation (None: the plan's choice, 3;
    3: tiles decoded once into a bf16 LDS tile, bf16 queries, probabilities
    and matrix instructions; 0: the same in f16; 1: as 0 with K decoded in
    registers inside the matrix loop; 2: as 0 with a byte-table decode; 4
    and 5: native MX scores -- MXFP4 (4) or MXFP8 (5) keys, MXFP8 queries,
    the scaled matrix instruction, under looser accuracy contracts); schedule: issue
    order of the Q tiles (0: the plan's choice; SCHEDULE_HEAVIEST,
    SCHEDULE_STREAM, SCHEDULE_REQUEST, or SCHEDULE_PAIRED -- Q tiles t and
    QT - 1 - t of a uniform, unsplit batch of 4-wave tiles in one 8-wave
    workgroup)."""
    return Plan(qo_indptr, kv_lens, num_q_heads, num_kv_heads, head_dim, page_size, kv_indptr,
                l2_bytes, split_len, tile_waves, dequant_mode, cu_count, schedule)


def paged_prefill_causal(q: torch.Tensor, qo_indptr: torch.Tensor, kv_indptr: torch.Tensor,
                         page_table: torch.Tensor, kv_lens: torch.Tensor, caches: PagedCache,
                         out: torch.Tensor, sm_scale: float, plan: Optional[Plan] = None,
                         dev_error: Optional[torch.Tensor] = None):
    """Causal prefill over the NVFP4 paged cache.  q/out: bf16 [total_q, H_q, D];
    qo_indptr, kv_indptr, page_table, kv_lens: int32 device tensors.  Without
    `plan`, qo_indptr and kv_lens may instead be host tensors (the plan is then
    computed here and the arrays are uploaded)."""
    dev = q.device
    if plan is None:
        plan = Plan(qo_indptr.cpu() if qo_indptr.device.type == "cpu" else _need_host("qo_indptr"),
                    kv_lens.cpu() if kv_lens.device.type == "cpu" else _need_host("kv_lens"),
                    q.shape[1], caches.num_kv_heads, caches.head_dim, caches.page_size)
    if qo_indptr.device.type == "cpu":
        qo_indptr = qo_indptr.to(torch.int32).pin_memory().to(dev, non_blocking=True)
    if kv_lens.device.type == "cpu":
        kv_lens = kv_lens.to(torch.int32).pin_memory().to(dev, non_blocking=True)
    for name, t, dt in (("q", q, torch.bfloat16), ("out", out, torch.bfloat16),
                        ("qo_indptr", qo_indptr, torch.int32), ("kv_indptr", kv_indptr, torch.int32),
                        ("page_table", page_table, torch.int32), ("kv_lens", kv_lens, torch.int32)):
        if t.dtype != dt or t.device != dev or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dt} tensor on {dev}")
    if q.dim() != 3 or out.shape != q.shape or q.shape[2] != caches.head_dim:
        raise ValueError("q/out must be [total_q, num_q_heads, head_dim]")
    if q.shape[0] != plan.total_q or q.shape[1] != plan.num_q_heads:
        raise ValueError("q does not match the plan")
    _check_batch_arrays(plan, qo_indptr, kv_indptr, kv_lens, page_table)
    ws = plan.workspace(dev)
    err = dev_error if dev_error is not None else device_error_word(dev)
    cs = caches._struct()
    _check(lib().paged_prefill_causal(
        _ptr(q), _ptr(qo_indptr), _ptr(kv_indptr), _ptr(page_table), _ptr(kv_lens), ctypes.byref(cs),
        _ptr(out), float(sm_scale), ctypes.byref(plan.struct), _ptr(ws),
        0 if ws is None else ws.numel(), _ptr(err), _stream(dev)), "paged_prefill_causal")
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20  # NVFP4KV_NOALLOC_SCRATCH_BYTES


def paged_prefill_causal_noalloc(q: torch.Tensor, qo_indptr: torch.Tensor, kv_indptr: torch.Tensor,
                                 page_table: torch.Tensor, kv_lens: torch.Tensor, caches: PagedCache,
                                 out: torch.Tensor, sm_scale: float, plan: Plan,
                                 dev_error: torch.Tensor):
    """paged_prefill_causal for callers that cannot allocate device memory:
    every argument is already on the device (no plan is built, nothing is
    uploaded, no workspace is requested) and the library takes its workspace
    from its own per-GPU array.  Calls overlapping on one GPU race."""
    dev = q.device
    for name, t, dt in (("q", q, torch.bfloat16), ("out", out, torch.bfloat16),
                        ("qo_indptr", qo_indptr, torch.int32), ("kv_indptr", kv_indptr, torch.int32),
                        ("page_table", page_table, torch.int32), ("kv_lens", kv_lens, torch.int32),
                        ("dev_error", dev_error, torch.int32)):
        if t.dtype != dt or t.device != dev or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dt} tensor on {dev}")
    if q.dim() != 3 or out.shape != q.shape or q.shape[2] != caches.head_dim:
        raise ValueError("q/out must be [total_q, num_q_heads, head_dim]")
    if q.shape[0] != plan.total_q or q.shape[1] != plan.num_q_heads:
        raise ValueError("q does not match the plan")
    _check_batch_arrays(plan, qo_indptr, kv_indptr, kv_lens, page_table)
    cs = caches._struct()
    _check(lib().paged_prefill_causal_noalloc(
        _ptr(q), _ptr(qo_indptr), _ptr(kv_indptr), _ptr(page_table), _ptr(kv_lens), ctypes.byref(cs),
        _ptr(out), float(sm_scale), ctypes.byref(plan.struct), _ptr(dev_error), _stream(dev)),
        "paged_prefill_causal_noalloc")
    return out


class DecodePlan:
    """Host-side plan of one decode step (one query token per request)."""

    def __init__(self, kv_lens, num_q_heads, num_kv_heads, head_dim, page_size, chunk_len: int = 0):
        kvl = _host_int32(kv_lens, "kv_lens")
        self.struct = DecodePlanStruct()
        _check(lib().nvfp4_decode_plan(_ptr(kvl), kvl.numel(), num_q_heads, num_kv_heads, head_dim,
                                       page_size, chunk_len, ctypes.byref(self.struct)),
               "nvfp4_decode_plan")
        self.kv_lens_host = kvl
        self.pages_needed = int(((kvl.to(torch.int64) + page_size - 1) // page_size).sum()) \
            if kvl.numel() else 0
        self._workspace = {}

    def __getattr__(self, name):
        if name == "struct":
            raise AttributeError(name)
        return getattr(self.struct, name)

    def workspace(self, device) -> Optional[torch.Tensor]:
        n = self.struct.workspace_bytes
        if n == 0:
            return None
        device = _norm_device(device)
        if device not in self._workspace:
            self._workspace[device] = torch.empty(n, dtype=torch.uint8, device=device)
        return self._workspace[device]


def decode_plan(kv_lens, num_q_heads, num_kv_heads, head_dim, page_size, chunk_len: int = 0) -> DecodePlan:
    """Host plan of one decode step.  chunk_len: keys per KV chunk (0 automatic,
    else a multiple of 64)."""
    return DecodePlan(kv_lens, num_q_heads, num_kv_heads, head_dim, page_size, chunk_len)


def paged_decode(q: torch.Tensor, kv_indptr: torch.Tensor, page_table: torch.Tensor,
                 kv_lens: torch.Tensor, caches: PagedCache, out: torch.Tensor, sm_scale: float,
                 plan: DecodePlan, dev_error: Optional[torch.Tensor] = None):
    """One decode step over the NVFP4 paged cache.  q/out: bf16 [batch, H_q, D];
    kv_indptr, page_table, kv_lens: int32 device tensors."""
    dev = q.device
    for name, t, dt in (("q", q, torch.bfloat16), ("out", out, torch.bfloat16),
                        ("kv_indptr", kv_indptr, torch.int32), ("page_table", page_table, torch.int32),
                        ("kv_lens", kv_lens, torch.int32)):
        if t.dtype != dt or t.device != dev or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dt} tensor on {dev}")
    if q.dim() != 3 or out.shape != q.shape or q.shape[2] != caches.head_dim:
        raise ValueError("q/out must be [batch, num_q_heads, head_dim]")
    if q.shape[0] != plan.batch or q.shape[1] != plan.num_q_heads:
        raise ValueError("q does not match the plan")
    _check_batch_arrays(plan, None, kv_indptr, kv_lens, page_table)
    ws = plan.workspace(dev)
    err = dev_error if dev_error is not None else device_error_word(dev)
    cs = caches._struct()
    _check(lib().paged_decode(
        _ptr(q), _ptr(kv_indptr), _ptr(page_table), _ptr(kv_lens), ctypes.byref(cs), _ptr(out),
        float(sm_scale), ctypes.byref(plan.struct), _ptr(ws), 0 if ws is None else ws.numel(),
        _ptr(err), _stream(dev)), "paged_decode")
    return out


def _check_batch_arrays(plan, qo_indptr, kv_indptr, kv_lens, page_table):
    """Element counts of the per-request device arrays against the plan (no
    device read): the kernels index them by request and page without bounds."""
    B = plan.batch
    if qo_indptr is not None and qo_indptr.numel() != B + 1:
        raise ValueError(f"qo_indptr must have batch + 1 = {B + 1} entries")
    if kv_indptr.numel() != B + 1:
        raise ValueError(f"kv_indptr must have batch + 1 = {B + 1} entries")
    if kv_lens.numel() != B:
        raise ValueError(f"kv_lens must have batch = {B} entries")
    need = plan.pages_needed
    if page_table.numel() < need:
        raise ValueError(f"page_table has {page_table.numel()} entries; the batch's requests "
                         f"own {need}")


def _need_host(name):
    raise ValueError(f"{name} must be a host tensor when no plan is given")
