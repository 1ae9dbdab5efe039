"""Thin ctypes binding of ``libhisparse.so``.

Argument marshalling only: every step of the swap-in path runs in the HIP
library.  The module-level ``hisparse_*`` functions mirror the C entry points
one to one (pointers as Python ints); :class:`HiSparseState` and
:class:`HostKV` are conveniences that pass torch tensors / pinned host buffers
through them.

torch is imported before the library is loaded so that the library binds to
the HIP runtime torch already loaded (both export the same soname), and
streams and device pointers are shared between the two.
"""
from __future__ import annotations

import ctypes
import pathlib

import numpy as np
import torch

LIB_PATH = pathlib.Path(__file__).resolve().with_name("libhisparse.so")

HISPARSE_OK = 0
HISPARSE_E_INVAL = -1
HISPARSE_E_NOMEM = -2
HISPARSE_E_HIP = -3
HISPARSE_E_UNSUPPORTED = -4

ERR_BAD_INDEX = 1
ERR_DUP_REQUEST = 2
ERR_PAGE_OVERFLOW = 4
ERR_BAD_ROW = 8
ERR_BAD_PLAN = 16

POLICY = {"lru": 0, "clock": 1}

MAX_HOT = 32768
MAX_WORKING_SET = 8192

c_i32 = ctypes.c_int32
c_vp = ctypes.c_void_p


class HisparseConfig(ctypes.Structure):
    _fields_ = [
        ("max_requests", c_i32), ("num_layers", c_i32), ("hot_buffer_size", c_i32),
        ("top_k", c_i32), ("max_steps", c_i32), ("page_size", c_i32),
        ("item_size_bytes", c_i32), ("max_seq_len", c_i32), ("policy", c_i32),
        ("max_batch", c_i32), ("host_kv", ctypes.POINTER(c_vp)),
        ("dev_kv", ctypes.POINTER(c_vp)), ("admission", c_i32), ("extra_rows", c_i32),
    ]


class HisparseMissPlan(ctypes.Structure):
    _fields_ = [("miss_src", c_vp), ("miss_dst", c_vp), ("victim", c_vp), ("capacity", c_i32),
                ("flags", c_i32)]


HISPARSE_PLAN_DEFER_COPY = 1


class HisparseTopkCall(ctypes.Structure):
    _fields_ = [
        ("batch", c_i32), ("max_len", c_i32), ("k", c_i32), ("logits", c_vp),
        ("seq_lens", c_vp), ("plan", c_vp), ("plan_ints", ctypes.c_size_t), ("mode", c_i32),
        ("page_table", c_vp), ("pt_stride", c_i32), ("page_size", c_i32),
        ("row_offsets", c_vp), ("indices", c_vp), ("locs", c_vp), ("workspace", c_vp),
        ("workspace_bytes", ctypes.c_size_t), ("error_word", c_vp),
    ]


INDEX_MODE = {"none": 0, "paged": 1, "ragged": 2}
ADMISSION = {"recent": 0, "frequent": 1, "first": 2}
TOPK_CHUNK = 32768


class HisparseProfile(ctypes.Structure):
    _fields_ = [("calls", ctypes.c_int64), ("plan_ms", ctypes.c_double),
                ("copy_ms", ctypes.c_double), ("fused_calls", ctypes.c_int64)]


_SIGNATURES = {
    "hisparse_device_rows_per_request": (ctypes.c_int64, [ctypes.POINTER(HisparseConfig)]),
    "hisparse_state_create": (ctypes.c_int, [ctypes.POINTER(HisparseConfig), c_vp,
                                             ctypes.POINTER(c_vp)]),
    "hisparse_state_destroy": (None, [c_vp]),
    "hisparse_swap_in_selected": (ctypes.c_int, [c_vp, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp,
                                                 c_vp, c_vp, c_vp,
                                                 ctypes.POINTER(HisparseMissPlan), c_vp]),
    "hisparse_swap_in_spec_multistep": (ctypes.c_int, [c_vp, c_i32, c_i32, c_i32, c_vp, c_vp,
                                                       c_vp, c_vp, c_vp,
                                                       ctypes.POINTER(HisparseMissPlan),
                                                       c_vp]),
    "hisparse_copy_planned": (ctypes.c_int, [c_vp, c_i32, c_i32, c_vp,
                                             ctypes.POINTER(HisparseMissPlan), c_vp]),
    "hisparse_sparse_mla_workspace_bytes": (ctypes.c_size_t, [c_vp, c_i32, c_i32, c_i32]),
    "hisparse_sparse_mla_decode": (ctypes.c_int, [c_vp, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp,
                                                  c_vp, ctypes.c_float, c_vp, c_vp, c_vp,
                                                  ctypes.c_size_t, c_vp]),
    "hisparse_topk_plan_ints": (ctypes.c_size_t, [c_i32, c_i32]),
    "hisparse_topk_plan": (ctypes.c_int, [c_i32, c_i32, c_vp, c_vp, ctypes.c_size_t, c_vp]),
    "hisparse_topk_workspace_bytes": (ctypes.c_size_t, [c_i32, c_i32, c_i32]),
    "hisparse_topk_index_build": (ctypes.c_int, [ctypes.POINTER(HisparseTopkCall), c_vp]),
    "hisparse_topk_index_build_noalloc": (ctypes.c_int, [ctypes.POINTER(HisparseTopkCall),
                                                         c_vp]),
    "hisparse_request_reset": (ctypes.c_int, [c_vp, c_i32, c_vp, c_vp]),
    "hisparse_plan_capacity": (c_i32, [c_vp]),
    "hisparse_state_export": (ctypes.c_int, [c_vp, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "hisparse_state_import": (ctypes.c_int, [c_vp, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp]),
    "hisparse_get_error_flags": (ctypes.c_int, [c_vp, ctypes.POINTER(ctypes.c_uint32), c_i32,
                                                c_vp]),
    "hisparse_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "hisparse_host_alloc": (ctypes.c_int, [ctypes.c_size_t, ctypes.POINTER(c_vp)]),
    "hisparse_host_free": (ctypes.c_int, [c_vp]),
    "hisparse_profile_enable": (ctypes.c_int, [c_vp, c_i32]),
    "hisparse_profile_read": (ctypes.c_int, [c_vp, ctypes.POINTER(HisparseProfile)]),
}

EXPORTED = tuple(_SIGNATURES)

_lib = None


class HiSparseError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {strerror(code)} ({code})")
        self.code = code


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_attention_kv_request_amd.build`")
        handle = ctypes.CDLL(str(LIB_PATH))
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def strerror(code: int) -> str:
    return lib().hisparse_strerror(code).decode()


def _check(code: int, what: str) -> int:
    if code != HISPARSE_OK:
        raise HiSparseError(code, what)
    return code


# -- one-to-one wrappers of the C entry points ---------------------------------

def hisparse_device_rows_per_request(cfg: HisparseConfig) -> int:
    return lib().hisparse_device_rows_per_request(ctypes.byref(cfg))


def hisparse_state_create(cfg: HisparseConfig, stream: int) -> int:
    out = c_vp()
    _check(lib().hisparse_state_create(ctypes.byref(cfg), stream, ctypes.byref(out)),
           "hisparse_state_create")
    return out.value


def hisparse_state_destroy(st: int) -> None:
    lib().hisparse_state_destroy(st)


def hisparse_swap_in_selected(st, layer_id, batch, req_pool_indices, seq_lens, topk_indices,
                              out_locs, miss_count, page_table, num_pages, plan, stream) -> int:
    return lib().hisparse_swap_in_selected(st, layer_id, batch, req_pool_indices, seq_lens,
                                           topk_indices, out_locs, miss_count, page_table,
                                           num_pages, plan, stream)


def hisparse_swap_in_spec_multistep(st, layer_id, batch, num_steps, req_pool_indices, seq_lens,
                                    topk_indices, out_locs, miss_count, plan, stream) -> int:
    return lib().hisparse_swap_in_spec_multistep(st, layer_id, batch, num_steps,
                                                 req_pool_indices, seq_lens, topk_indices,
                                                 out_locs, miss_count, plan, stream)


def hisparse_copy_planned(st, layer_id, batch, miss_count, plan, stream) -> int:
    return lib().hisparse_copy_planned(st, layer_id, batch, miss_count, plan, stream)


def hisparse_sparse_mla_workspace_bytes(st, batch, num_heads, n_locs) -> int:
    return lib().hisparse_sparse_mla_workspace_bytes(st, batch, num_heads, n_locs)


def hisparse_sparse_mla_decode(st, layer_id, batch, num_heads, n_locs, q, locs, page_table,
                               softmax_scale, out, lse, workspace, workspace_bytes,
                               stream) -> int:
    return lib().hisparse_sparse_mla_decode(st, layer_id, batch, num_heads, n_locs, q, locs,
                                            page_table, softmax_scale, out, lse, workspace,
                                            workspace_bytes, stream)


def hisparse_topk_plan_ints(batch, max_len) -> int:
    return lib().hisparse_topk_plan_ints(batch, max_len)


def hisparse_topk_plan(batch, max_len, seq_lens, plan, plan_ints, stream) -> int:
    return lib().hisparse_topk_plan(batch, max_len, seq_lens, plan, plan_ints, stream)


def hisparse_topk_workspace_bytes(batch, max_len, k) -> int:
    return lib().hisparse_topk_workspace_bytes(batch, max_len, k)


def hisparse_topk_index_build(call: HisparseTopkCall, stream) -> int:
    return lib().hisparse_topk_index_build(ctypes.byref(call), stream)


def hisparse_topk_index_build_noalloc(call: HisparseTopkCall, stream) -> int:
    return lib().hisparse_topk_index_build_noalloc(ctypes.byref(call), stream)


def hisparse_request_reset(st, n, req_pool_indices, stream) -> int:
    return lib().hisparse_request_reset(st, n, req_pool_indices, stream)


def hisparse_plan_capacity(st) -> int:
    return lib().hisparse_plan_capacity(st)


def hisparse_state_export(st, req, layer, slot_key_h, policy_h, ctrl_h, key_slot_h, stream):
    return lib().hisparse_state_export(st, req, layer, slot_key_h, policy_h, ctrl_h,
                                       key_slot_h, stream)


def hisparse_state_import(st, req, layer, slot_key_h, policy_h, ctrl_h, stream):
    return lib().hisparse_state_import(st, req, layer, slot_key_h, policy_h, ctrl_h, stream)


def hisparse_get_error_flags(st, clear: bool, stream) -> int:
    v = ctypes.c_uint32()
    _check(lib().hisparse_get_error_flags(st, ctypes.byref(v), int(clear), stream),
           "hisparse_get_error_flags")
    return v.value


def hisparse_host_alloc(nbytes: int) -> int:
    p = c_vp()
    _check(lib().hisparse_host_alloc(nbytes, ctypes.byref(p)), "hisparse_host_alloc")
    return p.value


def hisparse_host_free(ptr: int) -> None:
    _check(lib().hisparse_host_free(ptr), "hisparse_host_free")


def hisparse_profile_enable(st, enable: bool) -> None:
    _check(lib().hisparse_profile_enable(st, int(enable)), "hisparse_profile_enable")


def hisparse_profile_read(st) -> dict:
    p = HisparseProfile()
    _check(lib().hisparse_profile_read(st, ctypes.byref(p)), "hisparse_profile_read")
    return {"calls": p.calls, "plan_ms": p.plan_ms, "copy_ms": p.copy_ms,
            "fused_calls": p.fused_calls}


# -- conveniences ----------------------------------------------------------------

class HostKV:
    """Pinned, device-readable host buffer of one layer: uint8 [R, N, item]."""

    def __init__(self, requests: int, seq_len: int, unit_bytes: int):
        self.shape = (requests, seq_len, unit_bytes)
        self.nbytes = requests * seq_len * unit_bytes
        self.ptr = hisparse_host_alloc(self.nbytes)
        raw = (ctypes.c_uint8 * self.nbytes).from_address(self.ptr)
        self.array = np.ctypeslib.as_array(raw).reshape(self.shape)

    def tensor(self) -> torch.Tensor:
        """A CPU torch view sharing the pinned memory."""
        return torch.from_numpy(self.array)

    def free(self):
        if self.ptr:
            self.array = None
            hisparse_host_free(self.ptr)
            self.ptr = 0

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: torch.Tensor | None, dtype=torch.int32) -> int:
    if t is None:
        return 0
    if not t.is_cuda or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"expected a contiguous {dtype} CUDA tensor")
    return t.data_ptr()


class HiSparseState:
    """Owns a library state plus (optionally) the device KV buffers of every layer.

    ``host_kv``: list of :class:`HostKV` (one per layer).  ``dev_kv``: list of
    uint8 CUDA tensors ``[R, rows, item]`` (token) or ``[R, H, P * item]``
    (page); allocated here when omitted.
    """

    def __init__(self, *, max_requests, num_layers, hot_buffer_size, top_k, item_size_bytes,
                 max_seq_len, host_kv, max_steps=1, page_size=1, policy="lru",
                 max_batch=None, dev_kv=None, stream=None, admission="recent", extra_rows=0):
        self.cfg = HisparseConfig(
            max_requests=max_requests, num_layers=num_layers, hot_buffer_size=hot_buffer_size,
            top_k=top_k, max_steps=max_steps, page_size=page_size,
            item_size_bytes=item_size_bytes, max_seq_len=max_seq_len, policy=POLICY[policy],
            max_batch=max_batch or max_requests, admission=ADMISSION[admission],
            extra_rows=extra_rows)
        rows = hisparse_device_rows_per_request(self.cfg)
        if rows < 0:
            raise HiSparseError(rows, "hisparse_device_rows_per_request")
        self.rows = rows
        self.policy = policy
        self.admission = admission
        self.extra_rows = extra_rows
        self.page_size = page_size
        self.host_kv = host_kv
        unit = item_size_bytes * page_size
        if dev_kv is None:
            dev_kv = [torch.zeros((max_requests, rows, unit), dtype=torch.uint8, device="cuda")
                      for _ in range(num_layers)]
        self.dev_kv = dev_kv
        self._host_ptrs = (c_vp * num_layers)(*[h.ptr for h in host_kv])
        self._dev_ptrs = (c_vp * num_layers)(*[d.data_ptr() for d in dev_kv])
        self.cfg.host_kv = ctypes.cast(self._host_ptrs, ctypes.POINTER(c_vp))
        self.cfg.dev_kv = ctypes.cast(self._dev_ptrs, ctypes.POINTER(c_vp))
        self.handle = hisparse_state_create(self.cfg, _stream(stream))
        self.capacity = hisparse_plan_capacity(self.handle)

    # shapes
    @property
    def hot(self):
        return self.cfg.hot_buffer_size

    @property
    def nkeys(self):
        return self.cfg.max_seq_len // self.page_size

    def close(self):
        if getattr(self, "handle", None):
            torch.cuda.synchronize()
            hisparse_state_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @staticmethod
    def _plan(plan, defer_copy=False):
        if plan is None:
            if defer_copy:
                raise ValueError("defer_copy needs a plan to replay")
            return None
        src, dst, vic = plan
        flags = HISPARSE_PLAN_DEFER_COPY if defer_copy else 0
        return ctypes.byref(HisparseMissPlan(_ptr(src), _ptr(dst), _ptr(vic), src.shape[-1],
                                             flags))

    def swap_in_selected(self, layer_id, req_pool_indices, seq_lens, topk_indices, out_locs,
                         miss_count, page_table=None, num_pages=None, plan=None, stream=None,
                         defer_copy=False):
        """``defer_copy``: write the plan without copying; the caller runs
        :meth:`copy_planned` on it (HISPARSE_PLAN_DEFER_COPY)."""
        batch = int(req_pool_indices.shape[0])
        rc = hisparse_swap_in_selected(
            self.handle, layer_id, batch, _ptr(req_pool_indices), _ptr(seq_lens),
            _ptr(topk_indices), _ptr(out_locs), _ptr(miss_count), _ptr(page_table),
            _ptr(num_pages), self._plan(plan, defer_copy), _stream(stream))
        return _check(rc, "hisparse_swap_in_selected")

    def swap_in_spec_multistep(self, layer_id, req_pool_indices, seq_lens, topk_indices,
                               out_locs, miss_count, plan=None, stream=None, defer_copy=False):
        batch = int(req_pool_indices.shape[0])
        num_steps = int(topk_indices.shape[1])
        rc = hisparse_swap_in_spec_multistep(
            self.handle, layer_id, batch, num_steps, _ptr(req_pool_indices), _ptr(seq_lens),
            _ptr(topk_indices), _ptr(out_locs), _ptr(miss_count),
            self._plan(plan, defer_copy), _stream(stream))
        return _check(rc, "hisparse_swap_in_spec_multistep")

    def copy_planned(self, layer_id, miss_count, plan, stream=None):
        """Replays ``plan = (miss_src, miss_dst, victim)`` int32 [batch, cap]."""
        batch = int(miss_count.shape[0])
        rc = hisparse_copy_planned(self.handle, layer_id, batch, _ptr(miss_count),
                                   self._plan(plan), _stream(stream))
        return _check(rc, "hisparse_copy_planned")

    def sparse_mla_decode(self, layer_id, q, locs, out, lse=None, page_table=None,
                          softmax_scale=None, workspace=None, stream=None):
        """Decode attention of ``q`` (bf16 [B, heads, 576]) over ``locs``
        (int32 [B, n]) into ``out`` (float32 [B, heads, 512]) and ``lse``."""
        B, heads, dim = q.shape
        n = int(locs.shape[1])
        if q.dtype != torch.bfloat16 or dim != 576 or not q.is_contiguous():
            raise ValueError("q must be a contiguous bfloat16 [B, heads, 576] tensor")
        if out.dtype != torch.float32 or not out.is_contiguous():
            raise ValueError("out must be a contiguous float32 tensor")
        need = hisparse_sparse_mla_workspace_bytes(self.handle, B, heads, n)
        if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        scale = softmax_scale if softmax_scale is not None else 576 ** -0.5
        wptr = workspace.data_ptr() if (need and workspace is not None) else 0
        rc = hisparse_sparse_mla_decode(
            self.handle, layer_id, B, heads, n, q.data_ptr(), _ptr(locs), _ptr(page_table),
            scale, out.data_ptr(), lse.data_ptr() if lse is not None else 0, wptr,
            need, _stream(stream))
        return _check(rc, "hisparse_sparse_mla_decode")

    def request_reset(self, req_pool_indices: torch.Tensor, stream=None):
        rc = hisparse_request_reset(self.handle, int(req_pool_indices.shape[0]),
                                    _ptr(req_pool_indices), _stream(stream))
        return _check(rc, "hisparse_request_reset")

    def export(self, req: int, layer: int, with_map: bool = False, stream=None) -> dict:
        H = self.hot
        slot_key = np.empty(H, np.int32)
        policy = np.empty(H, np.int32)
        ctrl = np.empty(2, np.int32)
        key_slot = np.empty(self.nkeys, np.int32) if with_map else None
        rc = hisparse_state_export(
            self.handle, req, layer, slot_key.ctypes.data, policy.ctypes.data, ctrl.ctypes.data,
            key_slot.ctypes.data if with_map else None, _stream(stream))
        _check(rc, "hisparse_state_export")
        out = {"slot_key": slot_key, "ctrl": ctrl, "key_slot": key_slot}
        out["ts" if self.policy == "lru" else "ref"] = policy
        return out

    def import_(self, req: int, layer: int, slot_key, policy, ctrl, stream=None):
        slot_key = np.ascontiguousarray(slot_key, np.int32)
        policy = np.ascontiguousarray(policy, np.int32)
        ctrl = np.ascontiguousarray(ctrl, np.int32)
        rc = hisparse_state_import(self.handle, req, layer, slot_key.ctypes.data,
                                   policy.ctypes.data, ctrl.ctypes.data, _stream(stream))
        return _check(rc, "hisparse_state_import")

    def error_flags(self, clear: bool = True, stream=None) -> int:
        return hisparse_get_error_flags(self.handle, clear, _stream(stream))

    def profile(self, enable: bool):
        hisparse_profile_enable(self.handle, enable)

    def profile_read(self) -> dict:
        return hisparse_profile_read(self.handle)


class TopkIndexBuilder:
    """Top-k selection + index-table build for `batch` rows of up to
    `max_len` scores (torch tensors on one device).  Holds the plan of the
    current sequence lengths, the candidate workspace and an error word;
    :meth:`plan` once per step, :meth:`build` once per layer."""

    def __init__(self, batch: int, max_len: int, k: int, device="cuda"):
        self.batch, self.max_len, self.k = batch, max_len, k
        ints = hisparse_topk_plan_ints(batch, max_len)
        if ints == 0:
            raise HiSparseError(HISPARSE_E_INVAL, "hisparse_topk_plan_ints")
        c = HisparseTopkCall(batch=batch, max_len=max_len, k=k)
        code = hisparse_topk_index_build(c, 0)      # shape check only: rejected before launch
        if code == HISPARSE_E_UNSUPPORTED:
            raise HiSparseError(code, "hisparse_topk_index_build")
        self.plan_buf = torch.zeros(ints, dtype=torch.int32, device=device)
        ws = hisparse_topk_workspace_bytes(batch, max_len, k)
        self.workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=device)
        self.workspace_bytes = ws
        self.err = torch.zeros(1, dtype=torch.int32, device=device)

    def plan(self, seq_lens: torch.Tensor, stream=None):
        assert seq_lens.dtype == torch.int32 and seq_lens.numel() == self.batch
        _check(hisparse_topk_plan(self.batch, self.max_len, _ptr(seq_lens), _ptr(self.plan_buf),
                                  self.plan_buf.numel(), _stream(stream)), "hisparse_topk_plan")

    def build(self, logits: torch.Tensor, seq_lens: torch.Tensor, indices: torch.Tensor,
              locs: torch.Tensor | None = None, mode: str = "none", page_table=None,
              page_size: int = 1, row_offsets=None, stream=None, noalloc: bool = False):
        """noalloc: call hisparse_topk_index_build_noalloc (the library's fixed
        scratch instead of this builder's workspace)."""
        assert logits.dtype == torch.float32 and logits.is_contiguous()
        assert tuple(logits.shape) == (self.batch, self.max_len)
        assert tuple(indices.shape) == (self.batch, self.k) and indices.dtype == torch.int32
        c = HisparseTopkCall()
        c.batch, c.max_len, c.k = self.batch, self.max_len, self.k
        c.logits = logits.data_ptr()
        c.seq_lens = _ptr(seq_lens)
        c.plan = _ptr(self.plan_buf)
        c.plan_ints = self.plan_buf.numel()
        c.mode = INDEX_MODE[mode]
        c.page_table = _ptr(page_table)
        c.pt_stride = 0 if page_table is None else page_table.shape[1]
        c.page_size = page_size
        c.row_offsets = _ptr(row_offsets)
        c.indices = _ptr(indices)
        c.locs = _ptr(locs)
        c.workspace = self.workspace.data_ptr() if self.workspace_bytes and not noalloc else None
        c.workspace_bytes = 0 if noalloc else self.workspace_bytes
        c.error_word = _ptr(self.err)
        if noalloc:
            _check(hisparse_topk_index_build_noalloc(c, _stream(stream)),
                   "hisparse_topk_index_build_noalloc")
        else:
            _check(hisparse_topk_index_build(c, _stream(stream)), "hisparse_topk_index_build")

    def error_flags(self, clear: bool = True) -> int:
        v = int(self.err.item()) & 0xFFFFFFFF
        if clear:
            self.err.zero_()
        return v
