"""Thin Python binding of libpakv (ctypes). Argument marshalling only: every
step of the attention path runs in the library's HIP kernels.

Tensors are torch tensors on the GPU; BF16 data may be ``torch.bfloat16`` or
``torch.int16`` bit patterns. Work is queued on torch's current stream unless
a stream is given. The library never allocates device memory, so outputs and
the decode workspace are allocated here with torch when not supplied.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpakv.so")

PA_OK = 0
PA_ERR_INVALID = 2
PA_ERR_WORKSPACE = 5
PA_ERR_CAPACITY = 7
PA_ERR_STATE = 8
STATUS_NAMES = {7: "PA_ERR_CAPACITY", 8: "PA_ERR_STATE",
                0: "PA_OK", 1: "PA_ERR_NULL", 2: "PA_ERR_INVALID", 3: "PA_ERR_UNSUPPORTED",
                4: "PA_ERR_ALIGN", 5: "PA_ERR_WORKSPACE", 6: "PA_ERR_LAUNCH"}
EXPORTS = ["pa_pool_create", "pa_pool_destroy", "pa_kv_append", "pa_decode_workspace_bytes",
           "pa_split_tokens", "pa_decode", "pa_decode_append", "pa_status_str", "pa_profile_start",
           "pa_profile_stop", "pa_stream_read", "pa_decode_plan_capacity", "pa_decode_plan",
           "pa_decode_planned", "pa_sched_create", "pa_sched_destroy", "pa_sched_submit",
           "pa_sched_submit_shared", "pa_sched_admit", "pa_sched_slot", "pa_sched_advance",
           "pa_sched_finish", "pa_sched_block_tables", "pa_sched_context_lens", "pa_sched_stats",
           "pa_kv_write", "pa_prefill", "pa_prefill_plan_capacity", "pa_prefill_plan",
           "pa_prefill_planned", "pa_decode_planned_host", "pa_decode_static"]

_lib = None


class PakvError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS_NAMES.get(status, status)} ({status_str(status)})")


def lib() -> ctypes.CDLL:
    """Load libpakv.so from the package directory (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run python -m paged_kv_decode_02_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    c = ctypes
    L.pa_pool_create.argtypes = [c.POINTER(c.c_void_p), c.c_void_p, c.c_void_p, c.c_int32,
                                 c.c_int32, c.c_int32, c.c_int32]
    L.pa_pool_create.restype = c.c_int
    L.pa_pool_destroy.argtypes = [c.c_void_p]
    L.pa_pool_destroy.restype = None
    L.pa_kv_append.argtypes = [c.c_void_p, c.c_void_p, c.c_void_p, c.c_int32, c.c_void_p,
                               c.c_int32, c.c_void_p, c.c_void_p]
    L.pa_kv_append.restype = c.c_int
    L.pa_decode_workspace_bytes.argtypes = [c.c_void_p, c.c_int32, c.c_int32, c.c_int32]
    L.pa_decode_workspace_bytes.restype = c.c_size_t
    L.pa_split_tokens.argtypes = [c.c_int32]
    L.pa_split_tokens.restype = c.c_int32
    L.pa_decode.argtypes = [c.c_void_p, c.c_void_p, c.c_int32, c.c_int32, c.c_void_p, c.c_int32,
                            c.c_void_p, c.c_float, c.c_void_p, c.c_void_p, c.c_size_t, c.c_void_p]
    L.pa_decode.restype = c.c_int
    L.pa_decode_append.argtypes = [c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p,
                                   c.c_int32, c.c_int32, c.c_void_p, c.c_int32, c.c_void_p,
                                   c.c_float, c.c_void_p, c.c_void_p, c.c_size_t, c.c_void_p]
    L.pa_decode_append.restype = c.c_int
    L.pa_status_str.argtypes = [c.c_int]
    L.pa_status_str.restype = c.c_char_p
    L.pa_profile_start.argtypes = []
    L.pa_profile_start.restype = c.c_int
    L.pa_profile_stop.argtypes = [c.POINTER(c.c_double), c.POINTER(c.c_int64)]
    L.pa_profile_stop.restype = c.c_int
    L.pa_stream_read.argtypes = [c.c_void_p, c.c_size_t, c.c_void_p, c.c_void_p]
    L.pa_stream_read.restype = c.c_int
    L.pa_decode_plan_capacity.argtypes = [c.c_void_p, c.c_int32, c.c_int32]
    L.pa_decode_plan_capacity.restype = c.c_int64
    L.pa_decode_plan.argtypes = [c.c_void_p, c.c_void_p, c.c_int32, c.c_int32, c.c_int32, c.c_void_p,
                                 c.c_int64, c.POINTER(c.c_int32)]
    L.pa_decode_plan.restype = c.c_int
    L.pa_decode_planned.argtypes = [c.c_void_p, c.c_void_p, c.c_int32, c.c_int32, c.c_void_p, c.c_int32,
                                    c.c_void_p, c.c_float, c.c_void_p, c.c_void_p, c.c_size_t,
                                    c.c_void_p, c.c_int32, c.c_void_p]
    L.pa_decode_planned.restype = c.c_int
    L.pa_decode_planned_host.argtypes = list(L.pa_decode_planned.argtypes)
    L.pa_decode_planned_host.restype = c.c_int
    L.pa_decode_static.argtypes = [c.c_void_p, c.c_void_p, c.c_int32, c.c_int32, c.c_void_p, c.c_int32,
                                   c.c_void_p, c.c_float, c.c_void_p, c.c_void_p]
    L.pa_decode_static.restype = c.c_int
    i32p, i64p = c.POINTER(c.c_int32), c.POINTER(c.c_int64)
    L.pa_sched_create.argtypes = [c.POINTER(c.c_void_p), c.c_int32, c.c_int32, c.c_int32, c.c_int32,
                                  c.c_int32]
    L.pa_sched_create.restype = c.c_int
    L.pa_sched_destroy.argtypes = [c.c_void_p]
    L.pa_sched_destroy.restype = None
    L.pa_sched_submit.argtypes = [c.c_void_p, c.c_int32, c.c_int32, i64p]
    L.pa_sched_submit.restype = c.c_int
    L.pa_sched_submit_shared.argtypes = [c.c_void_p, c.c_int64, c.c_int32, c.c_int32, c.c_int32, i64p]
    L.pa_sched_submit_shared.restype = c.c_int
    L.pa_sched_admit.argtypes = [c.c_void_p, c.c_void_p, c.c_int32, i32p]
    L.pa_sched_admit.restype = c.c_int
    L.pa_sched_slot.argtypes = [c.c_void_p, c.c_int64, i32p]
    L.pa_sched_slot.restype = c.c_int
    L.pa_sched_advance.argtypes = [c.c_void_p, c.c_int64, c.c_int32]
    L.pa_sched_advance.restype = c.c_int
    L.pa_sched_finish.argtypes = [c.c_void_p, c.c_int64]
    L.pa_sched_finish.restype = c.c_int
    L.pa_sched_block_tables.argtypes = [c.c_void_p]
    L.pa_sched_block_tables.restype = i32p
    L.pa_sched_context_lens.argtypes = [c.c_void_p]
    L.pa_sched_context_lens.restype = i32p
    L.pa_sched_stats.argtypes = [c.c_void_p, i32p, i32p, i32p]
    L.pa_sched_stats.restype = c.c_int
    L.pa_kv_write.argtypes = [c.c_void_p, c.c_void_p, c.c_void_p, c.c_int32, c.c_int32, c.c_int32,
                              c.c_void_p, c.c_void_p, c.c_int32, c.c_void_p, c.c_void_p]
    L.pa_kv_write.restype = c.c_int
    L.pa_prefill.argtypes = [c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p, c.c_int32, c.c_int32,
                             c.c_int32, c.c_int32, c.c_void_p, c.c_void_p, c.c_int32, c.c_void_p,
                             c.c_float, c.c_void_p, c.c_void_p]
    L.pa_prefill.restype = c.c_int
    L.pa_prefill_plan_capacity.argtypes = [c.c_void_p, c.c_int32, c.c_int32, c.c_int32]
    L.pa_prefill_plan_capacity.restype = c.c_int64
    L.pa_prefill_plan.argtypes = [c.c_void_p, c.c_void_p, c.c_void_p, c.c_int32, c.c_int32, c.c_int32,
                                  c.c_int32, c.c_void_p, c.c_int64, c.POINTER(c.c_int32)]
    L.pa_prefill_plan.restype = c.c_int
    L.pa_prefill_planned.argtypes = [c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p, c.c_int32, c.c_int32,
                                     c.c_int32, c.c_int32, c.c_void_p, c.c_void_p, c.c_int32, c.c_void_p,
                                     c.c_float, c.c_void_p, c.c_void_p, c.c_int32, c.c_void_p]
    L.pa_prefill_planned.restype = c.c_int
    _lib = L
    return L


def status_str(status: int) -> str:
    return lib().pa_status_str(int(status)).decode()


def _check(status: int, what: str):
    if status != PA_OK:
        raise PakvError(status, what)


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _need(t, name, dtypes, ndim=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name}: expected {ndim} dims, got {tuple(t.shape)}")


def _shape(t, name, expected):
    if tuple(t.shape) != tuple(expected):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(expected)}")


def _same_device(pool, *tensors):
    dev = pool.k_pages.device
    for t in tensors:
        if t is not None and t.device != dev:
            raise ValueError(f"tensor on {t.device}, pool on {dev}")


def _check_decode_args(pool, q, block_tables, context_lens, out):
    """Shapes of a decode call against the pool and the batch: q ``[B][Hq][d]``
    with d the pool's head_dim and Hq a multiple of its KV heads, one block
    table row and one context length per sequence, out ``[B][Hq][d]``."""
    num_seqs, num_q_heads, d = q.shape
    if d != pool.head_dim:
        raise ValueError(f"q head_dim {d} != pool head_dim {pool.head_dim}")
    if num_q_heads % pool.num_kv_heads != 0:
        raise ValueError(f"{num_q_heads} query heads are not a multiple of {pool.num_kv_heads} KV heads")
    if block_tables.shape[0] != num_seqs:
        raise ValueError(f"block_tables has {block_tables.shape[0]} rows for {num_seqs} sequences")
    if context_lens.numel() != num_seqs:
        raise ValueError(f"context_lens has {context_lens.numel()} values for {num_seqs} sequences")
    if out is not None:
        _shape(out, "out", (num_seqs, num_q_heads, d))
    _same_device(pool, q, block_tables, context_lens, out)


def _check_new_rows(pool, num_seqs, k_new, v_new, positions):
    """k_new / v_new ``[B][Hkv][d]`` and one position per sequence."""
    want = (num_seqs, pool.num_kv_heads, pool.head_dim)
    _shape(k_new, "k_new", want)
    _shape(v_new, "v_new", want)
    if positions.numel() != num_seqs:
        raise ValueError(f"positions has {positions.numel()} values for {num_seqs} sequences")
    _same_device(pool, k_new, v_new, positions)


def _bf16_types():
    import torch
    return (torch.bfloat16, torch.int16)


class Pool:
    """A caller-owned K/V page pool: K ``[P][Hkv][d/32][16][32]``, V
    ``[P][Hkv][d][16]``."""

    def __init__(self, k_pages, v_pages):
        _need(k_pages, "k_pages", _bf16_types(), 5)
        _need(v_pages, "v_pages", _bf16_types(), 4)
        num_pages, hkv, slabs, page, width = k_pages.shape
        d = slabs * width
        if width != 32:
            raise ValueError(f"k_pages shape {tuple(k_pages.shape)}: the last dim holds 32 head dims")
        if tuple(v_pages.shape) != (num_pages, hkv, d, page):
            raise ValueError(f"v_pages shape {tuple(v_pages.shape)} does not match K {tuple(k_pages.shape)}")
        handle = ctypes.c_void_p()
        _check(lib().pa_pool_create(ctypes.byref(handle), _ptr(k_pages), _ptr(v_pages), num_pages,
                                    page, hkv, d), "pa_pool_create")
        self.handle = handle
        self.k_pages, self.v_pages = k_pages, v_pages
        self.num_pages, self.num_kv_heads, self.page_size, self.head_dim = num_pages, hkv, page, d

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            lib().pa_pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def split_tokens(head_dim: int) -> int:
    return int(lib().pa_split_tokens(head_dim))


def decode_workspace_bytes(pool: Pool, num_seqs: int, num_q_heads: int, max_pages_per_seq: int) -> int:
    return int(lib().pa_decode_workspace_bytes(pool.handle, num_seqs, num_q_heads, max_pages_per_seq))


def kv_append(pool: Pool, k_new, v_new, block_tables, positions, stream=None):
    """Write the new token's K/V (``[B][Hkv][d]``) at ``positions`` (pa_kv_append)."""
    import torch
    _need(k_new, "k_new", _bf16_types(), 3)
    _need(v_new, "v_new", _bf16_types(), 3)
    _need(block_tables, "block_tables", (torch.int32,), 2)
    _need(positions, "positions", (torch.int32,), 1)
    num_seqs = block_tables.shape[0]
    _check_new_rows(pool, num_seqs, k_new, v_new, positions)
    _same_device(pool, block_tables)
    _check(lib().pa_kv_append(pool.handle, _ptr(k_new), _ptr(v_new), num_seqs, _ptr(block_tables),
                              block_tables.shape[1], _ptr(positions), _stream(stream)),
           "pa_kv_append")


def decode(pool: Pool, q, block_tables, context_lens, scale: float, out=None, workspace=None,
           stream=None):
    """Paged decode attention (pa_decode). Returns ``out`` (FP32 ``[B][Hq][d]``)."""
    import torch
    _need(q, "q", _bf16_types(), 3)
    _need(block_tables, "block_tables", (torch.int32,), 2)
    _need(context_lens, "context_lens", (torch.int32,), 1)
    _check_decode_args(pool, q, block_tables, context_lens, out)
    num_seqs, num_q_heads, d = q.shape
    stride = block_tables.shape[1]
    if out is None:
        out = torch.empty((num_seqs, num_q_heads, d), dtype=torch.float32, device=q.device)
    _need(out, "out", (torch.float32,), 3)
    need = decode_workspace_bytes(pool, num_seqs, num_q_heads, stride)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pa_decode(pool.handle, _ptr(q), num_seqs, num_q_heads, _ptr(block_tables), stride,
                           _ptr(context_lens), float(scale), _ptr(out), _ptr(workspace), ws_bytes,
                           _stream(stream)), "pa_decode")
    return out


def decode_static(pool: Pool, q, block_tables, context_lens, scale: float, out=None, stream=None):
    """pa_decode with the library's static scratch instead of a workspace
    (pa_decode_static: nothing allocated on the device by the call)."""
    import torch
    _need(q, "q", _bf16_types(), 3)
    _need(block_tables, "block_tables", (torch.int32,), 2)
    _need(context_lens, "context_lens", (torch.int32,), 1)
    _check_decode_args(pool, q, block_tables, context_lens, out)
    num_seqs, num_q_heads, d = q.shape
    if out is None:
        out = torch.empty((num_seqs, num_q_heads, d), dtype=torch.float32, device=q.device)
    _need(out, "out", (torch.float32,), 3)
    _check(lib().pa_decode_static(pool.handle, _ptr(q), num_seqs, num_q_heads, _ptr(block_tables),
                                  block_tables.shape[1], _ptr(context_lens), float(scale), _ptr(out),
                                  _stream(stream)), "pa_decode_static")
    return out


def decode_plan_capacity(pool: Pool, num_seqs: int, max_pages_per_seq: int) -> int:
    """int32 words a decode plan may need (pa_decode_plan_capacity)."""
    cap = int(lib().pa_decode_plan_capacity(pool.handle, int(num_seqs), int(max_pages_per_seq)))
    if cap < 0:
        raise PakvError(PA_ERR_INVALID, "pa_decode_plan_capacity")
    return cap


def decode_plan_into(pool: Pool, context_lens_host, num_q_heads: int, max_pages_per_seq: int, out) -> int:
    """Write the launch plan for these host context lengths into ``out`` (host
    int32 memory: a numpy array or a CPU torch tensor, e.g. pinned, of at least
    decode_plan_capacity words); returns the number of words (pa_decode_plan)."""
    import numpy as np
    ctx = np.ascontiguousarray(np.asarray(context_lens_host, dtype=np.int32))
    if ctx.ndim != 1:
        raise ValueError("context_lens_host must be 1-D")
    if isinstance(out, np.ndarray):
        if out.dtype != np.int32 or not out.flags.c_contiguous:
            raise ValueError("out must be a contiguous int32 array")
        addr, size = out.ctypes.data, out.size
    else:
        import torch
        if out.dtype != torch.int32 or out.is_cuda or not out.is_contiguous():
            raise ValueError("out must be a contiguous host int32 tensor")
        addr, size = out.data_ptr(), out.numel()
    n = ctypes.c_int32(0)
    _check(lib().pa_decode_plan(pool.handle, ctx.ctypes.data, ctx.size, int(num_q_heads),
                                int(max_pages_per_seq), addr, size, ctypes.byref(n)), "pa_decode_plan")
    return n.value


def decode_plan(pool: Pool, context_lens_host, num_q_heads: int, max_pages_per_seq: int):
    """Host-side launch plan for these context lengths (pa_decode_plan): an int32
    numpy array of work items, 8 words each (units ``b | split << 20`` or -1,
    then their rotations), the largest item first."""
    import numpy as np
    num_seqs = np.asarray(context_lens_host).size
    plan = np.zeros(max(decode_plan_capacity(pool, num_seqs, max_pages_per_seq), 1), dtype=np.int32)
    n = decode_plan_into(pool, context_lens_host, num_q_heads, max_pages_per_seq, plan)
    return plan[:n].copy()


def decode_planned(pool: Pool, q, block_tables, context_lens, scale: float, plan, out=None,
                   workspace=None, stream=None):
    """pa_decode driven by a launch plan (pa_decode_planned); ``plan`` is a device
    int32 tensor holding what decode_plan returned for the same lengths."""
    import torch
    _need(q, "q", _bf16_types(), 3)
    _need(block_tables, "block_tables", (torch.int32,), 2)
    _need(context_lens, "context_lens", (torch.int32,), 1)
    _need(plan, "plan", (torch.int32,), 1)
    _check_decode_args(pool, q, block_tables, context_lens, out)
    _same_device(pool, plan)
    num_seqs, num_q_heads, d = q.shape
    stride = block_tables.shape[1]
    if out is None:
        out = torch.empty((num_seqs, num_q_heads, d), dtype=torch.float32, device=q.device)
    _need(out, "out", (torch.float32,), 3)
    need = decode_workspace_bytes(pool, num_seqs, num_q_heads, stride)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pa_decode_planned(pool.handle, _ptr(q), num_seqs, num_q_heads, _ptr(block_tables),
                                   stride, _ptr(context_lens), float(scale), _ptr(out), _ptr(workspace),
                                   ws_bytes, _ptr(plan), plan.numel(), _stream(stream)),
           "pa_decode_planned")
    return out


def _host_plan_array(plan_host):
    import numpy as np
    if not isinstance(plan_host, np.ndarray) or plan_host.dtype != np.int32 or plan_host.ndim != 1 \
            or not plan_host.flags.c_contiguous:
        raise ValueError("plan_host must be a contiguous 1-D int32 numpy array")
    return plan_host


def decode_planned_host(pool: Pool, q, block_tables, context_lens, scale: float, plan_host, out=None,
                        workspace=None, stream=None):
    """pa_decode driven by a plan in host memory (pa_decode_planned_host):
    ``plan_host`` is the int32 numpy array decode_plan returned (at most 2048
    words); it travels in the kernel's arguments, so no device copy is made."""
    import torch
    _need(q, "q", _bf16_types(), 3)
    _need(block_tables, "block_tables", (torch.int32,), 2)
    _need(context_lens, "context_lens", (torch.int32,), 1)
    plan_host = _host_plan_array(plan_host)
    _check_decode_args(pool, q, block_tables, context_lens, out)
    num_seqs, num_q_heads, d = q.shape
    stride = block_tables.shape[1]
    if out is None:
        out = torch.empty((num_seqs, num_q_heads, d), dtype=torch.float32, device=q.device)
    _need(out, "out", (torch.float32,), 3)
    need = decode_workspace_bytes(pool, num_seqs, num_q_heads, stride)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pa_decode_planned_host(pool.handle, _ptr(q), num_seqs, num_q_heads, _ptr(block_tables),
                                        stride, _ptr(context_lens), float(scale), _ptr(out), _ptr(workspace),
                                        ws_bytes, plan_host.ctypes.data, plan_host.size, _stream(stream)),
           "pa_decode_planned_host")
    return out


class HostPlan:
    """A host buffer for the decode plans of one batch shape, remade by one C
    call (pa_decode_plan) from the current contents of ``context_lens_host``
    (a contiguous int32 numpy array the caller keeps updating). ``make()``
    returns the plan's length in words; the words are in ``buf``."""

    def __init__(self, pool: Pool, context_lens_host, num_q_heads: int, max_pages_per_seq: int):
        import numpy as np
        ctx = context_lens_host
        if not isinstance(ctx, np.ndarray) or ctx.dtype != np.int32 or ctx.ndim != 1 or not ctx.flags.c_contiguous:
            raise ValueError("context_lens_host must be a contiguous 1-D int32 numpy array")
        self.ctx = ctx
        self.cap = decode_plan_capacity(pool, ctx.size, max_pages_per_seq)
        self.buf = np.zeros(max(self.cap, 1), dtype=np.int32)
        self.words = 0
        self._n = ctypes.c_int32(0)
        self._call = (lib().pa_decode_plan, pool.handle, ctx.ctypes.data, ctx.size, int(num_q_heads),
                      int(max_pages_per_seq), self.buf.ctypes.data, self.cap, ctypes.byref(self._n))
        self._pool = pool   # keeps the descriptor alive

    def make(self) -> int:
        f, *args = self._call
        _check(f(*args), "pa_decode_plan")
        self.words = self._n.value
        return self.words


INLINE_PLAN_WORDS = 2048   # plans this small travel in the kernel's arguments (8 KiB)


class DevicePlan:
    """A HostPlan plus a device copy: ``upload(stream)`` remakes the plan on the
    host, stages it in one of two pinned buffers and queues its copy to the
    device buffer on ``stream`` (a staging buffer is reused only after the copy
    that read it has run). For plans too large to travel in the kernel's
    arguments; one upload serves every layer of a step."""

    def __init__(self, pool: Pool, context_lens_host, num_q_heads: int, max_pages_per_seq: int, device):
        import torch
        self.host = HostPlan(pool, context_lens_host, num_q_heads, max_pages_per_seq)
        self.ctx = self.host.ctx
        cap = max(self.host.cap, 1)
        self.pinned = [torch.empty(cap, dtype=torch.int32, pin_memory=True) for _ in range(2)]
        self.pinned_np = [t.numpy() for t in self.pinned]
        self.done = [None, None]
        self.dev = torch.empty(cap, dtype=torch.int32, device=device)
        self.words = 0
        self._k = 0

    def upload(self, stream) -> int:
        import torch
        words = self.host.make()
        k = self._k
        self._k ^= 1
        if self.done[k] is not None:
            self.done[k].synchronize()
        self.pinned_np[k][:words] = self.host.buf[:words]
        with torch.cuda.stream(stream):
            self.dev[:words].copy_(self.pinned[k][:words], non_blocking=True)
            ev = torch.cuda.Event()
            ev.record(stream)
        self.done[k] = ev
        self.words = words
        return words


class PreparedDecode:
    """A planned decode launch with its arguments checked and marshalled once:
    calling it queues the decode of this layer with the plan's current words,
    pa_decode_planned_host for a HostPlan (the plan in the kernel's
    arguments; at most 2048 words) or pa_decode_planned for a DevicePlan. The
    tensors must stay alive and unchanged in shape (their contents may
    change)."""

    def __init__(self, pool: Pool, q, block_tables, context_lens, scale: float, plan, out,
                 workspace=None, stream=None):
        import torch
        _need(q, "q", _bf16_types(), 3)
        _need(block_tables, "block_tables", (torch.int32,), 2)
        _need(context_lens, "context_lens", (torch.int32,), 1)
        _need(out, "out", (torch.float32,), 3)
        _check_decode_args(pool, q, block_tables, context_lens, out)
        num_seqs, num_q_heads, _ = q.shape
        if plan.ctx.size != num_seqs:
            raise ValueError("the plan is for another batch size")
        stride = block_tables.shape[1]
        need = decode_workspace_bytes(pool, num_seqs, num_q_heads, stride)
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        if ws_bytes < need:
            raise ValueError(f"workspace of {ws_bytes} bytes, {need} needed")
        self._keep = (pool, q, block_tables, context_lens, out, workspace, plan)
        self._plan = plan
        on_device = isinstance(plan, DevicePlan)
        self._name = "pa_decode_planned" if on_device else "pa_decode_planned_host"
        self._f = getattr(lib(), self._name)
        self._args = (pool.handle, _ptr(q), num_seqs, num_q_heads, _ptr(block_tables), stride,
                      _ptr(context_lens), float(scale), _ptr(out), _ptr(workspace), ws_bytes,
                      _ptr(plan.dev) if on_device else plan.buf.ctypes.data)
        self._stream = _stream(stream)

    def __call__(self):
        st = self._f(*self._args, self._plan.words, self._stream)
        if st != PA_OK:
            raise PakvError(st, self._name)


class PreparedAppend:
    """pa_kv_append with its arguments checked and marshalled once."""

    def __init__(self, pool: Pool, k_new, v_new, block_tables, positions, stream=None):
        import torch
        _need(k_new, "k_new", _bf16_types(), 3)
        _need(v_new, "v_new", _bf16_types(), 3)
        _need(block_tables, "block_tables", (torch.int32,), 2)
        _need(positions, "positions", (torch.int32,), 1)
        num_seqs = block_tables.shape[0]
        _check_new_rows(pool, num_seqs, k_new, v_new, positions)
        _same_device(pool, block_tables)
        self._keep = (pool, k_new, v_new, block_tables, positions)
        self._f = lib().pa_kv_append
        self._args = (pool.handle, _ptr(k_new), _ptr(v_new), num_seqs, _ptr(block_tables), block_tables.shape[1],
                      _ptr(positions), _stream(stream))

    def __call__(self):
        st = self._f(*self._args)
        if st != PA_OK:
            raise PakvError(st, "pa_kv_append")


def _chunk_common(q_or_k, query_start, block_tables, context_lens, max_chunk):
    import torch
    _need(query_start, "query_start", (torch.int32,), 1)
    _need(block_tables, "block_tables", (torch.int32,), 2)
    _need(context_lens, "context_lens", (torch.int32,), 1)
    num_seqs = block_tables.shape[0]
    if query_start.numel() != num_seqs + 1 or context_lens.numel() != num_seqs:
        raise ValueError("query_start must hold num_seqs + 1 offsets and context_lens num_seqs values")
    return num_seqs, q_or_k.shape[0], block_tables.shape[1], int(max_chunk)


def _check_chunk_rows(pool, num_rows, k_rows, v_rows, q=None, out=None, *others):
    """Chunk rows: k_rows / v_rows ``[N][Hkv][d]``, q and out ``[N][Hq][d]`` with
    Hq a multiple of the pool's KV heads and d its head_dim."""
    want = (num_rows, pool.num_kv_heads, pool.head_dim)
    _shape(k_rows, "k_rows", want)
    _shape(v_rows, "v_rows", want)
    if q is not None:
        if q.shape[2] != pool.head_dim or q.shape[1] % pool.num_kv_heads != 0:
            raise ValueError(f"q shape {tuple(q.shape)} does not fit the pool "
                             f"({pool.num_kv_heads} KV heads, head_dim {pool.head_dim})")
        if out is not None:
            _shape(out, "out", tuple(q.shape))
    _same_device(pool, k_rows, v_rows, q, out, *others)


def kv_write(pool: Pool, k_rows, v_rows, query_start, block_tables, context_lens, max_chunk: int,
             stream=None):
    """Write chunks of new tokens' K/V (``[N][Hkv][d]``) into their pages (pa_kv_write)."""
    _need(k_rows, "k_rows", _bf16_types(), 3)
    _need(v_rows, "v_rows", _bf16_types(), 3)
    num_seqs, num_rows, stride, max_chunk = _chunk_common(k_rows, query_start, block_tables,
                                                          context_lens, max_chunk)
    _check_chunk_rows(pool, num_rows, k_rows, v_rows, None, None, query_start, block_tables, context_lens)
    _check(lib().pa_kv_write(pool.handle, _ptr(k_rows), _ptr(v_rows), num_seqs, num_rows, max_chunk,
                             _ptr(query_start), _ptr(block_tables), stride, _ptr(context_lens),
                             _stream(stream)), "pa_kv_write")


def prefill(pool: Pool, q, k_rows, v_rows, query_start, block_tables, context_lens, scale: float,
            max_chunk: int, out=None, stream=None):
    """Paged prefill (pa_prefill): write the chunks' K/V, then causal attention for
    every chunk row. Returns ``out`` (FP32 ``[N][Hq][d]``)."""
    import torch
    _need(q, "q", _bf16_types(), 3)
    _need(k_rows, "k_rows", _bf16_types(), 3)
    _need(v_rows, "v_rows", _bf16_types(), 3)
    num_seqs, num_rows, stride, max_chunk = _chunk_common(q, query_start, block_tables, context_lens,
                                                          max_chunk)
    if out is not None:
        _need(out, "out", (torch.float32,), 3)
    _check_chunk_rows(pool, num_rows, k_rows, v_rows, q, out, query_start, block_tables, context_lens)
    if out is None:
        out = torch.empty(tuple(q.shape), dtype=torch.float32, device=q.device)
    _check(lib().pa_prefill(pool.handle, _ptr(q), _ptr(k_rows), _ptr(v_rows), num_seqs, q.shape[1],
                            num_rows, max_chunk, _ptr(query_start), _ptr(block_tables), stride,
                            _ptr(context_lens), float(scale), _ptr(out), _stream(stream)),
           "pa_prefill")
    return out


def prefill_plan_capacity(pool: Pool, num_seqs: int, num_q_heads: int, max_chunk: int) -> int:
    cap = int(lib().pa_prefill_plan_capacity(pool.handle, int(num_seqs), int(num_q_heads), int(max_chunk)))
    if cap < 0:
        raise PakvError(PA_ERR_INVALID, "pa_prefill_plan_capacity")
    return cap


def _host_i32(a, name):
    import numpy as np
    a = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    if a.ndim != 1:
        raise ValueError(f"{name} must be 1-D")
    return a


def prefill_plan_into(pool: Pool, context_lens_host, chunk_lens_host, num_q_heads: int,
                      max_pages_per_seq: int, max_chunk: int, out) -> int:
    """Write the prefill launch plan for these host lengths into ``out`` (host
    int32 memory of at least prefill_plan_capacity items: a numpy array or a CPU
    torch tensor, e.g. pinned); returns the number of items (pa_prefill_plan)."""
    import numpy as np
    ctx = _host_i32(context_lens_host, "context_lens_host")
    chunks = _host_i32(chunk_lens_host, "chunk_lens_host")
    if chunks.size != ctx.size:
        raise ValueError("context_lens_host and chunk_lens_host differ in length")
    if isinstance(out, np.ndarray):
        if out.dtype != np.int32 or not out.flags.c_contiguous:
            raise ValueError("out must be a contiguous int32 array")
        addr, size = out.ctypes.data, out.size
    else:
        import torch
        if out.dtype != torch.int32 or out.is_cuda or not out.is_contiguous():
            raise ValueError("out must be a contiguous host int32 tensor")
        addr, size = out.data_ptr(), out.numel()
    n = ctypes.c_int32(0)
    _check(lib().pa_prefill_plan(pool.handle, ctx.ctypes.data, chunks.ctypes.data, ctx.size,
                                 int(num_q_heads), int(max_pages_per_seq), int(max_chunk), addr, size,
                                 ctypes.byref(n)), "pa_prefill_plan")
    return n.value


def prefill_plan(pool: Pool, context_lens_host, chunk_lens_host, num_q_heads: int, max_pages_per_seq: int,
                 max_chunk: int):
    """Host-side prefill launch plan (pa_prefill_plan): an int32 numpy array of
    items ``b | row_block << 20``, the costliest row block first."""
    import numpy as np
    num_seqs = np.asarray(context_lens_host).size
    cap = prefill_plan_capacity(pool, num_seqs, num_q_heads, max_chunk)
    plan = np.zeros(max(cap, 1), dtype=np.int32)
    n = prefill_plan_into(pool, context_lens_host, chunk_lens_host, num_q_heads, max_pages_per_seq,
                          max_chunk, plan)
    return plan[:n].copy()


def prefill_planned(pool: Pool, q, k_rows, v_rows, query_start, block_tables, context_lens, scale: float,
                    max_chunk: int, plan, out=None, stream=None):
    """pa_prefill driven by a launch plan (pa_prefill_planned); ``plan`` is a
    device int32 tensor holding what prefill_plan returned for the same lengths."""
    import torch
    _need(q, "q", _bf16_types(), 3)
    _need(k_rows, "k_rows", _bf16_types(), 3)
    _need(v_rows, "v_rows", _bf16_types(), 3)
    _need(plan, "plan", (torch.int32,), 1)
    num_seqs, num_rows, stride, max_chunk = _chunk_common(q, query_start, block_tables, context_lens,
                                                          max_chunk)
    if out is not None:
        _need(out, "out", (torch.float32,), 3)
    _check_chunk_rows(pool, num_rows, k_rows, v_rows, q, out, query_start, block_tables, context_lens)
    if out is None:
        out = torch.empty(tuple(q.shape), dtype=torch.float32, device=q.device)
    _check(lib().pa_prefill_planned(pool.handle, _ptr(q), _ptr(k_rows), _ptr(v_rows), num_seqs, q.shape[1],
                                    num_rows, max_chunk, _ptr(query_start), _ptr(block_tables), stride,
                                    _ptr(context_lens), float(scale), _ptr(out), _ptr(plan), plan.numel(),
                                    _stream(stream)), "pa_prefill_planned")
    return out


def decode_append(pool: Pool, q, k_new, v_new, positions, block_tables, context_lens, scale: float,
                  out=None, workspace=None, stream=None):
    """Append each sequence's new token then decode, in one launch (pa_decode_append)."""
    import torch
    _need(q, "q", _bf16_types(), 3)
    _need(k_new, "k_new", _bf16_types(), 3)
    _need(v_new, "v_new", _bf16_types(), 3)
    _need(positions, "positions", (torch.int32,), 1)
    _need(block_tables, "block_tables", (torch.int32,), 2)
    _need(context_lens, "context_lens", (torch.int32,), 1)
    _check_decode_args(pool, q, block_tables, context_lens, out)
    _check_new_rows(pool, q.shape[0], k_new, v_new, positions)
    num_seqs, num_q_heads, d = q.shape
    stride = block_tables.shape[1]
    if out is None:
        out = torch.empty((num_seqs, num_q_heads, d), dtype=torch.float32, device=q.device)
    _need(out, "out", (torch.float32,), 3)
    need = decode_workspace_bytes(pool, num_seqs, num_q_heads, stride)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pa_decode_append(pool.handle, _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(positions),
                                  num_seqs, num_q_heads, _ptr(block_tables), stride,
                                  _ptr(context_lens), float(scale), _ptr(out), _ptr(workspace),
                                  ws_bytes, _stream(stream)), "pa_decode_append")
    return out


def profile_start():
    _check(lib().pa_profile_start(), "pa_profile_start")


PROFILE_KINDS = ("decode", "merge", "append", "write", "prefill")


def profile_stop():
    """Returns {kind: (ms, launches)} for the kinds in PROFILE_KINDS."""
    ms = (ctypes.c_double * len(PROFILE_KINDS))()
    n = (ctypes.c_int64 * len(PROFILE_KINDS))()
    _check(lib().pa_profile_stop(ms, n), "pa_profile_stop")
    return {k: (ms[i], n[i]) for i, k in enumerate(PROFILE_KINDS)}


def stream_read(src, sink, stream=None):
    """Read all of ``src`` with 16-byte loads (bandwidth ceiling measurement)."""
    nbytes = src.numel() * src.element_size()
    _check(lib().pa_stream_read(_ptr(src), nbytes, _ptr(sink), _stream(stream)), "pa_stream_read")


PA_BATCH_CONTINUOUS = 0
PA_BATCH_STATIC = 1


class Scheduler:
    """Host page allocator and FIFO admission over a shared page pool
    (pakv_sched.h). ``block_tables`` / ``context_lens`` are numpy views of the
    scheduler's own host arrays ([L][max_batch][max_pages_per_seq] and
    [max_batch]); they change as requests are admitted, advanced and finished."""

    def __init__(self, num_pages: int, num_layers: int, max_batch: int, max_pages_per_seq: int,
                 mode: int = PA_BATCH_CONTINUOUS):
        import numpy as np
        h = ctypes.c_void_p()
        _check(lib().pa_sched_create(ctypes.byref(h), num_pages, num_layers, max_batch,
                                     max_pages_per_seq, mode), "pa_sched_create")
        self.handle = h
        self.num_pages, self.num_layers = num_pages, num_layers
        self.max_batch, self.stride = max_batch, max_pages_per_seq
        bt = lib().pa_sched_block_tables(h)
        cl = lib().pa_sched_context_lens(h)
        self.block_tables = np.ctypeslib.as_array(bt, shape=(num_layers, max_batch, max_pages_per_seq))
        self.context_lens = np.ctypeslib.as_array(cl, shape=(max_batch,))

    def submit(self, prompt_tokens: int, max_new_tokens: int) -> int:
        rid = ctypes.c_int64(0)
        _check(lib().pa_sched_submit(self.handle, prompt_tokens, max_new_tokens, ctypes.byref(rid)),
               "pa_sched_submit")
        return rid.value

    def submit_shared(self, parent: int, shared_tokens: int, prompt_tokens: int,
                      max_new_tokens: int) -> int:
        rid = ctypes.c_int64(0)
        _check(lib().pa_sched_submit_shared(self.handle, parent, shared_tokens, prompt_tokens,
                                            max_new_tokens, ctypes.byref(rid)),
               "pa_sched_submit_shared")
        return rid.value

    def admit(self, capacity: Optional[int] = None):
        import numpy as np
        cap = self.max_batch if capacity is None else capacity
        out = np.zeros(max(cap, 1), dtype=np.int64)
        n = ctypes.c_int32(0)
        _check(lib().pa_sched_admit(self.handle, out.ctypes.data, cap, ctypes.byref(n)), "pa_sched_admit")
        return [int(x) for x in out[:n.value]]

    def slot(self, rid: int) -> int:
        s = ctypes.c_int32(0)
        _check(lib().pa_sched_slot(self.handle, rid, ctypes.byref(s)), "pa_sched_slot")
        return s.value

    def advance(self, rid: int, tokens: int = 1):
        _check(lib().pa_sched_advance(self.handle, rid, tokens), "pa_sched_advance")

    def finish(self, rid: int):
        _check(lib().pa_sched_finish(self.handle, rid), "pa_sched_finish")

    def stats(self):
        f, q, r = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int32(0)
        _check(lib().pa_sched_stats(self.handle, ctypes.byref(f), ctypes.byref(q), ctypes.byref(r)),
               "pa_sched_stats")
        return {"free_pages": f.value, "queued": q.value, "running": r.value}

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            lib().pa_sched_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
