"""ctypes binding of ``libnp_paged.so`` (the C ABI declared in np_paged.h).

Argument marshalling only: every check, plan and kernel runs in the native
library. torch is used for device memory and the current HIP stream. If the
library has not been built, importing the entry points raises at once; there
is no fallback path.
"""

from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libnp_paged.so")
TRACE_LIB_PATH = os.path.join(PKG, "libnp_paged_trace.so")

NP_F32, NP_F16, NP_BF16 = 0, 1, 2

STATUS_NAMES = [
    "NP_OK", "NP_ERR_NULL_PTR", "NP_ERR_BAD_DTYPE", "NP_ERR_BAD_SHAPE", "NP_ERR_BAD_STRIDE",
    "NP_ERR_MISALIGNED", "NP_ERR_BAD_GQA", "NP_ERR_BAD_CONTEXT_LEN", "NP_ERR_BAD_BLOCK_TABLE",
    "NP_ERR_UNSUPPORTED", "NP_ERR_WORKSPACE_TOO_SMALL", "NP_ERR_BAD_PLAN", "NP_ERR_HIP",
    "NP_ERR_POOL_EXHAUSTED",
]
STATUS = {name: i for i, name in enumerate(STATUS_NAMES)}


class NPError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        name = STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else str(status)
        super().__init__(f"{where}: {name} ({_lib().np_status_string(status).decode()})")


class Desc(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32), ("num_seqs", ctypes.c_int32), ("n_q_total", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
        ("n_blocks", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
        ("reserved0", ctypes.c_int32),
        ("q_stride", ctypes.c_int64 * 2), ("kv_stride", ctypes.c_int64 * 3),
        ("out_stride", ctypes.c_int64 * 2), ("bt_stride", ctypes.c_int64),
        ("scale", ctypes.c_float), ("reserved1", ctypes.c_int32),
    ]


class PlanOpts(ctypes.Structure):
    _fields_ = [
        ("num_cus", ctypes.c_int32), ("wgs_per_cu", ctypes.c_int32),
        ("min_blocks_per_split", ctypes.c_int32), ("max_blocks_per_split", ctypes.c_int32),
        ("force_blocks_per_split", ctypes.c_int32), ("combine_mode", ctypes.c_int32),
        ("schedule", ctypes.c_int32), ("segment_cost", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


_LIB = None
_TRACE_LIB = None
_P = ctypes.c_void_p
_I32P = ctypes.POINTER(ctypes.c_int32)


def _lib():
    global _LIB
    if _LIB is None:
        _LIB = _load(LIB_PATH)
    return _LIB


def trace_library():
    """The trace build (libnp_paged_trace.so: the same entry points plus
    np_debug_set_trace); raises if it has not been built."""
    global _TRACE_LIB
    if _TRACE_LIB is None:
        lib = _load(TRACE_LIB_PATH)
        lib.np_debug_set_trace.restype = ctypes.c_int
        lib.np_debug_set_trace.argtypes = [_P, ctypes.c_size_t]
        _TRACE_LIB = lib
    return _TRACE_LIB


def _load(path):
    """Load one build of the library and declare its C signatures."""
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with paged_kv_cache_178_amd.build.build() "
            "(there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    lib.np_status_string.restype = ctypes.c_char_p
    lib.np_status_string.argtypes = [ctypes.c_int]
    lib.np_next_pow2.restype = ctypes.c_int32
    lib.np_next_pow2.argtypes = [ctypes.c_int32]
    lib.np_check_paged_inputs.restype = ctypes.c_int
    lib.np_check_paged_inputs.argtypes = [ctypes.POINTER(Desc), _P, _P, _P, _P, _P, _P,
                                          _I32P, _I32P, _I32P]
    lib.np_plan.restype = ctypes.c_int
    lib.np_plan.argtypes = [ctypes.POINTER(Desc), _I32P, _I32P, ctypes.POINTER(PlanOpts),
                            ctypes.POINTER(_P)]
    lib.np_plan_destroy.restype = None
    lib.np_plan_destroy.argtypes = [_P]
    lib.np_plan_workspace_bytes.restype = ctypes.c_size_t
    lib.np_plan_workspace_bytes.argtypes = [_P]
    for name in ("np_plan_blocks_per_split", "np_plan_max_splits", "np_plan_is_prefill",
                 "np_plan_schedule"):
        getattr(lib, name).restype = ctypes.c_int32
        getattr(lib, name).argtypes = [_P]
    lib.np_plan_num_work_items.restype = ctypes.c_int64
    lib.np_plan_num_work_items.argtypes = [_P]
    lib.np_plan_work_item.restype = ctypes.c_int
    lib.np_plan_work_item.argtypes = [_P, ctypes.c_int64, _I32P]
    lib.np_plan_launch_shape.restype = ctypes.c_int
    lib.np_plan_launch_shape.argtypes = [_P, ctypes.POINTER(ctypes.c_uint32),
                                         ctypes.POINTER(ctypes.c_uint32),
                                         ctypes.POINTER(ctypes.c_uint32)]
    lib.np_paged_attention_decode.restype = ctypes.c_int
    lib.np_paged_attention_decode.argtypes = [ctypes.POINTER(Desc), _P, _P, _P, _P, _P, _P,
                                              _P, _P, ctypes.c_size_t, _P]
    lib.np_paged_attention_decode_noalloc.restype = ctypes.c_int
    lib.np_paged_attention_decode_noalloc.argtypes = [ctypes.POINTER(Desc), _P, _P, _P, _P, _P,
                                                      _P, _P, _P]
    lib.np_paged_attention_prefill.restype = ctypes.c_int
    lib.np_paged_attention_prefill.argtypes = [ctypes.POINTER(Desc), _P, _P, _P, _P, _P,
                                               _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.np_paged_kv_append.restype = ctypes.c_int
    lib.np_paged_kv_append.argtypes = [ctypes.POINTER(Desc), _P, _P, _P,
                                       ctypes.POINTER(ctypes.c_int64), _P, _P, _P, _P, _P,
                                       _P]
    lib.np_alloc_create.restype = ctypes.c_int
    lib.np_alloc_create.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_int32, _I32P, ctypes.POINTER(_P)]
    lib.np_alloc_destroy.restype = None
    lib.np_alloc_destroy.argtypes = [_P]
    lib.np_alloc_extend.restype = ctypes.c_int
    lib.np_alloc_extend.argtypes = [_P, ctypes.c_int32, ctypes.c_int32]
    lib.np_alloc_release.restype = ctypes.c_int
    lib.np_alloc_release.argtypes = [_P, ctypes.c_int32]
    lib.np_alloc_free_blocks.restype = ctypes.c_int32
    lib.np_alloc_free_blocks.argtypes = [_P]
    lib.np_alloc_block_table.restype = _I32P
    lib.np_alloc_block_table.argtypes = [_P]
    lib.np_alloc_context_lens.restype = _I32P
    lib.np_alloc_context_lens.argtypes = [_P]
    lib.np_probe_empty.restype = ctypes.c_int
    lib.np_probe_empty.argtypes = [_P]
    lib.np_probe_stream_read.restype = ctypes.c_int
    lib.np_probe_stream_read.argtypes = [_P, ctypes.c_size_t, ctypes.c_uint32, _P,
                                         ctypes.c_size_t, _P]
    lib.np_probe_stream_read_ex.restype = ctypes.c_int
    lib.np_probe_stream_read_ex.argtypes = [_P, ctypes.c_size_t, ctypes.c_uint32,
                                            ctypes.c_uint32, ctypes.c_uint32, _P,
                                            ctypes.c_size_t, _P]
    return lib


def library():
    """The loaded ctypes library (raises if it has not been built)."""
    return _lib()


# ------------------------------------------------------------- marshalling


def _dtype_code(t) -> int:
    import torch

    return {torch.float32: NP_F32, torch.float16: NP_F16, torch.bfloat16: NP_BF16}.get(t.dtype, 99)


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _i32_host(a):
    """Pointer to a host int32 buffer (torch CPU tensor or numpy array), plus
    the object that keeps it alive."""
    if a is None:
        return None, None
    import numpy as np

    if hasattr(a, "detach"):
        a = a.detach().to("cpu").numpy()
    arr = np.ascontiguousarray(a, dtype=np.int32)
    return arr.ctypes.data_as(_I32P), arr


def make_desc(q, k_pool, block_table, out=None, n_q_total=None, scale=None) -> Desc:
    """Descriptor from torch tensors: q/out [rows, Hq, d], pools [n_blocks, B,
    Hkv, d], block_table [num_seqs, max_blocks]. Strides are read from the
    tensors (in elements)."""
    d = Desc()
    d.dtype = _dtype_code(q)
    d.num_seqs = int(block_table.shape[0])
    d.n_q_total = int(q.shape[0]) if n_q_total is None else int(n_q_total)
    d.num_q_heads = int(q.shape[1])
    d.num_kv_heads = int(k_pool.shape[2])
    d.head_dim = int(q.shape[2])
    d.block_size = int(k_pool.shape[1])
    d.n_blocks = int(k_pool.shape[0])
    d.max_blocks_per_seq = int(block_table.shape[1])
    d.q_stride[0], d.q_stride[1] = int(q.stride(0)), int(q.stride(1))
    d.kv_stride[0], d.kv_stride[1], d.kv_stride[2] = (int(k_pool.stride(0)),
                                                      int(k_pool.stride(1)),
                                                      int(k_pool.stride(2)))
    o = q if out is None else out
    d.out_stride[0], d.out_stride[1] = int(o.stride(0)), int(o.stride(1))
    d.bt_stride = int(block_table.stride(0))
    d.scale = 0.0 if scale is None else float(scale)
    return d


def make_desc_contiguous(q, k_cache, out=None, n_q_total=None, scale=None,
                         block_size: int = 16) -> Desc:
    """Descriptor for dense caches k_cache/v_cache [num_seqs, capacity, Hkv, d]
    (capacity a multiple of block_size, rows of a sequence adjacent); the
    block table is then NULL: sequence s's block j is physical block
    s * (capacity / block_size) + j."""
    ns, cap, hkv, hd = (int(x) for x in k_cache.shape)
    if cap % block_size or k_cache.stride(0) != cap * k_cache.stride(1):
        raise ValueError("k_cache must be [num_seqs, capacity, Hkv, d] with capacity a "
                         "multiple of block_size and sequences stored back to back")
    d = Desc()
    d.dtype = _dtype_code(q)
    d.num_seqs = ns
    d.n_q_total = int(q.shape[0]) if n_q_total is None else int(n_q_total)
    d.num_q_heads = int(q.shape[1])
    d.num_kv_heads = hkv
    d.head_dim = int(q.shape[2])
    d.block_size = block_size
    d.max_blocks_per_seq = cap // block_size
    d.n_blocks = ns * d.max_blocks_per_seq
    d.q_stride[0], d.q_stride[1] = int(q.stride(0)), int(q.stride(1))
    s1 = int(k_cache.stride(1))
    d.kv_stride[0], d.kv_stride[1], d.kv_stride[2] = block_size * s1, s1, int(k_cache.stride(2))
    o = q if out is None else out
    d.out_stride[0], d.out_stride[1] = int(o.stride(0)), int(o.stride(1))
    d.bt_stride = d.max_blocks_per_seq
    d.scale = 0.0 if scale is None else float(scale)
    return d


class Plan:
    """Owns one np_plan_t (made, used and released by the same library)."""

    def __init__(self, handle: int, lib=None):
        self.handle = ctypes.c_void_p(handle)
        self.lib = lib if lib is not None else _lib()

    def __del__(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            self.lib.np_plan_destroy(self.handle)
            self.handle = None

    @property
    def workspace_bytes(self) -> int:
        return int(self.lib.np_plan_workspace_bytes(self.handle))

    @property
    def blocks_per_split(self) -> int:
        return int(self.lib.np_plan_blocks_per_split(self.handle))

    @property
    def max_splits(self) -> int:
        return int(self.lib.np_plan_max_splits(self.handle))

    @property
    def schedule(self) -> int:
        """1: uniform splits, 2: stream-K, 0: prefill."""
        return int(self.lib.np_plan_schedule(self.handle))

    @property
    def is_prefill(self) -> bool:
        return bool(self.lib.np_plan_is_prefill(self.handle))

    def work_items(self):
        n = int(self.lib.np_plan_num_work_items(self.handle))
        buf = (ctypes.c_int32 * 5)()
        items = []
        for i in range(n):
            st = self.lib.np_plan_work_item(self.handle, i, buf)
            if st:
                raise NPError(st, "np_plan_work_item")
            items.append(tuple(buf))
        return items

    def launch_shape(self):
        grid = (ctypes.c_uint32 * 3)()
        wg = ctypes.c_uint32()
        comb = ctypes.c_uint32()
        st = self.lib.np_plan_launch_shape(self.handle, grid, ctypes.byref(wg),
                                           ctypes.byref(comb))
        if st:
            raise NPError(st, "np_plan_launch_shape")
        return tuple(grid), int(wg.value), int(comb.value)


def next_pow2(x: int) -> int:
    return int(_lib().np_next_pow2(int(x)))


def np_check_paged_inputs(desc: Desc, q, k_pool, v_pool, block_table, context_lens, out,
                          block_table_host=None, context_lens_host=None,
                          q_start_host=None) -> int:
    """Status of the host-side validation (0 = OK). Device tensors or raw
    integer addresses are accepted for the device pointers."""
    bt_p, bt_keep = _i32_host(block_table_host)
    ln_p, ln_keep = _i32_host(context_lens_host)
    qs_p, qs_keep = _i32_host(q_start_host)

    def addr(x):
        return x if isinstance(x, int) or x is None else _ptr(x)

    st = _lib().np_check_paged_inputs(ctypes.byref(desc), addr(q), addr(k_pool), addr(v_pool),
                                      addr(block_table), addr(context_lens), addr(out),
                                      bt_p, ln_p, qs_p)
    del bt_keep, ln_keep, qs_keep
    return int(st)


def np_plan(desc: Desc, context_lens_host, q_start_host=None, opts: PlanOpts | None = None,
            lib=None) -> Plan:
    """`lib`: the library to plan with (default the product library; pass
    trace_library() for a plan launched through the trace build)."""
    lib = lib if lib is not None else _lib()
    ln_p, ln_keep = _i32_host(context_lens_host)
    qs_p, qs_keep = _i32_host(q_start_host)
    h = ctypes.c_void_p()
    st = lib.np_plan(ctypes.byref(desc), ln_p, qs_p,
                     ctypes.byref(opts) if opts is not None else None, ctypes.byref(h))
    del ln_keep, qs_keep
    if st:
        raise NPError(st, "np_plan")
    return Plan(h.value, lib)


def _stream(stream):
    if stream is not None:
        return int(stream)
    import torch

    return int(torch.cuda.current_stream().cuda_stream)


def np_paged_attention_decode(desc: Desc, plan: Plan, q, k_pool, v_pool, block_table,
                              context_lens, out, workspace=None, stream=None) -> None:
    """Launch through the library that made `plan`."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = plan.lib.np_paged_attention_decode(ctypes.byref(desc), plan.handle, _ptr(q),
                                          _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
                                          _ptr(context_lens), _ptr(out), _ptr(workspace),
                                          ws_bytes, _stream(stream))
    if st:
        raise NPError(st, "np_paged_attention_decode")


def np_paged_attention_decode_noalloc(desc: Desc, plan: Plan, q, k_pool, v_pool, block_table,
                                      context_lens, out, stream=None) -> None:
    """The allocation-free decode: the library's per-device scratch array is
    the workspace."""
    st = plan.lib.np_paged_attention_decode_noalloc(ctypes.byref(desc), plan.handle, _ptr(q),
                                                    _ptr(k_pool), _ptr(v_pool),
                                                    _ptr(block_table), _ptr(context_lens),
                                                    _ptr(out), _stream(stream))
    if st:
        raise NPError(st, "np_paged_attention_decode_noalloc")


def np_paged_attention_prefill(desc: Desc, plan: Plan, q, k_pool, v_pool, block_table,
                               context_lens, q_start, out, workspace=None,
                               stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _lib().np_paged_attention_prefill(ctypes.byref(desc), plan.handle, _ptr(q),
                                           _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
                                           _ptr(context_lens), _ptr(q_start), _ptr(out),
                                           _ptr(workspace), ws_bytes, _stream(stream))
    if st:
        raise NPError(st, "np_paged_attention_prefill")


# --------------------------------------------------------- convenience layer


def np_paged_kv_append(desc: Desc, plan: Plan, k_new, v_new, block_table, context_lens,
                       new_start, k_pool, v_pool, new_stride=None, stream=None) -> None:
    """Scatter rows of k_new / v_new ([rows, Hkv, d], device) into the pools.
    `plan` is np_plan(desc, lens_host, new_start_host); new_stride defaults to
    k_new's (row, head) element strides."""
    if new_stride is None:
        new_stride = (k_new.stride(0), k_new.stride(1))
        if (v_new.stride(0), v_new.stride(1)) != tuple(new_stride):
            raise ValueError("k_new and v_new must share their (row, head) strides")
    st_arr = (ctypes.c_int64 * 2)(*new_stride)
    st = _lib().np_paged_kv_append(ctypes.byref(desc), plan.handle, _ptr(k_new), _ptr(v_new),
                                   st_arr, _ptr(block_table), _ptr(context_lens),
                                   _ptr(new_start), _ptr(k_pool), _ptr(v_pool), _stream(stream))
    if st:
        raise NPError(st, "np_paged_kv_append")


class BlockAllocator:
    """Host block allocator (np_alloc_*): tables and lengths come back as
    numpy copies."""

    def __init__(self, n_blocks: int, block_size: int, num_seqs: int, max_blocks_per_seq: int,
                 free_order=None):
        import numpy as np

        self.num_seqs, self.max_blocks = num_seqs, max_blocks_per_seq
        fo_p, self._fo = _i32_host(free_order)
        h = _P()
        st = _lib().np_alloc_create(n_blocks, block_size, num_seqs, max_blocks_per_seq, fo_p,
                                    ctypes.byref(h))
        if st:
            raise NPError(st, "np_alloc_create")
        self.handle = h
        self._np = np

    def __del__(self):
        if getattr(self, "handle", None) and _LIB is not None:
            _LIB.np_alloc_destroy(self.handle)
            self.handle = None

    def extend(self, seq: int, new_len: int) -> None:
        st = _lib().np_alloc_extend(self.handle, seq, new_len)
        if st:
            raise NPError(st, "np_alloc_extend")

    def release(self, seq: int) -> None:
        st = _lib().np_alloc_release(self.handle, seq)
        if st:
            raise NPError(st, "np_alloc_release")

    def free_blocks(self) -> int:
        return int(_lib().np_alloc_free_blocks(self.handle))

    def block_table(self):
        p = _lib().np_alloc_block_table(self.handle)
        n = self.num_seqs * self.max_blocks
        return self._np.ctypeslib.as_array(p, shape=(n,)).reshape(self.num_seqs,
                                                                  self.max_blocks).copy()

    def context_lens(self):
        p = _lib().np_alloc_context_lens(self.handle)
        return self._np.ctypeslib.as_array(p, shape=(self.num_seqs,)).copy()


def workspace_for(plan: Plan, device):
    """A zeroed device byte buffer of the plan's workspace size (256-byte
    aligned by the caching allocator), or None when the plan needs none. The
    library leaves its arrival counters zero after every call, so the buffer
    can be reused by later calls on the same stream."""
    import torch

    n = plan.workspace_bytes
    return None if n == 0 else torch.zeros(n, dtype=torch.uint8, device=device)


def decode(q, k_pool, v_pool, block_table, context_lens, out=None, scale=None,
           context_lens_host=None, opts: PlanOpts | None = None, check_tables=False):
    """One decode call on device tensors: check, plan, launch. Returns out."""
    import torch

    if out is None:
        out = torch.empty_like(q)
    desc = make_desc(q, k_pool, block_table, out=out, scale=scale)
    lens_h = context_lens.cpu() if context_lens_host is None else context_lens_host
    st = np_check_paged_inputs(desc, q, k_pool, v_pool, block_table, context_lens, out,
                               block_table.cpu() if check_tables else None, lens_h, None)
    if st:
        raise NPError(st, "np_check_paged_inputs")
    plan = np_plan(desc, lens_h, None, opts)
    ws = workspace_for(plan, q.device)
    np_paged_attention_decode(desc, plan, q, k_pool, v_pool, block_table, context_lens, out, ws)
    return out


def prefill(q, k_pool, v_pool, block_table, context_lens, q_start, out=None, scale=None,
            context_lens_host=None, q_start_host=None, check_tables=False):
    """One chunked-prefill call on device tensors: check, plan, launch."""
    import torch

    if out is None:
        out = torch.empty_like(q)
    desc = make_desc(q, k_pool, block_table, out=out, scale=scale)
    lens_h = context_lens.cpu() if context_lens_host is None else context_lens_host
    qs_h = q_start.cpu() if q_start_host is None else q_start_host
    st = np_check_paged_inputs(desc, q, k_pool, v_pool, block_table, context_lens, out,
                               block_table.cpu() if check_tables else None, lens_h, qs_h)
    if st:
        raise NPError(st, "np_check_paged_inputs")
    plan = np_plan(desc, lens_h, qs_h)
    ws = workspace_for(plan, q.device)
    np_paged_attention_prefill(desc, plan, q, k_pool, v_pool, block_table, context_lens,
                               q_start, out, ws)
    return out


def np_probe_empty(stream=None) -> None:
    st = _lib().np_probe_empty(_stream(stream))
    if st:
        raise NPError(st, "np_probe_empty")


def np_probe_stream_read(src, num_wgs: int, sink, stream=None) -> None:
    st = _lib().np_probe_stream_read(_ptr(src), src.numel() * src.element_size(), int(num_wgs),
                                     _ptr(sink), sink.numel() * sink.element_size(),
                                     _stream(stream))
    if st:
        raise NPError(st, "np_probe_stream_read")


def np_probe_stream_read_ex(src, num_wgs: int, wg_size: int, loads_per_thread: int, sink,
                            stream=None) -> None:
    st = _lib().np_probe_stream_read_ex(_ptr(src), src.numel() * src.element_size(),
                                        int(num_wgs), int(wg_size), int(loads_per_thread),
                                        _ptr(sink), sink.numel() * sink.element_size(),
                                        _stream(stream))
    if st:
        raise NPError(st, "np_probe_stream_read_ex")


def set_trace(buf) -> None:
    """Register a device int32 buffer with the trace build (None: off)."""
    lib = trace_library()
    st = lib.np_debug_set_trace(None if buf is None else _ptr(buf),
                                0 if buf is None else buf.numel() * buf.element_size())
    if st:
        raise NPError(st, "np_debug_set_trace")
