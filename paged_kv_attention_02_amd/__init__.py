"""Paged KV attention for one batch on AMD Instinct MI355X (gfx950).

Thin ctypes binding over ``libpka.so`` (C ABI declared in ``include/pka.h``).
This module only marshals arguments: every step of the attention path --
metadata, cache write, decode, extend -- runs in the library's HIP kernels.
PyTorch provides device memory and the current HIP stream.  If the library is
not built, importing the binding's entry points raises: there is no fallback.

Typical use::

    import paged_kv_attention_02_amd as pka
    ctx = pka.Context(num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
                      num_pages=pool_pages, q_dtype="bf16", kv_dtype="bf16",
                      scale=128 ** -0.5)
    md = pka.Batch(ctx, "decode", batch=B, num_q_tokens=B, max_kv_pages=pages)
    md.init(seq_lens, None, page_table)          # device int32 tensors
    pka.save_kv(ctx, md, k_new, v_new, k_pool, v_pool)
    pka.attn_decode(ctx, md, q, k_pool, v_pool, out, workspace=md.workspace)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpka.so")

MODES = {"extend": 0, "decode": 1, "idle": 2, "target_verify": 3, "draft_extend": 4}
SPEC_MODES = {"prefill": 0, "decode": 1}
DTYPES = {"f32": 0, "bf16": 1, "fp8": 2}
PATHS = {0: "none", 1: "decode", 2: "extend"}
STATUS = {0: "PKA_OK", -1: "PKA_ERR_INVALID_ARG", -2: "PKA_ERR_UNSUPPORTED",
          -3: "PKA_ERR_WORKSPACE", -4: "PKA_ERR_HIP"}
DEV_FLAGS = {1: "BAD_LENGTH", 2: "BAD_PAGE", 4: "TABLE_SHORT", 8: "CAPACITY"}
# The scratch array of pka_forward_with_metadata_noalloc (PKA_NOALLOC_SCRATCH_BYTES in pka.h).
NOALLOC_SCRATCH_BYTES = 64 << 20


class PkaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("q_dtype", ctypes.c_int),
                ("kv_dtype", ctypes.c_int), ("scale", ctypes.c_float),
                ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
                ("v_head_dim", ctypes.c_int32), ("max_q_per_request", ctypes.c_int32)]


class BatchStruct(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int), ("batch", ctypes.c_int32),
                ("num_q_tokens", ctypes.c_int32), ("max_kv_pages", ctypes.c_int64),
                ("kv_indptr", ctypes.c_void_p), ("kv_indices", ctypes.c_void_p),
                ("kv_last_page_len", ctypes.c_void_p), ("qo_indptr", ctypes.c_void_p),
                ("out_cache_loc", ctypes.c_void_p), ("plan", ctypes.c_void_p)]


class Sizes(ctypes.Structure):
    _fields_ = [("kv_indptr", ctypes.c_int64), ("kv_indices", ctypes.c_int64),
                ("kv_last_page_len", ctypes.c_int64), ("qo_indptr", ctypes.c_int64),
                ("out_cache_loc", ctypes.c_int64), ("plan", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_int64)]


# Every symbol the header declares, with its ctypes signature.
_VP, _I32, _I64, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
SIGNATURES = {
    "pka_create": (ctypes.c_int, [ctypes.POINTER(Config), ctypes.POINTER(_VP)]),
    "pka_destroy": (None, [_VP]),
    "pka_batch_sizes": (ctypes.c_int, [_VP, ctypes.c_int, _I32, _I32, _I64, ctypes.POINTER(Sizes)]),
    "pka_init_metadata": (ctypes.c_int, [_VP, _VP, _VP, _VP, _I32, _I32,
                                         ctypes.POINTER(BatchStruct), _VP]),
    "pka_save_kv": (ctypes.c_int, [_VP, ctypes.POINTER(BatchStruct), _VP, _VP, _VP, _VP, _VP]),
    "pka_attn_decode": (ctypes.c_int, [_VP, ctypes.POINTER(BatchStruct), _VP, _VP, _VP, _VP, _VP,
                                       _VP, _SZ, _VP]),
    "pka_attn_extend": (ctypes.c_int, [_VP, ctypes.POINTER(BatchStruct), _VP, _VP, _VP, _VP, _VP,
                                       _VP, _SZ, _VP]),
    "pka_select_path": (ctypes.c_int, [ctypes.c_int, ctypes.c_int]),
    "pka_forward": (ctypes.c_int, [_VP, ctypes.c_int, ctypes.c_int, ctypes.POINTER(BatchStruct),
                                   _VP, _VP, _VP, ctypes.c_int, _VP, _VP, _VP, _VP, _VP, _SZ, _VP]),
    "pka_forward_with_metadata": (ctypes.c_int, [_VP, ctypes.c_int, ctypes.c_int, _VP, _VP, _VP, _I32,
                                                 _I32, ctypes.POINTER(BatchStruct), _VP, _VP, _VP,
                                                 ctypes.c_int, _VP, _VP, _VP, _VP, _VP, _SZ, _VP]),
    "pka_forward_with_metadata_noalloc": (ctypes.c_int, [_VP, ctypes.c_int, ctypes.c_int, _VP, _VP, _VP,
                                                         _I32, _I32, ctypes.POINTER(BatchStruct), _VP, _VP,
                                                         _VP, ctypes.c_int, _VP, _VP, _VP, _VP, _VP]),
    "pka_read_status": (ctypes.c_int, [ctypes.POINTER(BatchStruct), ctypes.POINTER(_I32), _VP]),
    "pka_describe": (ctypes.c_int, [_VP, ctypes.c_int, ctypes.c_int, _I32, _I32, ctypes.c_int,
                                    ctypes.c_char_p, _SZ]),
    "pka_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "pka_last_error": (ctypes.c_char_p, []),
    "pka_version": (ctypes.c_char_p, []),
}

_lib = None


def lib():
    """Load libpka.so (built in-tree); raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m paged_kv_attention_02_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise PkaError(status, lib().pka_last_error().decode())


def version() -> str:
    return lib().pka_version().decode()


def select_path(mode: str, spec_mode: str = "prefill") -> str:
    """ForwardMode -> path ("decode", "extend" or "none")."""
    return PATHS[lib().pka_select_path(MODES[mode], SPEC_MODES[spec_mode])]


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


class Context:
    """Per-layer attention parameters (host-only handle, no device memory)."""

    def __init__(self, num_q_heads: int, num_kv_heads: int, head_dim: int, page_size: int,
                 num_pages: int, q_dtype: str = "bf16", kv_dtype: str = "bf16",
                 scale: Optional[float] = None, k_scale: float = 1.0, v_scale: float = 1.0,
                 v_head_dim: Optional[int] = None, max_q_per_request: int = 0):
        """head_dim: query/key head width; v_head_dim: value/output head
        width (None: the same as head_dim); max_q_per_request: the most query
        tokens a request carries in a verify batch on the decode path (0: 16)."""
        dv = head_dim if v_head_dim is None else v_head_dim
        self.cfg = Config(num_q_heads, num_kv_heads, head_dim, page_size, num_pages,
                          DTYPES[q_dtype], DTYPES[kv_dtype],
                          head_dim ** -0.5 if scale is None else scale, k_scale, v_scale, dv,
                          max_q_per_request)
        self.q_dtype, self.kv_dtype = q_dtype, kv_dtype
        self.num_q_heads, self.num_kv_heads, self.head_dim = num_q_heads, num_kv_heads, head_dim
        self.v_head_dim = dv
        self.page_size, self.num_pages = page_size, num_pages
        h = ctypes.c_void_p()
        _check(lib().pka_create(ctypes.byref(self.cfg), ctypes.byref(h)))
        self.handle = h

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value and _lib is not None:
            _lib.pka_destroy(h)
            self.handle = None

    def sizes(self, mode: str, batch: int, num_q_tokens: int, max_kv_pages: int) -> Sizes:
        s = Sizes()
        _check(lib().pka_batch_sizes(self.handle, MODES[mode], batch, num_q_tokens, max_kv_pages,
                                     ctypes.byref(s)))
        return s

    def describe(self, mode: str, batch: int, num_q_tokens: int, spec_mode: str = "prefill",
                 with_metadata: bool = False) -> str:
        """The kernels and launch shape a batch of this shape resolves to."""
        buf = ctypes.create_string_buffer(1024)
        _check(lib().pka_describe(self.handle, MODES[mode], SPEC_MODES[spec_mode], batch,
                                  num_q_tokens, int(bool(with_metadata)), buf, len(buf)))
        return buf.value.decode()

    def pool_shape(self):
        """Shape of the K pool."""
        return (self.num_pages * self.page_size, self.num_kv_heads, self.head_dim)

    def v_pool_shape(self):
        return (self.num_pages * self.page_size, self.num_kv_heads, self.v_head_dim)


class Batch:
    """Device metadata arrays of one batch (allocated with torch)."""

    def __init__(self, ctx: Context, mode: str, batch: int, num_q_tokens: int, max_kv_pages: int,
                 device="cuda"):
        import torch
        self.ctx, self.mode = ctx, mode
        sz = ctx.sizes(mode, batch, num_q_tokens, max_kv_pages)
        i32 = dict(dtype=torch.int32, device=device)
        self.kv_indptr = torch.zeros(sz.kv_indptr, **i32)
        self.kv_indices = torch.zeros(sz.kv_indices, **i32)
        self.kv_last_page_len = torch.zeros(sz.kv_last_page_len, **i32)
        self.qo_indptr = torch.zeros(sz.qo_indptr, **i32)
        self.out_cache_loc = torch.zeros(sz.out_cache_loc, **i32)
        self.plan = torch.zeros(sz.plan, **i32)
        self.workspace = (torch.empty(max(sz.workspace_bytes, 16), dtype=torch.uint8, device=device)
                          if sz.workspace_bytes > 0 else None)
        self.s = BatchStruct(MODES[mode], batch, num_q_tokens, max_kv_pages,
                             self.kv_indptr.data_ptr(), self.kv_indices.data_ptr(),
                             self.kv_last_page_len.data_ptr(), self.qo_indptr.data_ptr(),
                             self.out_cache_loc.data_ptr(), self.plan.data_ptr())

    @property
    def batch(self) -> int:
        return self.s.batch

    @property
    def num_q_tokens(self) -> int:
        return self.s.num_q_tokens

    def _check_inputs(self, seq_lens, extend_lens, page_table):
        import torch
        for name, t in (("seq_lens", seq_lens), ("extend_lens", extend_lens),
                        ("page_table", page_table)):
            if t is not None and (t.dtype != torch.int32 or not t.is_cuda):
                raise ValueError(f"{name} must be a device int32 tensor")
        if page_table.dim() != 2 or page_table.stride(1) != 1:
            raise ValueError("page_table must be [B, cols] with unit column stride")
        if seq_lens.numel() != self.batch or page_table.shape[0] != self.batch:
            raise ValueError("seq_lens / page_table rows must match the batch size")
        self._keep = (seq_lens, extend_lens, page_table)

    def init(self, seq_lens, extend_lens, page_table, stream=None):
        """Build the index buffers from device int32 seq_lens [B], extend_lens
        [B] (None for decode) and page_table [B, cols] (row stride >= cols)."""
        self._check_inputs(seq_lens, extend_lens, page_table)
        _check(lib().pka_init_metadata(self.ctx.handle, seq_lens.data_ptr(), _ptr(extend_lens),
                                       page_table.data_ptr(), page_table.stride(0),
                                       page_table.shape[1], ctypes.byref(self.s), _stream(stream)))

    def status(self, stream=None) -> int:
        """Synchronise and read the device status flags (0 = clean)."""
        v = ctypes.c_int32()
        _check(lib().pka_read_status(ctypes.byref(self.s), ctypes.byref(v), _stream(stream)))
        return v.value


def _check_rows(ctx: Context, t, rows: int, heads: int, dtype: str, name: str, value: bool = False):
    """value: the tensor has value-width rows (v_new, v_pool, out)."""
    import torch
    want = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}[dtype]
    if t.dtype != want or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous device {want} tensor, got {t.dtype}")
    width = ctx.v_head_dim if value else ctx.head_dim
    if tuple(t.shape) != (rows, heads, width):
        raise ValueError(f"{name}: expected shape {(rows, heads, width)}, got {tuple(t.shape)}")


def _check_pools(ctx: Context, k_pool, v_pool):
    slots = ctx.num_pages * ctx.page_size
    _check_rows(ctx, k_pool, slots, ctx.num_kv_heads, ctx.kv_dtype, "k_pool")
    _check_rows(ctx, v_pool, slots, ctx.num_kv_heads, ctx.kv_dtype, "v_pool", value=True)


def save_kv(ctx: Context, md: Batch, k_new, v_new, k_pool, v_pool, stream=None):
    _check_rows(ctx, k_new, md.num_q_tokens, ctx.num_kv_heads, ctx.q_dtype, "k_new")
    _check_rows(ctx, v_new, md.num_q_tokens, ctx.num_kv_heads, ctx.q_dtype, "v_new", value=True)
    _check_pools(ctx, k_pool, v_pool)
    _check(lib().pka_save_kv(ctx.handle, ctypes.byref(md.s), k_new.data_ptr(), v_new.data_ptr(),
                             k_pool.data_ptr(), v_pool.data_ptr(), _stream(stream)))


def _attn_common(ctx, md, q, k_pool, v_pool, out, lse):
    import torch
    _check_rows(ctx, q, md.num_q_tokens, ctx.num_q_heads, ctx.q_dtype, "q")
    _check_rows(ctx, out, md.num_q_tokens, ctx.num_q_heads, ctx.q_dtype, "out", value=True)
    _check_pools(ctx, k_pool, v_pool)
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or tuple(lse.shape) != (md.num_q_tokens, ctx.num_q_heads)):
        raise ValueError("lse must be a contiguous fp32 [num_q_tokens, num_q_heads] tensor")


def _ws(workspace):
    return (None, 0) if workspace is None else (workspace.data_ptr(), workspace.numel() * workspace.element_size())


def attn_decode(ctx: Context, md: Batch, q, k_pool, v_pool, out, lse=None, workspace=None,
                stream=None):
    _attn_common(ctx, md, q, k_pool, v_pool, out, lse)
    wp, wb = _ws(md.workspace if workspace is None else workspace)
    _check(lib().pka_attn_decode(ctx.handle, ctypes.byref(md.s), q.data_ptr(), k_pool.data_ptr(),
                                 v_pool.data_ptr(), out.data_ptr(), _ptr(lse), wp, wb,
                                 _stream(stream)))


def attn_extend(ctx: Context, md: Batch, q, k_pool, v_pool, out, lse=None, workspace=None,
                stream=None):
    _attn_common(ctx, md, q, k_pool, v_pool, out, lse)
    wp, wb = _ws(md.workspace if workspace is None else workspace)
    _check(lib().pka_attn_extend(ctx.handle, ctypes.byref(md.s), q.data_ptr(), k_pool.data_ptr(),
                                 v_pool.data_ptr(), out.data_ptr(), _ptr(lse), wp, wb,
                                 _stream(stream)))


def forward(ctx: Context, mode: str, md: Batch, q, k_new, v_new, k_pool, v_pool, out, lse=None,
            save_kv_cache: bool = True, spec_mode: str = "prefill", workspace=None, stream=None):
    """One layer: optional cache write, then the path pka_select_path picks."""
    if mode != "idle":
        _attn_common(ctx, md, q, k_pool, v_pool, out, lse)
        if save_kv_cache:
            _check_rows(ctx, k_new, md.num_q_tokens, ctx.num_kv_heads, ctx.q_dtype, "k_new")
            _check_rows(ctx, v_new, md.num_q_tokens, ctx.num_kv_heads, ctx.q_dtype, "v_new", value=True)
    wp, wb = _ws(md.workspace if workspace is None else workspace)
    _check(lib().pka_forward(ctx.handle, MODES[mode], SPEC_MODES[spec_mode], ctypes.byref(md.s),
                             _ptr(q), _ptr(k_new), _ptr(v_new), int(bool(save_kv_cache)),
                             _ptr(k_pool), _ptr(v_pool), _ptr(out), _ptr(lse), wp, wb,
                             _stream(stream)))


def forward_with_metadata(ctx: Context, mode: str, md: Batch, seq_lens, extend_lens, page_table, q,
                          k_new, v_new, k_pool, v_pool, out, lse=None, save_kv_cache: bool = True,
                          spec_mode: str = "prefill", workspace=None, stream=None):
    """md.init(seq_lens, extend_lens, page_table) followed by forward(...), as
    one library call (one decode launch builds both for bf16 / fp8 decode
    batches)."""
    if mode != "idle":
        md._check_inputs(seq_lens, extend_lens, page_table)
        _attn_common(ctx, md, q, k_pool, v_pool, out, lse)
        if save_kv_cache:
            _check_rows(ctx, k_new, md.num_q_tokens, ctx.num_kv_heads, ctx.q_dtype, "k_new")
            _check_rows(ctx, v_new, md.num_q_tokens, ctx.num_kv_heads, ctx.q_dtype, "v_new", value=True)
    wp, wb = _ws(md.workspace if workspace is None else workspace)
    _check(lib().pka_forward_with_metadata(
        ctx.handle, MODES[mode], SPEC_MODES[spec_mode], _ptr(seq_lens), _ptr(extend_lens),
        _ptr(page_table), 0 if page_table is None else page_table.stride(0),
        0 if page_table is None else page_table.shape[1], ctypes.byref(md.s), _ptr(q), _ptr(k_new),
        _ptr(v_new), int(bool(save_kv_cache)), _ptr(k_pool), _ptr(v_pool), _ptr(out), _ptr(lse), wp,
        wb, _stream(stream)))


def forward_with_metadata_noalloc(ctx: Context, mode: str, md: Batch, seq_lens, extend_lens, page_table,
                                  q, k_new, v_new, k_pool, v_pool, out, lse=None,
                                  save_kv_cache: bool = True, spec_mode: str = "prefill", stream=None):
    """forward_with_metadata without a workspace: the decode partials live in
    the library's per-device scratch array (NOALLOC_SCRATCH_BYTES); nothing
    is allocated by the call."""
    if mode != "idle":
        md._check_inputs(seq_lens, extend_lens, page_table)
        _attn_common(ctx, md, q, k_pool, v_pool, out, lse)
        if save_kv_cache:
            _check_rows(ctx, k_new, md.num_q_tokens, ctx.num_kv_heads, ctx.q_dtype, "k_new")
            _check_rows(ctx, v_new, md.num_q_tokens, ctx.num_kv_heads, ctx.q_dtype, "v_new", value=True)
    _check(lib().pka_forward_with_metadata_noalloc(
        ctx.handle, MODES[mode], SPEC_MODES[spec_mode], _ptr(seq_lens), _ptr(extend_lens),
        _ptr(page_table), 0 if page_table is None else page_table.stride(0),
        0 if page_table is None else page_table.shape[1], ctypes.byref(md.s), _ptr(q), _ptr(k_new),
        _ptr(v_new), int(bool(save_kv_cache)), _ptr(k_pool), _ptr(v_pool), _ptr(out), _ptr(lse),
        _stream(stream)))
