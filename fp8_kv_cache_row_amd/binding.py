"""Thin ctypes binding of libfp8kv.so.

The calls keep the C names (fp8kv_quantize_rows, fp8kv_decode_attn,
fp8kv_decode_attn_rows, fp8kv_decode_attn_append, fp8kv_prefill_attn, ...).  This module only marshals arguments: it takes torch
device tensors, checks dtypes/shapes that the C ABI cannot see, passes raw
pointers and the current stream, and raises on a non-OK status.  Every step of
the computation runs in the library's HIP kernels; there is no fallback.

`Fp8KvPool` allocates one layer of the page-size-1 FP8 row pool with torch
(device memory plumbing) and exposes it as the C `fp8kv_pool_layer` struct.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

HEAD_DIM = 128           # prefill, and the default pool head dim
HEAD_DIMS = (128, 256)   # pool / quantize / decode head dims
CODE_FORMATS = {"e4m3": 0, "int8": 1}
MAX_QUERY_ROWS = 8
_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfp8kv.so")
_HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "fp8kv.h")

_lib: Optional[ctypes.CDLL] = None


class Fp8KvError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call} failed: {status_string(status)} (status {status})")


class PoolLayer(ctypes.Structure):
    """Mirror of `fp8kv_pool_layer` in include/fp8kv.h."""
    _fields_ = [
        ("k_codes", ctypes.c_void_p),
        ("v_codes", ctypes.c_void_p),
        ("k_scales", ctypes.c_void_p),
        ("v_scales", ctypes.c_void_p),
        ("num_rows", ctypes.c_int64),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("code_row_stride", ctypes.c_int64),
        ("scale_row_stride", ctypes.c_int64),
        ("code_format", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


def lib_path() -> str:
    return _LIB_PATH


def header_path() -> str:
    return _HEADER


def load() -> ctypes.CDLL:
    """Load libfp8kv.so; fails loudly if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
    L = ctypes.CDLL(_LIB_PATH)
    P = ctypes.POINTER(PoolLayer)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    L.fp8kv_quantize_rows.argtypes = [P, vp, vp, i64, vp, i32, vp]
    L.fp8kv_quantize_rows.restype = ctypes.c_int
    L.fp8kv_decode_workspace_bytes.argtypes = [i32, i32, i32, i32]
    L.fp8kv_decode_workspace_bytes.restype = sz
    L.fp8kv_decode_attn.argtypes = [P, vp, i32, i32, vp, i64, vp, i32, f32, i32, vp, sz, vp, vp]
    L.fp8kv_decode_attn.restype = ctypes.c_int
    L.fp8kv_decode_attn_rows.argtypes = [P, vp, i32, i32, i32, vp, i64, vp, i32, i32, f32, i32, vp, sz, vp, vp]
    L.fp8kv_decode_attn_rows.restype = ctypes.c_int
    L.fp8kv_decode_attn_append.argtypes = [P, vp, i32, i32, vp, vp, i64, vp, vp, i64, vp, i32, f32, i32, vp, sz,
                                           vp, vp]
    L.fp8kv_decode_attn_append.restype = ctypes.c_int
    L.fp8kv_decode_attn_append_noalloc.argtypes = [P, vp, i32, i32, vp, vp, i64, vp, vp, i64, vp, i32, f32, i32,
                                                   vp, vp]
    L.fp8kv_decode_attn_append_noalloc.restype = ctypes.c_int
    L.fp8kv_decode_attn_append_window.argtypes = [P, vp, i32, i32, vp, vp, i64, vp, vp, i64, vp, i32, i32, f32, i32,
                                                  vp, sz, vp, vp]
    L.fp8kv_decode_attn_append_window.restype = ctypes.c_int
    L.fp8kv_decode_attn_rows_append.argtypes = [P, vp, i32, i32, i32, vp, vp, i64, vp, vp, i64, vp, i32, i32, f32,
                                                i32, vp, sz, vp, vp]
    L.fp8kv_decode_attn_rows_append.restype = ctypes.c_int
    L.fp8kv_decode_stage1.argtypes = [P, vp, i32, i32, vp, i64, vp, i32, f32, i32, vp, sz, vp]
    L.fp8kv_decode_stage1.restype = ctypes.c_int
    L.fp8kv_decode_stage1_valu.argtypes = [P, vp, i32, i32, vp, i64, vp, i32, f32, i32, vp, sz, vp]
    L.fp8kv_decode_stage1_valu.restype = ctypes.c_int
    L.fp8kv_decode_merge.argtypes = [i32, i32, i32, i32, vp, sz, vp, vp]
    L.fp8kv_decode_merge.restype = ctypes.c_int
    L.fp8kv_prefill_attn.argtypes = [P, vp, vp, vp, i32, i32, vp, i32, vp, vp, i64, f32, vp, vp]
    L.fp8kv_prefill_attn.restype = ctypes.c_int
    L.fp8kv_prefill_attn_workspace.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp, i32, f32, vp, vp]
    L.fp8kv_prefill_attn_workspace.restype = ctypes.c_int
    L.fp8kv_status_string.argtypes = [ctypes.c_int]
    L.fp8kv_status_string.restype = ctypes.c_char_p
    _lib = L
    return L


def declared_symbols() -> list:
    """Function names declared in include/fp8kv.h."""
    text = open(_HEADER).read()
    decl = r"^(?:fp8kv_status|size_t|const char \*)\s*(fp8kv_\w+)\s*\("
    return sorted(set(re.findall(decl, text, flags=re.M)))


def status_string(status: int) -> str:
    return load().fp8kv_status_string(int(status)).decode()


def _check(status: int, call: str) -> None:
    if status != 0:
        raise Fp8KvError(status, call)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dev_check(t: torch.Tensor, name: str, dtype: torch.dtype) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _bits(t: torch.Tensor) -> torch.Tensor:
    """bf16 tensors are passed to the ABI as their 16-bit patterns."""
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


# ------------------------------------------------------------------- pool --

class Fp8KvPool:
    """One layer of the page-size-1 FP8 row pool, allocated on the current device.

    layout="separate": k_codes/v_codes uint8 [R][Hkv][D], k_scales/v_scales
      float32 [R][Hkv] (four allocations); D = head_dim, 128 or 256.
    layout="interleaved": one record per row holding K codes, V codes, K scales,
      V scales back to back (rounded up to 16 bytes), so every byte of a row is
      in one contiguous span.
    layout="interleaved64" / "interleaved128": the same record padded to a
      multiple of 64 / 128 bytes, so every record starts on a 64- / 128-byte
      boundary (memory-sector alignment; the padding is never read).
    layout="split": two allocations, one record per row holding the K and V
      codes of all KV heads (2 * Hkv * D bytes) and one holding its K and V
      scales (2 * Hkv floats).
    code_format: "e4m3" (OCP E4M3FN, scale amax/448) or "int8" (symmetric, scale amax/127).
    """

    LAYOUTS = ("separate", "interleaved", "interleaved64", "interleaved128", "split")

    def __init__(self, num_rows: int, n_kv_heads: int, layout: str = "separate",
                 device: Optional[torch.device] = None, head_dim: int = HEAD_DIM, code_format: str = "e4m3"):
        dev = device or torch.device("cuda", torch.cuda.current_device())
        self.num_rows, self.n_kv_heads, self.layout = int(num_rows), int(n_kv_heads), layout
        self.head_dim = int(head_dim)
        if code_format not in CODE_FORMATS:
            raise ValueError(f"unknown code format {code_format!r}")
        self.code_format = code_format
        H, D = self.n_kv_heads, self.head_dim
        if layout == "separate":
            self.k_codes = torch.zeros((num_rows, H, D), dtype=torch.uint8, device=dev)
            self.v_codes = torch.zeros((num_rows, H, D), dtype=torch.uint8, device=dev)
            self.k_scales = torch.zeros((num_rows, H), dtype=torch.float32, device=dev)
            self.v_scales = torch.zeros((num_rows, H), dtype=torch.float32, device=dev)
            code_stride, scale_stride = H * D, H
            ptrs = [t.data_ptr() for t in (self.k_codes, self.v_codes, self.k_scales, self.v_scales)]
            self._buffers = [self.k_codes, self.v_codes, self.k_scales, self.v_scales]
        elif layout.startswith("interleaved"):
            align = {"interleaved": 16, "interleaved64": 64, "interleaved128": 128}.get(layout)
            if align is None:
                raise ValueError(f"unknown pool layout {layout!r}")
            rec = -(-(2 * H * D + 2 * H * 4) // align) * align
            self.record = torch.zeros((num_rows, rec), dtype=torch.uint8, device=dev)
            self.k_codes = self.record[:, :H * D].view(num_rows, H, D)
            self.v_codes = self.record[:, H * D:2 * H * D].view(num_rows, H, D)
            base = self.record.data_ptr()
            self.k_scales = None  # views of the record; read back with scales()
            self.v_scales = None
            code_stride, scale_stride = rec, rec // 4
            ptrs = [base, base + H * D, base + 2 * H * D, base + 2 * H * D + 4 * H]
            self._buffers = [self.record]
        elif layout == "split":
            self.codes_record = torch.zeros((num_rows, 2 * H * D), dtype=torch.uint8, device=dev)
            self.scales_record = torch.zeros((num_rows, 2 * H), dtype=torch.float32, device=dev)
            self.k_codes = self.codes_record[:, :H * D].view(num_rows, H, D)
            self.v_codes = self.codes_record[:, H * D:].view(num_rows, H, D)
            self.k_scales = None  # views of the scale record; read back with scales()
            self.v_scales = None
            cb, sb = self.codes_record.data_ptr(), self.scales_record.data_ptr()
            code_stride, scale_stride = 2 * H * D, 2 * H
            ptrs = [cb, cb + H * D, sb, sb + 4 * H]
            self._buffers = [self.codes_record, self.scales_record]
        else:
            raise ValueError(f"unknown pool layout {layout!r}")
        self.layer = PoolLayer(ptrs[0], ptrs[1], ptrs[2], ptrs[3], self.num_rows, H, D,
                               code_stride, scale_stride, CODE_FORMATS[code_format], 0)

    def scales(self):
        """(k_scales, v_scales) as float32 [R][Hkv] tensors (copies for the interleaved layout)."""
        if self.layout == "separate":
            return self.k_scales, self.v_scales
        H = self.n_kv_heads
        if self.layout == "split":
            return self.scales_record[:, :H].contiguous(), self.scales_record[:, H:].contiguous()
        off = 2 * H * self.head_dim
        ks = self.record[:, off:off + 4 * H].contiguous().view(torch.float32)
        vs = self.record[:, off + 4 * H:off + 8 * H].contiguous().view(torch.float32)
        return ks, vs

    def codes(self):
        return self.k_codes.contiguous(), self.v_codes.contiguous()

    def byte_size(self) -> int:
        return sum(b.numel() * b.element_size() for b in self._buffers)


# ------------------------------------------------------------------ calls --

def fp8kv_quantize_rows(pool: Fp8KvPool, k: torch.Tensor, v: torch.Tensor, slots: torch.Tensor,
                        stream=None) -> None:
    """Quantize bf16 K/V rows [N][Hkv][D] into pool rows slots[N] (int32)."""
    _dev_check(k, "k", torch.bfloat16)
    _dev_check(v, "v", torch.bfloat16)
    _dev_check(slots, "slots", torch.int32)
    n = int(slots.numel())
    D = pool.head_dim
    if k.shape != v.shape or k.dim() != 3 or k.shape[0] != n or k.shape[1:] != (pool.n_kv_heads, D):
        raise ValueError(f"k/v must be [{n}][{pool.n_kv_heads}][{D}], got {tuple(k.shape)} / {tuple(v.shape)}")
    if k.stride(2) != 1 or k.stride(1) != D or v.stride(2) != 1 or v.stride(1) != D:
        raise ValueError(f"k and v need contiguous [Hkv][{D}] rows")
    # a single token may carry any token stride (even 0); only token 0 is read
    stride = k.stride(0) if n > 1 else pool.n_kv_heads * D
    if n > 1 and v.stride(0) != stride:
        raise ValueError("k and v need the same token stride")
    st = load().fp8kv_quantize_rows(ctypes.byref(pool.layer), _ptr(_bits(k)), _ptr(_bits(v)), stride,
                                    _ptr(slots), n, _stream(stream))
    _check(st, "fp8kv_quantize_rows")


def fp8kv_decode_workspace_bytes(n_queries: int, n_q_heads: int, head_dim: int = HEAD_DIM,
                                 max_splits: int = 0) -> int:
    return int(load().fp8kv_decode_workspace_bytes(n_queries, n_q_heads, head_dim, max_splits))


def decode_workspace(n_queries: int, n_q_heads: int, max_splits: int = 0, device=None,
                     head_dim: int = HEAD_DIM) -> torch.Tensor:
    """Workspace for `n_queries` query rows (batch * n_qrows) of n_q_heads heads."""
    nbytes = fp8kv_decode_workspace_bytes(n_queries, n_q_heads, head_dim, max_splits)
    return torch.empty(nbytes, dtype=torch.uint8, device=device or "cuda")


def _decode_args(pool, q, row_table, seq_lens, max_seq_len, sm_scale, max_splits, workspace, multi=False):
    """Common marshalling; q is [B][Hq][D] or, with multi, [B][n_qrows][Hq][D]."""
    _dev_check(q, "q", torch.bfloat16)
    _dev_check(row_table, "row_table", torch.int32)
    _dev_check(seq_lens, "seq_lens", torch.int32)
    D = pool.head_dim
    want = 4 if multi else 3
    if q.dim() != want or q.shape[-1] != D or not q.is_contiguous():
        shape = "[B][n_qrows][Hq]" if multi else "[B][Hq]"
        raise ValueError(f"q must be a contiguous {shape}[{D}] bf16 tensor")
    B, Hq = int(q.shape[0]), int(q.shape[-2])
    nq = int(q.shape[1]) if multi else 1
    if row_table.dim() != 2 or row_table.shape[0] != B or row_table.stride(1) != 1:
        raise ValueError("row_table must be [B][stride] with unit inner stride")
    if seq_lens.numel() != B:
        raise ValueError("seq_lens must have B entries")
    if workspace is None:
        workspace = decode_workspace(B * nq, Hq, max_splits, q.device, D)
    # a size-1 batch dimension may carry any stride (even 0); only row 0 is read
    table_stride = row_table.stride(0) if B > 1 else max(int(row_table.shape[1]), 1)
    return dict(pool=ctypes.byref(pool.layer), q=_ptr(_bits(q)), B=B, nq=nq, Hq=Hq, table=_ptr(row_table),
                table_stride=table_stride, seq_lens=_ptr(seq_lens), max_seq_len=int(max_seq_len),
                sm_scale=float(sm_scale), max_splits=int(max_splits), ws=_ptr(workspace),
                ws_bytes=workspace.numel() * workspace.element_size()), workspace


def fp8kv_decode_attn(pool: Fp8KvPool, q: torch.Tensor, row_table: torch.Tensor, seq_lens: torch.Tensor,
                      max_seq_len: int, sm_scale: float, max_splits: int = 0,
                      workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
    """Decode attention: q bf16 [B][Hq][D], row_table int32 [B][stride], seq_lens int32 [B]."""
    a, workspace = _decode_args(pool, q, row_table, seq_lens, max_seq_len, sm_scale, max_splits, workspace)
    if out is None:
        out = torch.empty_like(q)
    st = load().fp8kv_decode_attn(a["pool"], a["q"], a["B"], a["Hq"], a["table"], a["table_stride"], a["seq_lens"],
                                  a["max_seq_len"], a["sm_scale"], a["max_splits"], a["ws"], a["ws_bytes"],
                                  _ptr(_bits(out)), _stream(stream))
    _check(st, "fp8kv_decode_attn")
    return out


def fp8kv_decode_attn_rows(pool: Fp8KvPool, q: torch.Tensor, row_table: torch.Tensor, seq_lens: torch.Tensor,
                           max_seq_len: int, sm_scale: float, window: int = 0, max_splits: int = 0,
                           workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                           stream=None) -> torch.Tensor:
    """Decode attention for n_qrows causal query rows per request (q bf16 [B][n_qrows][Hq][D],
    the request's last n_qrows positions) with an optional sliding window of `window` keys."""
    a, workspace = _decode_args(pool, q, row_table, seq_lens, max_seq_len, sm_scale, max_splits, workspace,
                                multi=True)
    if out is None:
        out = torch.empty_like(q)
    st = load().fp8kv_decode_attn_rows(a["pool"], a["q"], a["B"], a["nq"], a["Hq"], a["table"], a["table_stride"],
                                       a["seq_lens"], a["max_seq_len"], int(window), a["sm_scale"], a["max_splits"],
                                       a["ws"], a["ws_bytes"], _ptr(_bits(out)), _stream(stream))
    _check(st, "fp8kv_decode_attn_rows")
    return out


def fp8kv_decode_attn_rows_append(pool: Fp8KvPool, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                                  new_slots: torch.Tensor, row_table: torch.Tensor, seq_lens: torch.Tensor,
                                  max_seq_len: int, sm_scale: float, window: int = 0, max_splits: int = 0,
                                  workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                                  stream=None) -> torch.Tensor:
    """Several new tokens per request in one step: quantize token j of request b (k_new/v_new bf16
    [B][n_qrows][Hkv][D]) into pool row new_slots[b][j] (== row_table[b][seq_lens[b] - n_qrows + j])
    and attend with the n_qrows causal query rows (q bf16 [B][n_qrows][Hq][D]), optionally within a
    sliding window of `window` keys."""
    a, workspace = _decode_args(pool, q, row_table, seq_lens, max_seq_len, sm_scale, max_splits, workspace,
                                multi=True)
    B, nq, D = a["B"], a["nq"], pool.head_dim
    _dev_check(k_new, "k_new", torch.bfloat16)
    _dev_check(v_new, "v_new", torch.bfloat16)
    shape = (B, nq, pool.n_kv_heads, D)
    if tuple(k_new.shape) != shape or tuple(v_new.shape) != shape:
        raise ValueError(f"k_new/v_new must be {list(shape)}, got {tuple(k_new.shape)} / {tuple(v_new.shape)}")
    if not k_new.is_contiguous() or not v_new.is_contiguous():
        raise ValueError("k_new and v_new must be contiguous")
    _dev_check(new_slots, "new_slots", torch.int32)
    if new_slots.numel() != B * nq or not new_slots.is_contiguous():
        raise ValueError("new_slots must be a contiguous [B][n_qrows] tensor")
    if out is None:
        out = torch.empty_like(q)
    st = load().fp8kv_decode_attn_rows_append(a["pool"], a["q"], B, nq, a["Hq"], _ptr(_bits(k_new)),
                                              _ptr(_bits(v_new)), pool.n_kv_heads * D, _ptr(new_slots), a["table"],
                                              a["table_stride"], a["seq_lens"], a["max_seq_len"], int(window),
                                              a["sm_scale"], a["max_splits"], a["ws"], a["ws_bytes"],
                                              _ptr(_bits(out)), _stream(stream))
    _check(st, "fp8kv_decode_attn_rows_append")
    return out


def fp8kv_decode_attn_append(pool: Fp8KvPool, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                             new_slots: torch.Tensor, row_table: torch.Tensor, seq_lens: torch.Tensor,
                             max_seq_len: int, sm_scale: float, max_splits: int = 0,
                             workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                             stream=None, window: int = 0) -> torch.Tensor:
    """One decode step: quantize each request's new token (k_new/v_new bf16 [B][Hkv][D]) into
    pool row new_slots[b] (== row_table[b][seq_lens[b] - 1]) and attend over positions [0, seq_lens[b])
    (the last `window` of them when window > 0: fp8kv_decode_attn_append_window)."""
    a, workspace = _decode_args(pool, q, row_table, seq_lens, max_seq_len, sm_scale, max_splits, workspace)
    B, D = a["B"], pool.head_dim
    _dev_check(k_new, "k_new", torch.bfloat16)
    _dev_check(v_new, "v_new", torch.bfloat16)
    shape = (B, pool.n_kv_heads, D)
    if tuple(k_new.shape) != shape or tuple(v_new.shape) != shape:
        raise ValueError(f"k_new/v_new must be {list(shape)}, got {tuple(k_new.shape)} / {tuple(v_new.shape)}")
    if k_new.stride(2) != 1 or k_new.stride(1) != D or v_new.stride(2) != 1 or v_new.stride(1) != D:
        raise ValueError(f"k_new and v_new need contiguous [Hkv][{D}] rows")
    stride = k_new.stride(0) if B > 1 else pool.n_kv_heads * D
    if B > 1 and v_new.stride(0) != stride:
        raise ValueError("k_new and v_new need the same token stride")
    _dev_check(new_slots, "new_slots", torch.int32)
    if new_slots.numel() != B:
        raise ValueError("new_slots must have B entries")
    if out is None:
        out = torch.empty_like(q)
    if window:
        st = load().fp8kv_decode_attn_append_window(a["pool"], a["q"], B, a["Hq"], _ptr(_bits(k_new)),
                                                    _ptr(_bits(v_new)), stride, _ptr(new_slots), a["table"],
                                                    a["table_stride"], a["seq_lens"], a["max_seq_len"], int(window),
                                                    a["sm_scale"], a["max_splits"], a["ws"], a["ws_bytes"],
                                                    _ptr(_bits(out)), _stream(stream))
        _check(st, "fp8kv_decode_attn_append_window")
        return out
    st = load().fp8kv_decode_attn_append(a["pool"], a["q"], B, a["Hq"], _ptr(_bits(k_new)), _ptr(_bits(v_new)), stride,
                                         _ptr(new_slots), a["table"], a["table_stride"], a["seq_lens"],
                                         a["max_seq_len"], a["sm_scale"], a["max_splits"], a["ws"], a["ws_bytes"],
                                         _ptr(_bits(out)), _stream(stream))
    _check(st, "fp8kv_decode_attn_append")
    return out


def fp8kv_decode_attn_append_noalloc(pool: Fp8KvPool, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                                     new_slots: torch.Tensor, row_table: torch.Tensor, seq_lens: torch.Tensor,
                                     max_seq_len: int, sm_scale: float, max_splits: int = 0,
                                     out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """fp8kv_decode_attn_append without a workspace: the split partials live in the
    library's fixed per-device array (calls on one device must not overlap)."""
    _dev_check(q, "q", torch.bfloat16)
    _dev_check(row_table, "row_table", torch.int32)
    _dev_check(seq_lens, "seq_lens", torch.int32)
    D = pool.head_dim
    if q.dim() != 3 or q.shape[-1] != D or not q.is_contiguous():
        raise ValueError(f"q must be a contiguous [B][Hq][{D}] bf16 tensor")
    B, Hq = int(q.shape[0]), int(q.shape[1])
    if row_table.dim() != 2 or row_table.shape[0] != B or row_table.stride(1) != 1:
        raise ValueError("row_table must be [B][stride] with unit inner stride")
    if seq_lens.numel() != B:
        raise ValueError("seq_lens must have B entries")
    table_stride = row_table.stride(0) if B > 1 else max(int(row_table.shape[1]), 1)
    _dev_check(k_new, "k_new", torch.bfloat16)
    _dev_check(v_new, "v_new", torch.bfloat16)
    shape = (B, pool.n_kv_heads, D)
    if tuple(k_new.shape) != shape or tuple(v_new.shape) != shape:
        raise ValueError(f"k_new/v_new must be {list(shape)}, got {tuple(k_new.shape)} / {tuple(v_new.shape)}")
    if not k_new.is_contiguous() or not v_new.is_contiguous():
        raise ValueError("k_new and v_new must be contiguous")
    _dev_check(new_slots, "new_slots", torch.int32)
    if new_slots.numel() != B:
        raise ValueError("new_slots must have B entries")
    if out is None:
        out = torch.empty_like(q)
    st = load().fp8kv_decode_attn_append_noalloc(ctypes.byref(pool.layer), _ptr(_bits(q)), B, Hq, _ptr(_bits(k_new)),
                                                 _ptr(_bits(v_new)), pool.n_kv_heads * D, _ptr(new_slots),
                                                 _ptr(row_table), table_stride, _ptr(seq_lens), int(max_seq_len),
                                                 float(sm_scale), int(max_splits), _ptr(_bits(out)), _stream(stream))
    _check(st, "fp8kv_decode_attn_append_noalloc")
    return out


def fp8kv_decode_stage1(pool: Fp8KvPool, q: torch.Tensor, row_table: torch.Tensor, seq_lens: torch.Tensor,
                        max_seq_len: int, sm_scale: float, max_splits: int = 0,
                        workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """First (split-K) stage only; returns the workspace holding the partials."""
    a, workspace = _decode_args(pool, q, row_table, seq_lens, max_seq_len, sm_scale, max_splits, workspace)
    st = load().fp8kv_decode_stage1(a["pool"], a["q"], a["B"], a["Hq"], a["table"], a["table_stride"], a["seq_lens"],
                                    a["max_seq_len"], a["sm_scale"], a["max_splits"], a["ws"], a["ws_bytes"],
                                    _stream(stream))
    _check(st, "fp8kv_decode_stage1")
    return workspace


def fp8kv_decode_stage1_valu(pool: Fp8KvPool, q: torch.Tensor, row_table: torch.Tensor, seq_lens: torch.Tensor,
                             max_seq_len: int, sm_scale: float, max_splits: int = 0,
                             workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Stage 1 on the vector units (no MFMA), same partials as fp8kv_decode_stage1;
    returns the workspace for fp8kv_decode_merge."""
    a, workspace = _decode_args(pool, q, row_table, seq_lens, max_seq_len, sm_scale, max_splits, workspace)
    st = load().fp8kv_decode_stage1_valu(a["pool"], a["q"], a["B"], a["Hq"], a["table"], a["table_stride"],
                                         a["seq_lens"], a["max_seq_len"], a["sm_scale"], a["max_splits"], a["ws"],
                                         a["ws_bytes"], _stream(stream))
    _check(st, "fp8kv_decode_stage1_valu")
    return workspace


def fp8kv_decode_merge(workspace: torch.Tensor, batch: int, n_q_heads: int, max_splits: int = 0,
                       out: Optional[torch.Tensor] = None, stream=None, head_dim: int = HEAD_DIM) -> torch.Tensor:
    """Merge the partials of a preceding fp8kv_decode_stage1 into bf16 out [B][Hq][D]."""
    if out is None:
        out = torch.empty((batch, n_q_heads, head_dim), dtype=torch.bfloat16, device=workspace.device)
    st = load().fp8kv_decode_merge(batch, n_q_heads, head_dim, max_splits, _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _ptr(_bits(out)),
                                   _stream(stream))
    _check(st, "fp8kv_decode_merge")
    return out


def fp8kv_prefill_attn(pool: Fp8KvPool, q: torch.Tensor, k_cur: torch.Tensor, v_cur: torch.Tensor,
                       prefix_rows: Optional[torch.Tensor], ws_k: Optional[torch.Tensor],
                       ws_v: Optional[torch.Tensor], sm_scale: float, out: Optional[torch.Tensor] = None,
                       stream=None) -> torch.Tensor:
    """Prefill attention of a bf16 chunk over historical FP8 rows prefix_rows (int32 [P]).

    ws_k / ws_v: bf16 workspaces of at least P rows of [Hkv][128] (shared across layers).
    """
    for name, t in (("q", q), ("k_cur", k_cur), ("v_cur", v_cur)):
        _dev_check(t, name, torch.bfloat16)
        if not t.is_contiguous() or t.dim() != 3 or t.shape[2] != HEAD_DIM:
            raise ValueError(f"{name} must be a contiguous [T][H][128] bf16 tensor")
    T, Hq, _ = q.shape
    if k_cur.shape != (T, pool.n_kv_heads, HEAD_DIM) or v_cur.shape != k_cur.shape:
        raise ValueError("k_cur/v_cur must be [T][Hkv][128]")
    P = 0 if prefix_rows is None else int(prefix_rows.numel())
    cap = 0
    if P > 0:
        _dev_check(prefix_rows, "prefix_rows", torch.int32)
        for name, t in (("ws_k", ws_k), ("ws_v", ws_v)):
            _dev_check(t, name, torch.bfloat16)
            if not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous")
        cap = min(ws_k.numel(), ws_v.numel()) // (pool.n_kv_heads * HEAD_DIM)
    if out is None:
        out = torch.empty_like(q)
    st = load().fp8kv_prefill_attn(ctypes.byref(pool.layer), _ptr(_bits(q)), _ptr(_bits(k_cur)), _ptr(_bits(v_cur)),
                                   T, Hq, _ptr(prefix_rows) if P else None, P,
                                   _ptr(_bits(ws_k)) if P else None, _ptr(_bits(ws_v)) if P else None, cap,
                                   float(sm_scale), _ptr(_bits(out)), _stream(stream))
    _check(st, "fp8kv_prefill_attn")
    return out


def fp8kv_prefill_attn_workspace(q: torch.Tensor, k_cur: torch.Tensor, v_cur: torch.Tensor,
                                 ws_k: Optional[torch.Tensor], ws_v: Optional[torch.Tensor], sm_scale: float,
                                 out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Causal chunk attention over bf16 prefix rows already in a workspace (ws_k / ws_v
    [P][Hkv][128], or None for P = 0): step 2 of fp8kv_prefill_attn alone."""
    for name, t in (("q", q), ("k_cur", k_cur), ("v_cur", v_cur)):
        _dev_check(t, name, torch.bfloat16)
        if not t.is_contiguous() or t.dim() != 3 or t.shape[2] != HEAD_DIM:
            raise ValueError(f"{name} must be a contiguous [T][H][128] bf16 tensor")
    T, Hq, _ = q.shape
    Hkv = int(k_cur.shape[1])
    if k_cur.shape != (T, Hkv, HEAD_DIM) or v_cur.shape != k_cur.shape:
        raise ValueError("k_cur/v_cur must be [T][Hkv][128]")
    P = 0
    if ws_k is not None:
        for name, t in (("ws_k", ws_k), ("ws_v", ws_v)):
            _dev_check(t, name, torch.bfloat16)
            if not t.is_contiguous() or t.dim() != 3 or tuple(t.shape[1:]) != (Hkv, HEAD_DIM):
                raise ValueError(f"{name} must be a contiguous [P][{Hkv}][128] bf16 tensor")
        if ws_v.shape != ws_k.shape:
            raise ValueError("ws_k and ws_v must have the same shape")
        P = int(ws_k.shape[0])
    if out is None:
        out = torch.empty_like(q)
    st = load().fp8kv_prefill_attn_workspace(_ptr(_bits(q)), _ptr(_bits(k_cur)), _ptr(_bits(v_cur)), T, Hq, Hkv,
                                             _ptr(_bits(ws_k)) if P else None, _ptr(_bits(ws_v)) if P else None, P,
                                             float(sm_scale), _ptr(_bits(out)), _stream(stream))
    _check(st, "fp8kv_prefill_attn_workspace")
    return out
