"""Python binding of libtpla.so (ctypes).

Argument marshalling only: every computation runs in the library's HIP
kernels.  torch supplies device memory (tensors) and the current stream.
Functions raise TplaError on a non-zero status.  If the library has not been
built the first call raises RuntimeError; there is no fallback.
"""

from __future__ import annotations

import ctypes
import math
import os
import re
from typing import List, Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# TPLA_LIB names another build of the same library (the host-side
# sanitizer build, tensor_latent_decode_amd/build_sanitize.py)
LIB_PATH = os.environ.get("TPLA_LIB") or os.path.join(_HERE, "libtpla.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "tpla.h")

FP32, BF16 = 0, 1
STATUS = {0: "TPLA_OK", 1: "TPLA_ERR_NULL", 2: "TPLA_ERR_SHAPE", 3: "TPLA_ERR_ALIGN",
          4: "TPLA_ERR_DTYPE", 5: "TPLA_ERR_UNSUPPORTED", 6: "TPLA_ERR_WORKSPACE",
          7: "TPLA_ERR_HIP"}


class TplaError(RuntimeError):
    def __init__(self, func: str, status: int, message: str):
        self.status = status
        super().__init__(f"{func}: {STATUS.get(status, status)}: {message}")


class DecodeArgs(ctypes.Structure):
    """Mirror of tpla_decode_args (include/tpla.h)."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("d_s", ctypes.c_int32),
        ("d_r", ctypes.c_int32), ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int32), ("dtype", ctypes.c_int), ("scale", ctypes.c_float),
        ("q_latent", ctypes.c_void_p), ("q_latent_stride_b", ctypes.c_int64),
        ("q_latent_stride_h", ctypes.c_int64),
        ("q_rope", ctypes.c_void_p), ("q_rope_stride_b", ctypes.c_int64),
        ("q_rope_stride_h", ctypes.c_int64),
        ("cache", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
        ("out", ctypes.c_void_p), ("out_dtype", ctypes.c_int),
        ("out_stride_b", ctypes.c_int64), ("out_stride_h", ctypes.c_int64),
        ("lse", ctypes.c_void_p), ("num_splits", ctypes.c_int32),
    ]


class PrefillArgs(ctypes.Structure):
    """Mirror of tpla_prefill_args (include/tpla.h)."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("d_c", ctypes.c_int32),
        ("d_r", ctypes.c_int32), ("max_len", ctypes.c_int32), ("dtype", ctypes.c_int),
        ("scale", ctypes.c_float),
        ("q_latent", ctypes.c_void_p), ("q_latent_stride_b", ctypes.c_int64),
        ("q_latent_stride_t", ctypes.c_int64), ("q_latent_stride_h", ctypes.c_int64),
        ("q_rope", ctypes.c_void_p), ("q_rope_stride_b", ctypes.c_int64),
        ("q_rope_stride_t", ctypes.c_int64), ("q_rope_stride_h", ctypes.c_int64),
        ("kv", ctypes.c_void_p), ("kv_stride_b", ctypes.c_int64), ("kv_stride_t", ctypes.c_int64),
        ("seq_lens", ctypes.c_void_p),
        ("out", ctypes.c_void_p), ("out_dtype", ctypes.c_int),
        ("out_stride_b", ctypes.c_int64), ("out_stride_t", ctypes.c_int64),
        ("out_stride_h", ctypes.c_int64),
        ("lse", ctypes.c_void_p),
    ]


class RotateAppendArgs(ctypes.Structure):
    """Mirror of tpla_rotate_append_args (include/tpla.h)."""
    _fields_ = [
        ("n", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("q_dtype", ctypes.c_int), ("q_row_stride", ctypes.c_int64),
        ("q_out", ctypes.c_void_p), ("q_out_dtype", ctypes.c_int),
        ("q_out_row_stride", ctypes.c_int64), ("q_rows", ctypes.c_int64),
        ("latent", ctypes.c_void_p), ("rope", ctypes.c_void_p), ("src_dtype", ctypes.c_int),
        ("latent_row_stride", ctypes.c_int64), ("rope_row_stride", ctypes.c_int64),
        ("latent_out", ctypes.c_void_p), ("latent_out_row_stride", ctypes.c_int64),
        ("n_rows", ctypes.c_int32), ("row_seq", ctypes.c_void_p), ("row_pos", ctypes.c_void_p),
        ("caches", ctypes.POINTER(ctypes.c_void_p)), ("n_caches", ctypes.c_int32),
        ("first_shard", ctypes.c_int32), ("cache_dtype", ctypes.c_int),
        ("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32), ("d_s", ctypes.c_int32),
        ("d_r", ctypes.c_int32), ("block_table", ctypes.c_void_p),
        ("max_blocks_per_seq", ctypes.c_int32), ("batch", ctypes.c_int32),
        ("latent_norm", ctypes.c_int32), ("norm_eps", ctypes.c_float),
    ]


NORMS = {"none": 0, "global": 1, "slice": 2}   # TPLA_NORM_*

_lib = None


def lib() -> ctypes.CDLL:
    """Load libtpla.so once and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m tensor_latent_decode_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    dt = ctypes.c_int
    L.tpla_hadamard_latent.argtypes = [vp, dt, i64, vp, dt, i64, i64, i32, vp]
    L.tpla_append_kv.argtypes = [vp, dt, i32, i32, i32, i32, vp, i32, i32, vp, vp, i32, vp, i64,
                                 vp, i64, dt, vp]
    L.tpla_decode_workspace_size.argtypes = [ctypes.POINTER(DecodeArgs), ctypes.POINTER(sz)]
    L.tpla_decode_shard.argtypes = [ctypes.POINTER(DecodeArgs), vp, sz, vp]
    L.tpla_decode_shard_noalloc.argtypes = [ctypes.POINTER(DecodeArgs), vp]
    L.tpla_decode_noalloc_scratch_bytes.argtypes = []
    L.tpla_decode_noalloc_scratch_bytes.restype = sz
    L.tpla_combine_shards.argtypes = [ctypes.POINTER(vp), dt, i32, i32, i32, i32, vp, dt, i32, vp]
    L.tpla_rotate_append.argtypes = [ctypes.POINTER(RotateAppendArgs), vp]
    L.tpla_decode_suggest_splits.argtypes = [ctypes.POINTER(DecodeArgs), vp, ctypes.POINTER(i32)]
    L.tpla_decode_suggest_splits_cus.argtypes = [ctypes.POINTER(DecodeArgs), vp, i32,
                                                 ctypes.POINTER(i32)]
    L.tpla_up_project.argtypes = [vp, dt, i64, i64, vp, dt, i64, i64, vp, dt, i64, i64,
                                  i32, i32, i32, i32, i32, vp]
    L.tpla_mla_prefill.argtypes = [ctypes.POINTER(PrefillArgs), vp]
    for f in ("tpla_hadamard_latent", "tpla_append_kv", "tpla_decode_workspace_size",
              "tpla_decode_shard", "tpla_decode_shard_noalloc", "tpla_combine_shards", "tpla_rotate_append",
              "tpla_decode_suggest_splits", "tpla_decode_suggest_splits_cus", "tpla_up_project",
              "tpla_mla_prefill"):
        getattr(L, f).restype = ctypes.c_int
    L.tpla_status_string.argtypes = [ctypes.c_int]
    L.tpla_status_string.restype = ctypes.c_char_p
    L.tpla_last_error.argtypes = []
    L.tpla_last_error.restype = ctypes.c_char_p
    L.tpla_version.argtypes = []
    L.tpla_version.restype = ctypes.c_int32
    _lib = L
    return L


def header_functions() -> List[str]:
    """Names of the functions include/tpla.h declares."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tpla_[a-z_0-9]+)\s*\(", text)))


def _check(name: str, status: int) -> None:
    if status != 0:
        raise TplaError(name, status, lib().tpla_last_error().decode())


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return FP32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _dt_of(dtype: torch.dtype) -> int:
    return _dt(torch.empty(0, dtype=dtype))


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _gpu(*ts: Optional[torch.Tensor]) -> None:
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must live on the GPU")


def _rows(x: torch.Tensor):
    """(rows, n, row_stride) of a tensor whose leading dims collapse to one."""
    if x.dim() < 1 or x.stride(-1) != 1:
        raise ValueError("last dimension must be contiguous")
    n = x.shape[-1]
    if x.dim() == 1:
        return 1, n, n
    try:
        flat = x.view(-1, n)
    except RuntimeError as e:
        raise ValueError("rows must be addressable with a single row stride") from e
    return flat.shape[0], n, (flat.stride(0) if flat.shape[0] > 1 else n)


def hadamard_latent(x: torch.Tensor, out: Optional[torch.Tensor] = None,
                    out_dtype: Optional[torch.dtype] = None) -> torch.Tensor:
    """out[..., :] = x[..., :] @ H_n / sqrt(n) over the last dimension."""
    _gpu(x, out)
    if out is None:
        out = torch.empty(x.shape, dtype=out_dtype or x.dtype, device=x.device)
    if out.shape != x.shape:
        raise ValueError("out must have x's shape")
    rows, n, xs = _rows(x)
    _, _, ys = _rows(out)
    _check("tpla_hadamard_latent",
           lib().tpla_hadamard_latent(x.data_ptr(), _dt(x), xs, out.data_ptr(), _dt(out), ys,
                                      rows, n, _stream(x)))
    return out


def append_kv(cache: torch.Tensor, block_table: torch.Tensor, row_seq: torch.Tensor,
              row_pos: torch.Tensor, latent: torch.Tensor, rope: Optional[torch.Tensor],
              batch: Optional[int] = None) -> None:
    """Write rows [latent_t || rope_t] into the paged cache [blocks, bs, d_s + d_r]."""
    _gpu(cache, block_table, row_seq, row_pos, latent, rope)
    if rope is not None and rope.shape[-1] == 0:
        rope = None
    num_blocks, bs, width = cache.shape
    d_s = latent.shape[-1]
    d_r = 0 if rope is None else rope.shape[-1]
    if width != d_s + d_r or not cache.is_contiguous():
        raise ValueError("cache must be contiguous [num_blocks, block_size, d_s + d_r]")
    for t in (block_table, row_seq, row_pos):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError("block_table, row_seq, row_pos must be contiguous int32")
    n_rows = latent.shape[0]
    if latent.stride(-1) != 1 or (rope is not None and rope.stride(-1) != 1):
        raise ValueError("latent/rope rows must be contiguous")
    if rope is not None and rope.dtype != latent.dtype:
        raise ValueError("latent and rope must share a dtype")
    batch = block_table.shape[0] if batch is None else batch
    _check("tpla_append_kv",
           lib().tpla_append_kv(cache.data_ptr(), _dt(cache), num_blocks, bs, d_s, d_r,
                                block_table.data_ptr(), block_table.shape[1], batch,
                                row_seq.data_ptr(), row_pos.data_ptr(), n_rows,
                                latent.data_ptr(), latent.stride(0) if n_rows > 1 else d_s,
                                None if rope is None else rope.data_ptr(),
                                0 if rope is None else (rope.stride(0) if n_rows > 1 else d_r),
                                _dt(latent), _stream(cache)))


def rotate_append(q: Optional[torch.Tensor], q_out: Optional[torch.Tensor],
                  latent: Optional[torch.Tensor], rope: Optional[torch.Tensor],
                  row_seq: Optional[torch.Tensor] = None, row_pos: Optional[torch.Tensor] = None,
                  caches: Sequence[torch.Tensor] = (), block_table: Optional[torch.Tensor] = None,
                  first_shard: int = 0, latent_out: Optional[torch.Tensor] = None,
                  batch: Optional[int] = None, latent_norm: str = "none", norm_eps: float = 1e-6,
                  slice_width: Optional[int] = None) -> None:
    """One launch: q_out = q . H_n/sqrt(n) over the last dim; the new latent
    rows rotated the same way, RMS-normalised per `latent_norm` ("none",
    "global": the whole row, "slice": each slice_width-column slice on its
    own; slice_width defaults to the caches' d_s), stored into latent_out if
    given, and their shard slices first_shard, first_shard+1, ... appended
    with the rope into `caches` (each [num_blocks, block_size, d_s + d_r])."""
    if latent_norm not in NORMS:
        raise ValueError(f"latent_norm must be one of {sorted(NORMS)}")
    _gpu(q, q_out, latent, rope, row_seq, row_pos, block_table, latent_out, *caches)
    a = RotateAppendArgs()
    n = None
    if q is not None:
        if q_out is None or q_out.shape != q.shape:
            raise ValueError("q_out must have q's shape")
        rows, n, qs = _rows(q)
        _, _, qos = _rows(q_out)
        a.q, a.q_dtype, a.q_row_stride = q.data_ptr(), _dt(q), qs
        a.q_out, a.q_out_dtype, a.q_out_row_stride = q_out.data_ptr(), _dt(q_out), qos
        a.q_rows = rows
    if rope is not None and rope.shape[-1] == 0:
        rope = None
    keep = []
    if latent is not None:
        if latent.dim() != 2 or latent.stride(-1) != 1:
            raise ValueError("latent must be [n_rows, n] with contiguous rows")
        n_rows, nl = latent.shape
        if n is not None and nl != n:
            raise ValueError("latent and q rows must have the same width")
        n = nl
        a.latent, a.src_dtype = latent.data_ptr(), _dt(latent)
        a.latent_row_stride = latent.stride(0) if n_rows > 1 else n
        a.n_rows = n_rows
        if rope is not None:
            if rope.dtype != latent.dtype or rope.stride(-1) != 1:
                raise ValueError("rope must share latent's dtype and have contiguous rows")
            a.rope, a.d_r = rope.data_ptr(), rope.shape[-1]
            a.rope_row_stride = rope.stride(0) if n_rows > 1 else rope.shape[-1]
        if latent_out is not None:
            if latent_out.shape != latent.shape or latent_out.dtype != latent.dtype:
                raise ValueError("latent_out must match latent")
            a.latent_out = latent_out.data_ptr()
            a.latent_out_row_stride = latent_out.stride(0) if n_rows > 1 else n
        if caches:
            if block_table is None or row_seq is None or row_pos is None:
                raise ValueError("caches need block_table, row_seq and row_pos")
            for t in (block_table, row_seq, row_pos):
                if t.dtype != torch.int32 or not t.is_contiguous():
                    raise ValueError("block_table, row_seq, row_pos must be contiguous int32")
            c0 = caches[0]
            num_blocks, bs, width = c0.shape
            for c in caches:
                if c.shape != c0.shape or c.dtype != c0.dtype or not c.is_contiguous():
                    raise ValueError("caches must be alike and contiguous")
            arr = (ctypes.c_void_p * len(caches))(*[c.data_ptr() for c in caches])
            keep.append(arr)
            a.caches = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
            a.n_caches, a.first_shard, a.cache_dtype = len(caches), first_shard, _dt(c0)
            a.num_blocks, a.block_size, a.d_s = num_blocks, bs, width - a.d_r
            a.block_table, a.max_blocks_per_seq = block_table.data_ptr(), block_table.shape[1]
            a.batch = block_table.shape[0] if batch is None else batch
            a.row_seq, a.row_pos = row_seq.data_ptr(), row_pos.data_ptr()
    if n is None:
        return
    a.n = n
    a.latent_norm, a.norm_eps = NORMS[latent_norm], norm_eps
    if slice_width is not None:
        if caches and slice_width != a.d_s:
            raise ValueError("slice_width must equal the caches' d_s")
        a.d_s = slice_width
    elif latent_norm == "slice" and not caches:
        raise ValueError("the slice norm needs slice_width or caches")
    dev_t = q if q is not None else latent
    _check("tpla_rotate_append", lib().tpla_rotate_append(ctypes.byref(a), _stream(dev_t)))


def up_project(o: torch.Tensor, w: torch.Tensor, out: Optional[torch.Tensor] = None,
               accumulate: bool = False, out_dtype: Optional[torch.dtype] = None) -> torch.Tensor:
    """out[b, h, :] (+)= w[h] @ o[b, h, :] for o [B, H, d_s] and w [H, d_v, d_s]
    (W_UV's columns of one device's latent slice; a column slice of the full
    [H, d_v, d_c] weight is fine); accumulate=True adds into `out`, which is
    how the shards' terms are summed on one device."""
    _gpu(o, w, out)
    if o.dim() != 3 or w.dim() != 3 or o.stride(-1) != 1 or w.stride(-1) != 1:
        raise ValueError("o must be [B, H, d_s] and w [H, d_v, d_s] with contiguous last dims")
    B, H, d_s = o.shape
    if w.shape[0] != H or w.shape[2] != d_s:
        raise ValueError("w must be [H, d_v, d_s] matching o")
    d_v = w.shape[1]
    if out is None:
        if accumulate:
            raise ValueError("accumulate needs out")
        out = torch.empty((B, H, d_v), dtype=out_dtype or torch.float32, device=o.device)
    if out.shape != (B, H, d_v) or out.stride(-1) != 1:
        raise ValueError("out must be [B, H, d_v] with a contiguous last dim")
    _check("tpla_up_project",
           lib().tpla_up_project(o.data_ptr(), _dt(o), o.stride(0), o.stride(1),
                                 w.data_ptr(), _dt(w), w.stride(0), w.stride(1),
                                 out.data_ptr(), _dt(out), out.stride(0), out.stride(1),
                                 B, H, d_s, d_v, int(accumulate), _stream(o)))
    return out


def make_decode_args(q_latent: torch.Tensor, q_rope: Optional[torch.Tensor], cache: torch.Tensor,
                     block_table: torch.Tensor, seq_lens: torch.Tensor, scale: float,
                     max_seq_len: int, out: torch.Tensor, lse: Optional[torch.Tensor] = None,
                     num_splits: int = 0) -> DecodeArgs:
    if q_rope is not None and q_rope.shape[-1] == 0:
        q_rope = None
    B, H, d_s = q_latent.shape
    d_r = 0 if q_rope is None else q_rope.shape[-1]
    num_blocks, bs, width = cache.shape
    if width != d_s + d_r:
        raise ValueError(f"cache row width {width} != d_s + d_r = {d_s + d_r}")
    if q_latent.stride(-1) != 1 or (q_rope is not None and q_rope.stride(-1) != 1):
        raise ValueError("query rows must be contiguous in their last dimension")
    if out.shape != (B, H, d_s) or out.stride(-1) != 1:
        raise ValueError("out must be [batch, heads, d_s] with a contiguous last dimension")
    if lse is not None and (lse.shape != (B, H) or lse.dtype != torch.float32
                            or not lse.is_contiguous()):
        raise ValueError("lse must be contiguous float32 [batch, heads]")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_table and seq_lens must be int32")
    if not (block_table.is_contiguous() and seq_lens.is_contiguous()):
        raise ValueError("block_table and seq_lens must be contiguous")
    if q_rope is not None and q_rope.dtype != q_latent.dtype:
        raise ValueError("q_latent and q_rope must share a dtype")
    if cache.dtype != q_latent.dtype:
        raise ValueError("query and cache must share a dtype")
    a = DecodeArgs()
    a.batch, a.heads, a.d_s, a.d_r = B, H, d_s, d_r
    a.block_size, a.num_blocks, a.max_blocks_per_seq = bs, num_blocks, block_table.shape[1]
    a.max_seq_len = int(max_seq_len)
    a.dtype = _dt(q_latent)
    a.scale = float(scale)
    a.q_latent = q_latent.data_ptr()
    a.q_latent_stride_b, a.q_latent_stride_h = q_latent.stride(0), q_latent.stride(1)
    if q_rope is not None:
        a.q_rope = q_rope.data_ptr()
        a.q_rope_stride_b, a.q_rope_stride_h = q_rope.stride(0), q_rope.stride(1)
    else:
        a.q_rope, a.q_rope_stride_b, a.q_rope_stride_h = None, 0, 0
    a.cache = cache.data_ptr()
    a.block_table = block_table.data_ptr()
    a.seq_lens = seq_lens.data_ptr()
    a.out = out.data_ptr()
    a.out_dtype = _dt(out)
    a.out_stride_b, a.out_stride_h = out.stride(0), out.stride(1)
    a.lse = None if lse is None else lse.data_ptr()
    a.num_splits = int(num_splits)
    return a


def decode_suggest_splits(args: "DecodeArgs", seq_lens_host, cus: Optional[int] = None) -> int:
    """Split count for `args` from the host copy of the sequence lengths, for
    the current device, or for a device of `cus` CUs (no device query)."""
    import numpy as np
    lens = np.ascontiguousarray(np.asarray(seq_lens_host, dtype=np.int32))
    if lens.shape != (args.batch,):
        raise ValueError("seq_lens_host must hold one length per sequence")
    out = ctypes.c_int32(0)
    ptr = lens.ctypes.data_as(ctypes.c_void_p)
    if cus is None:
        _check("tpla_decode_suggest_splits",
               lib().tpla_decode_suggest_splits(ctypes.byref(args), ptr, ctypes.byref(out)))
    else:
        _check("tpla_decode_suggest_splits_cus",
               lib().tpla_decode_suggest_splits_cus(ctypes.byref(args), ptr, int(cus),
                                                    ctypes.byref(out)))
    return int(out.value)


def decode_workspace_size(args: DecodeArgs) -> int:
    n = ctypes.c_size_t(0)
    _check("tpla_decode_workspace_size", lib().tpla_decode_workspace_size(ctypes.byref(args),
                                                                          ctypes.byref(n)))
    return n.value


def decode_workspace(args: DecodeArgs, device=None) -> torch.Tensor:
    """A device workspace of the size tpla_decode_shard needs for `args`."""
    need = decode_workspace_size(args)
    return torch.empty(max(need, 1), dtype=torch.uint8, device=device or "cuda")


def decode_shard(q_latent: torch.Tensor, q_rope: Optional[torch.Tensor], cache: torch.Tensor,
                 block_table: torch.Tensor, seq_lens: torch.Tensor, scale: float,
                 max_seq_len: int, out: Optional[torch.Tensor] = None,
                 lse: Optional[torch.Tensor] = None, num_splits: int = 0,
                 workspace: Optional[torch.Tensor] = None,
                 out_dtype: torch.dtype = torch.float32):
    """One shard's decode step.  Returns (out [B, H, d_s], lse [B, H] or None)."""
    _gpu(q_latent, q_rope, cache, block_table, seq_lens, out, lse, workspace)
    B, H, d_s = q_latent.shape
    if out is None:
        out = torch.empty((B, H, d_s), dtype=out_dtype, device=q_latent.device)
    args = make_decode_args(q_latent, q_rope, cache, block_table, seq_lens, scale, max_seq_len,
                            out, lse, num_splits)
    if workspace is None:
        workspace = decode_workspace(args, q_latent.device)
    nbytes = workspace.numel() * workspace.element_size()
    _check("tpla_decode_shard", lib().tpla_decode_shard(ctypes.byref(args), workspace.data_ptr(),
                                                        nbytes, _stream(q_latent)))
    return out, lse


def decode_shard_noalloc(q_latent: torch.Tensor, q_rope: Optional[torch.Tensor],
                         cache: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
                         scale: float, max_seq_len: int, out: torch.Tensor,
                         lse: Optional[torch.Tensor] = None, num_splits: int = 0):
    """decode_shard through tpla_decode_shard_noalloc: the library's static device
    scratch holds the split outputs, and nothing is allocated (so `out` is required)."""
    _gpu(q_latent, q_rope, cache, block_table, seq_lens, out, lse)
    args = make_decode_args(q_latent, q_rope, cache, block_table, seq_lens, scale, max_seq_len,
                            out, lse, num_splits)
    _check("tpla_decode_shard_noalloc",
           lib().tpla_decode_shard_noalloc(ctypes.byref(args), _stream(q_latent)))
    return out, lse


def decode_noalloc_scratch_bytes() -> int:
    return int(lib().tpla_decode_noalloc_scratch_bytes())


def make_prefill_args(q_latent: torch.Tensor, q_rope: torch.Tensor, kv: torch.Tensor,
                      seq_lens: torch.Tensor, scale: float, out: torch.Tensor,
                      lse: Optional[torch.Tensor] = None) -> PrefillArgs:
    """Arguments of tpla_mla_prefill from q_latent [B, S, H, d_c], q_rope [B, S, H, d_r],
    kv [B, S, d_c + d_r] (rows [latent || rope key]), out [B, S, H, d_c]."""
    B, S, H, d_c = q_latent.shape
    d_r = q_rope.shape[3]
    if q_rope.shape[:3] != (B, S, H) or kv.shape[:2] != (B, S) or kv.shape[2] != d_c + d_r:
        raise ValueError("q_rope must be [B, S, H, d_r] and kv [B, S, d_c + d_r]")
    if out.shape != (B, S, H, d_c):
        raise ValueError("out must be [B, S, H, d_c]")
    for t in (q_latent, q_rope, kv, out):
        if t.stride(-1) != 1:
            raise ValueError("last dimension must be contiguous")
    if lse is not None and (lse.shape != (B, S, H) or not lse.is_contiguous()
                            or lse.dtype != torch.float32):
        raise ValueError("lse must be contiguous float32 [B, S, H]")
    a = PrefillArgs()
    a.batch, a.heads, a.d_c, a.d_r, a.max_len = B, H, d_c, d_r, S
    a.dtype, a.scale = _dt(q_latent), float(scale)
    a.q_latent = q_latent.data_ptr()
    a.q_latent_stride_b, a.q_latent_stride_t, a.q_latent_stride_h = q_latent.stride()[:3]
    a.q_rope = q_rope.data_ptr()
    a.q_rope_stride_b, a.q_rope_stride_t, a.q_rope_stride_h = q_rope.stride()[:3]
    a.kv = kv.data_ptr()
    a.kv_stride_b, a.kv_stride_t = kv.stride()[:2]
    a.seq_lens = seq_lens.data_ptr()
    a.out, a.out_dtype = out.data_ptr(), _dt(out)
    a.out_stride_b, a.out_stride_t, a.out_stride_h = out.stride()[:3]
    a.lse = lse.data_ptr() if lse is not None else None
    return a


def mla_prefill(q_latent: torch.Tensor, q_rope: torch.Tensor, kv: torch.Tensor,
                seq_lens: torch.Tensor, scale: float, out: Optional[torch.Tensor] = None,
                lse: Optional[torch.Tensor] = None, out_dtype: torch.dtype = torch.float32):
    """MLA-form prefill of a batch of prompts.  Returns (out [B, S, H, d_c], lse or None);
    positions at or past seq_lens[b] are left as they were in `out`."""
    _gpu(q_latent, q_rope, kv, seq_lens, out, lse)
    B, S, H, d_c = q_latent.shape
    if seq_lens.dtype != torch.int32 or seq_lens.numel() != B:
        raise ValueError("seq_lens must be int32 [B]")
    if out is None:
        out = torch.empty((B, S, H, d_c), dtype=out_dtype, device=q_latent.device)
    args = make_prefill_args(q_latent, q_rope, kv, seq_lens, scale, out, lse)
    _check("tpla_mla_prefill", lib().tpla_mla_prefill(ctypes.byref(args), _stream(q_latent)))
    return out, lse


def combine_shards(partials: Sequence[torch.Tensor], out: Optional[torch.Tensor] = None,
                   out_dtype: Optional[torch.dtype] = None, accumulate: bool = False) -> torch.Tensor:
    """out[b, h, g*d_s:(g+1)*d_s] (+)= partials[g][b, h, :]."""
    _gpu(*partials, out)
    tp = len(partials)
    B, H, d_s = partials[0].shape
    for p in partials:
        if p.shape != (B, H, d_s) or not p.is_contiguous() or p.dtype != partials[0].dtype:
            raise ValueError("partials must be contiguous [batch, heads, d_s] of one dtype")
    if out is None:
        out = torch.empty((B, H, tp * d_s), dtype=out_dtype or partials[0].dtype,
                          device=partials[0].device)
    if out.shape != (B, H, tp * d_s) or not out.is_contiguous():
        raise ValueError("out must be contiguous [batch, heads, tp*d_s]")
    ptrs = (ctypes.c_void_p * tp)(*[p.data_ptr() for p in partials])
    _check("tpla_combine_shards",
           lib().tpla_combine_shards(ptrs, _dt(partials[0]), tp, B, H, d_s, out.data_ptr(),
                                     _dt(out), int(accumulate), _stream(out)))
    return out


def version() -> int:
    return int(lib().tpla_version())


def default_scale(d_s_full: int, d_r: int) -> float:
    return 1.0 / math.sqrt(d_s_full + d_r)
