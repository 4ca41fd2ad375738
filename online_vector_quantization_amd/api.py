"""Thin Python binding of libtq.so (ctypes).

Argument marshalling only: every step of encode and decode runs in the HIP
kernels behind the C ABI (include/tq.h).  PyTorch provides device memory and
streams.  If libtq.so has not been built, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libtq.so")

TQ_OK, TQ_ERR_INVALID_ARG, TQ_ERR_UNSUPPORTED, TQ_ERR_ALLOC, TQ_ERR_DEVICE = 0, -1, -2, -3, -4
TQ_F32, TQ_BF16 = 0, 1

EXPORTED = (
    "tq_codebook_build", "tq_codebook_build_split", "tq_codebook_split_info", "tq_codebook_export_wide",
    "tq_codebook_free", "tq_codebook_info", "tq_codebook_export",
    "tq_codebook_export_f64", "tq_record_words", "tq_encode_kv", "tq_decode_workspace_bytes",
    "tq_decode_attention", "tq_decode_attention_static", "tq_append_decode", "tq_attention_logits", "tq_chunk_attention",
    "tq_chunk_workspace_bytes", "tq_status_string", "tq_last_error",
)


class TQError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        super().__init__(f"{where}: status {status}: {msg}")
        self.status = status


class TqCache(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("signs", ctypes.c_void_p), ("norms", ctypes.c_void_p),
                ("res_norms", ctypes.c_void_p), ("t_cap", ctypes.c_int64)]


_lib = None


def load_library() -> ctypes.CDLL:
    """Load libtq.so (after torch, so both share one HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m online_vector_quantization_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, u64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float
    pi32 = ctypes.POINTER(ctypes.c_int32)
    lib.tq_codebook_build.argtypes = [i32, i32, i32, u64, u64, i32, ctypes.POINTER(vp)]
    lib.tq_codebook_build_split.argtypes = [i32, i32, i32, i32, u64, u64, i32, ctypes.POINTER(vp)]
    lib.tq_codebook_split_info.argtypes = [vp, pi32, pi32]
    lib.tq_codebook_export_wide.argtypes = [vp, vp, vp]
    lib.tq_codebook_free.argtypes = [vp]
    lib.tq_codebook_info.argtypes = [vp, pi32, pi32, pi32, pi32]
    lib.tq_codebook_export.argtypes = [vp, vp, vp, vp, vp]
    lib.tq_codebook_export_f64.argtypes = [vp, vp, vp, vp, vp]
    lib.tq_record_words.argtypes = [vp, pi32, pi32]
    lib.tq_encode_kv.argtypes = [vp, vp, i32, i64, i64, vp, i64, vp, vp, vp, vp, vp, vp, vp]
    lib.tq_decode_workspace_bytes.argtypes = [i32, i32, i32, i64, ctypes.POINTER(ctypes.c_size_t)]
    lib.tq_decode_attention.argtypes = [vp, vp, vp, i32, ctypes.POINTER(TqCache), ctypes.POINTER(TqCache), vp,
                                        i32, i32, i32, f32, vp, i32, vp, vp, ctypes.c_size_t, vp]
    lib.tq_decode_attention_static.argtypes = [vp, vp, vp, i32, ctypes.POINTER(TqCache), ctypes.POINTER(TqCache),
                                               vp, i32, i32, i32, f32, vp, i32, vp, vp]
    lib.tq_append_decode.argtypes = [vp, vp, vp, vp, i32, vp, i32, ctypes.POINTER(TqCache), ctypes.POINTER(TqCache),
                                     vp, i32, i32, i32, f32, vp, i32, vp, ctypes.c_size_t, vp]
    lib.tq_chunk_workspace_bytes.argtypes = [i32, i32, i32, i32, i64, ctypes.POINTER(ctypes.c_size_t)]
    lib.tq_chunk_attention.argtypes = [vp, vp, vp, i32, ctypes.POINTER(TqCache), ctypes.POINTER(TqCache), vp,
                                       i32, i32, i32, i32, f32, vp, i32, vp, ctypes.c_size_t, vp]
    lib.tq_attention_logits.argtypes = [vp, vp, i32, ctypes.POINTER(TqCache), vp, i32, i32, i32, f32, vp, vp,
                                        ctypes.c_size_t, vp]
    for name in EXPORTED:
        if name not in ("tq_status_string", "tq_last_error"):
            getattr(lib, name).restype = ctypes.c_int
    lib.tq_status_string.argtypes = [ctypes.c_int]
    lib.tq_status_string.restype = ctypes.c_char_p
    lib.tq_last_error.argtypes = []
    lib.tq_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int, where: str):
    if status != TQ_OK:
        lib = load_library()
        raise TQError(status, where, lib.tq_last_error().decode(errors="replace"))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream, device) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


class Codebook:
    """Setup tables of one quantizer: Lloyd-Max codebook, rotation, QJL matrix.

    device=-1 builds a host-only handle (export works, encode/decode do not).
    wide_coords > 0 builds split widths (tq_codebook_build_split): rotated
    coordinates 0 .. wide_coords - 1 on the (mse_bits + 1)-bit codebook.
    """

    def __init__(self, head_dim: int = 128, mse_bits: int = 2, qjl_dim: int = 0,
                 rot_seed: int = 0, qjl_seed: int = 1, device: int = 0, wide_coords: int = 0):
        lib = load_library()
        h = ctypes.c_void_p()
        if wide_coords:
            _check(lib.tq_codebook_build_split(head_dim, mse_bits, wide_coords, qjl_dim, rot_seed, qjl_seed, device,
                                               ctypes.byref(h)), "tq_codebook_build_split")
        else:
            _check(lib.tq_codebook_build(head_dim, mse_bits, qjl_dim, rot_seed, qjl_seed, device, ctypes.byref(h)),
                   "tq_codebook_build")
        self._h = h
        self.head_dim, self.mse_bits, self.qjl_dim, self.device = head_dim, mse_bits, qjl_dim, device
        self.wide_coords = wide_coords
        self.rot_seed, self.qjl_seed = rot_seed, qjl_seed
        cw, sw = ctypes.c_int32(), ctypes.c_int32()
        _check(lib.tq_record_words(h, ctypes.byref(cw), ctypes.byref(sw)), "tq_record_words")
        self.code_words, self.sign_words = cw.value, sw.value

    @property
    def handle(self):
        if self._h is None:
            raise ValueError("codebook was closed")
        return self._h

    @property
    def levels(self) -> int:
        return 1 << self.mse_bits

    def close(self):
        if getattr(self, "_h", None) is not None:
            load_library().tq_codebook_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def export(self, f64: bool = False) -> dict:
        d, m, L = self.head_dim, self.qjl_dim, self.levels
        dt = np.float64 if f64 else np.float32
        c, t = np.zeros(L, dt), np.zeros(L - 1, dt)
        rot = np.zeros((d, d), dt)
        qjl = np.zeros((m, d), dt) if m else None
        fn = load_library().tq_codebook_export_f64 if f64 else load_library().tq_codebook_export
        _check(fn(self.handle, c.ctypes.data, t.ctypes.data, rot.ctypes.data,
                  None if qjl is None else qjl.ctypes.data), "tq_codebook_export")
        return {"centroids": c, "thresholds": t, "rotation": rot, "qjl": qjl}

    def split_info(self) -> tuple:
        """(wide_coords, wide_bits) as the library reports them ((0, 0) when uniform)."""
        wc, wb = ctypes.c_int32(), ctypes.c_int32()
        _check(load_library().tq_codebook_split_info(self.handle, ctypes.byref(wc), ctypes.byref(wb)),
               "tq_codebook_split_info")
        return wc.value, wb.value

    def export_wide(self) -> dict:
        """The wide codebook's fp32 centroids and thresholds (split widths only)."""
        L = 1 << (self.mse_bits + 1)
        c, t = np.zeros(L, np.float32), np.zeros(L - 1, np.float32)
        _check(load_library().tq_codebook_export_wide(self.handle, c.ctypes.data, t.ctypes.data),
               "tq_codebook_export_wide")
        return {"centroids": c, "thresholds": t}


@dataclass
class CompressedCache:
    """Device tensors of one compressed cache: codes[B,H,T,W], signs, norms, res_norms."""
    codes: torch.Tensor
    norms: torch.Tensor
    signs: Optional[torch.Tensor] = None
    res_norms: Optional[torch.Tensor] = None

    @property
    def t_cap(self) -> int:
        return self.codes.shape[2]

    @staticmethod
    def allocate(cb: Codebook, batch: int, n_kv_heads: int, t_cap: int, device=None) -> "CompressedCache":
        device = device if device is not None else torch.device("cuda", cb.device)
        shape = (batch, n_kv_heads, t_cap)
        codes = torch.zeros(*shape, cb.code_words, dtype=torch.int32, device=device)
        norms = torch.zeros(*shape, dtype=torch.float32, device=device)
        signs = res = None
        if cb.qjl_dim:
            signs = torch.zeros(*shape, cb.sign_words, dtype=torch.int32, device=device)
            res = torch.zeros(*shape, dtype=torch.float32, device=device)
        return CompressedCache(codes, norms, signs, res)

    def as_struct(self) -> TqCache:
        return TqCache(self.codes.data_ptr(), None if self.signs is None else self.signs.data_ptr(),
                       self.norms.data_ptr(), None if self.res_norms is None else self.res_norms.data_ptr(),
                       self.t_cap)

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.codes, self.norms, self.signs, self.res_norms)
                   if t is not None)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return TQ_F32
    if t.dtype == torch.bfloat16:
        return TQ_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _require_cuda(*tensors):
    for t in tensors:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must be on a GPU device")


def encode_kv(cb: Codebook, x: torch.Tensor, codes: torch.Tensor, norms: torch.Tensor,
              signs: Optional[torch.Tensor] = None, res_norms: Optional[torch.Tensor] = None,
              dst_row: Optional[torch.Tensor] = None, dbg_rot: Optional[torch.Tensor] = None,
              dbg_proj: Optional[torch.Tensor] = None, stream=None) -> None:
    """tq_encode_kv: x[n, d] rows (last dim contiguous) into cache rows.

    codes/signs/norms/res_norms are the cache arrays (any leading shape; rows are
    flattened); dst_row (int64[n]) maps input row i to a cache row (None: i).
    """
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D [n, d] with a contiguous last dimension")
    _require_cuda(x, codes, norms, signs, res_norms, dst_row, dbg_rot, dbg_proj)
    for t in (codes, norms, signs, res_norms, dbg_rot, dbg_proj):
        if t is not None and not t.is_contiguous():
            raise ValueError("output tensors must be contiguous")
    if dst_row is not None and (dst_row.dtype != torch.int64 or not dst_row.is_contiguous() or dst_row.numel() != x.shape[0]):
        raise ValueError("dst_row must be a contiguous int64 tensor with n entries")
    cache_rows = norms.numel()
    lib = load_library()
    _check(lib.tq_encode_kv(cb.handle, _ptr(x), _dtype_code(x), x.shape[0], x.stride(0), _ptr(dst_row), cache_rows,
                            _ptr(codes), _ptr(signs), _ptr(norms), _ptr(res_norms), _ptr(dbg_rot), _ptr(dbg_proj),
                            _stream_handle(stream, x.device)), "tq_encode_kv")


def encode_into_cache(cb: Codebook, x: torch.Tensor, cache: CompressedCache, dst_row=None,
                      dbg_rot=None, dbg_proj=None, stream=None) -> None:
    """encode_kv into the arrays of a CompressedCache."""
    encode_kv(cb, x, cache.codes, cache.norms, cache.signs, cache.res_norms, dst_row, dbg_rot, dbg_proj, stream)


def decode_workspace_bytes(batch: int, n_q_heads: int, n_kv_heads: int, t_cap: int) -> int:
    out = ctypes.c_size_t()
    _check(load_library().tq_decode_workspace_bytes(batch, n_q_heads, n_kv_heads, t_cap, ctypes.byref(out)),
           "tq_decode_workspace_bytes")
    return out.value


def alloc_workspace(batch: int, n_q_heads: int, n_kv_heads: int, t_cap: int, device) -> torch.Tensor:
    """Device scratch for tq_decode_attention."""
    n = decode_workspace_bytes(batch, n_q_heads, n_kv_heads, t_cap)
    return torch.empty(n, dtype=torch.uint8, device=device)


def chunk_workspace_bytes(batch: int, n_q_heads: int, n_kv_heads: int, n_new: int, t_cap: int) -> int:
    out = ctypes.c_size_t()
    _check(load_library().tq_chunk_workspace_bytes(batch, n_q_heads, n_kv_heads, n_new, t_cap, ctypes.byref(out)),
           "tq_chunk_workspace_bytes")
    return out.value


def alloc_chunk_workspace(batch: int, n_q_heads: int, n_kv_heads: int, n_new: int, t_cap: int, device):
    """Device scratch for tq_chunk_attention."""
    return torch.empty(chunk_workspace_bytes(batch, n_q_heads, n_kv_heads, n_new, t_cap), dtype=torch.uint8,
                       device=device)


def decode_attention(kcb: Codebook, vcb: Codebook, q: torch.Tensor, kcache: CompressedCache,
                     vcache: CompressedCache, seq_len: torch.Tensor, out: Optional[torch.Tensor] = None,
                     softmax_scale: float = 0.0, out_dtype=torch.float32,
                     dbg_scores: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
    """tq_decode_attention: q[B, Hq, d] against the compressed caches -> out[B, Hq, d]."""
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B, Hq, d] tensor")
    B, Hq, d = q.shape
    Hkv = kcache.codes.shape[1]
    if seq_len.dtype != torch.int32 or seq_len.numel() != B or not seq_len.is_contiguous():
        raise ValueError("seq_len must be a contiguous int32 tensor with B entries")
    if out is None:
        out = torch.empty(B, Hq, d, dtype=out_dtype, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(B, Hq, Hkv, kcache.t_cap, q.device)
    _require_cuda(q, seq_len, out, dbg_scores, workspace, kcache.codes, vcache.codes)
    ks, vs = kcache.as_struct(), vcache.as_struct()
    _check(load_library().tq_decode_attention(
        kcb.handle, vcb.handle, _ptr(q), _dtype_code(q), ctypes.byref(ks), ctypes.byref(vs), _ptr(seq_len),
        B, Hq, Hkv, float(softmax_scale), _ptr(out), _dtype_code(out), _ptr(dbg_scores), _ptr(workspace),
        workspace.numel(), _stream_handle(stream, q.device)), "tq_decode_attention")
    return out


def decode_attention_static(kcb: Codebook, vcb: Codebook, q: torch.Tensor, kcache: CompressedCache,
                            vcache: CompressedCache, seq_len: torch.Tensor, out: Optional[torch.Tensor] = None,
                            softmax_scale: float = 0.0, out_dtype=torch.float32,
                            dbg_scores: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """tq_decode_attention_static: decode_attention with the library's static scratch (no workspace)."""
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B, Hq, d] tensor")
    B, Hq, d = q.shape
    Hkv = kcache.codes.shape[1]
    if seq_len.dtype != torch.int32 or seq_len.numel() != B or not seq_len.is_contiguous():
        raise ValueError("seq_len must be a contiguous int32 tensor with B entries")
    if out is None:
        out = torch.empty(B, Hq, d, dtype=out_dtype, device=q.device)
    _require_cuda(q, seq_len, out, dbg_scores, kcache.codes, vcache.codes)
    ks, vs = kcache.as_struct(), vcache.as_struct()
    _check(load_library().tq_decode_attention_static(
        kcb.handle, vcb.handle, _ptr(q), _dtype_code(q), ctypes.byref(ks), ctypes.byref(vs), _ptr(seq_len),
        B, Hq, Hkv, float(softmax_scale), _ptr(out), _dtype_code(out), _ptr(dbg_scores),
        _stream_handle(stream, q.device)), "tq_decode_attention_static")
    return out


def chunk_attention(kcb: Codebook, vcb: Codebook, q: torch.Tensor, kcache: CompressedCache,
                    vcache: CompressedCache, seq_len: torch.Tensor, out: Optional[torch.Tensor] = None,
                    softmax_scale: float = 0.0, out_dtype=torch.float32, workspace: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """tq_chunk_attention: q [B, Hq, n_new, d], query j at position seq_len[b] - n_new + j attending
    causally over the compressed caches -> out [B, Hq, n_new, d]."""
    if q.dim() != 4 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B, Hq, n_new, d] tensor")
    B, Hq, n_new, d = q.shape
    Hkv = kcache.codes.shape[1]
    if seq_len.dtype != torch.int32 or seq_len.numel() != B or not seq_len.is_contiguous():
        raise ValueError("seq_len must be a contiguous int32 tensor with B entries")
    if out is None:
        out = torch.empty(B, Hq, n_new, d, dtype=out_dtype, device=q.device)
    if workspace is None:
        workspace = alloc_chunk_workspace(B, Hq, Hkv, n_new, kcache.t_cap, q.device)
    _require_cuda(q, seq_len, out, workspace, kcache.codes, vcache.codes)
    ks, vs = kcache.as_struct(), vcache.as_struct()
    _check(load_library().tq_chunk_attention(
        kcb.handle, vcb.handle, _ptr(q), _dtype_code(q), ctypes.byref(ks), ctypes.byref(vs), _ptr(seq_len),
        B, Hq, Hkv, n_new, float(softmax_scale), _ptr(out), _dtype_code(out), _ptr(workspace), workspace.numel(),
        _stream_handle(stream, q.device)), "tq_chunk_attention")
    return out


def append_decode(kcb: Codebook, vcb: Codebook, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                  kcache: CompressedCache, vcache: CompressedCache, seq_len: torch.Tensor,
                  out: Optional[torch.Tensor] = None, softmax_scale: float = 0.0, out_dtype=torch.float32,
                  workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """tq_append_decode: append k_new/v_new [B, Hkv, d] at position seq_len[b], attend q [B, Hq, d]
    over the grown caches, advance seq_len on the device.  No host synchronization."""
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B, Hq, d] tensor")
    B, Hq, d = q.shape
    Hkv = kcache.codes.shape[1]
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if t.shape != (B, Hkv, d) or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [B, Hkv, d] tensor")
    if k_new.dtype != v_new.dtype:
        raise ValueError("k_new and v_new must share a dtype")
    if seq_len.dtype != torch.int32 or seq_len.numel() != B or not seq_len.is_contiguous():
        raise ValueError("seq_len must be a contiguous int32 tensor with B entries")
    if out is None:
        out = torch.empty(B, Hq, d, dtype=out_dtype, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(B, Hq, Hkv, kcache.t_cap, q.device)
    _require_cuda(q, k_new, v_new, seq_len, out, workspace, kcache.codes, vcache.codes)
    ks, vs = kcache.as_struct(), vcache.as_struct()
    _check(load_library().tq_append_decode(
        kcb.handle, vcb.handle, _ptr(k_new), _ptr(v_new), _dtype_code(k_new), _ptr(q), _dtype_code(q),
        ctypes.byref(ks), ctypes.byref(vs), _ptr(seq_len), B, Hq, Hkv, float(softmax_scale), _ptr(out),
        _dtype_code(out), _ptr(workspace), workspace.numel(), _stream_handle(stream, q.device)), "tq_append_decode")
    return out


def attention_logits(kcb: Codebook, q: torch.Tensor, kcache: CompressedCache, seq_len: torch.Tensor,
                     logits: Optional[torch.Tensor] = None, softmax_scale: float = 0.0,
                     workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """tq_attention_logits: the scaled logits of q [B, Hq, d] against every cached key ->
    logits float32 [B, Hq, t_cap]; entries t >= seq_len[b] are not written (a new
    logits tensor starts at -inf)."""
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B, Hq, d] tensor")
    B, Hq, d = q.shape
    Hkv = kcache.codes.shape[1]
    if seq_len.dtype != torch.int32 or seq_len.numel() != B or not seq_len.is_contiguous():
        raise ValueError("seq_len must be a contiguous int32 tensor with B entries")
    if logits is None:
        logits = torch.full((B, Hq, kcache.t_cap), float("-inf"), dtype=torch.float32, device=q.device)
    if logits.dtype != torch.float32 or tuple(logits.shape) != (B, Hq, kcache.t_cap) or not logits.is_contiguous():
        raise ValueError("logits must be a contiguous float32 [B, Hq, t_cap] tensor")
    if workspace is None:
        workspace = alloc_workspace(B, Hq, Hkv, kcache.t_cap, q.device)
    _require_cuda(q, seq_len, logits, workspace, kcache.codes)
    ks = kcache.as_struct()
    _check(load_library().tq_attention_logits(
        kcb.handle, _ptr(q), _dtype_code(q), ctypes.byref(ks), _ptr(seq_len), B, Hq, Hkv, float(softmax_scale),
        _ptr(logits), _ptr(workspace), workspace.numel(), _stream_handle(stream, q.device)), "tq_attention_logits")
    return logits


def compressed_bytes_per_token(kcb: Codebook, vcb: Codebook) -> int:
    """Bytes of one (token, kv head) record pair: K codes + signs + nu + gamma, V codes + nu."""
    k = 4 * kcb.code_words + 4 * kcb.sign_words + 4 + (4 if kcb.qjl_dim else 0)
    v = 4 * vcb.code_words + 4
    return k + v


def chunk_uses_mfma(g: int, n_new: int) -> bool:
    """Whether tq_chunk_attention takes its matrix-core kernel (16 or more query rows per kv head)."""
    return g * n_new >= 16
