"""MI355X (gfx950) compressed sparse attention: thin Python binding of libcsa.so.

Every step of the path (compress_insert, index_topk, attend, inv_rope, rope_table) runs in the
HIP kernels of libcsa.so; this module only marshals torch tensors (device memory) and the current
torch stream into the C ABI declared in include/csa.h. There is no fallback: if the library is not
built, or a call returns an error status, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcsa.so")

F32, BF16, FP8, FP4 = 0, 1, 2, 3
SCORE_DOT, SCORE_WRELU = 0, 1
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported configuration", 3: "workspace missing or too small",
          4: "HIP launch failed", 5: "request exceeds the fixed scratch of a no-allocation entry point"}
NOALLOC_SCRATCH_BYTES = 64 << 20  # CSA_NOALLOC_SCRATCH_BYTES


class CsaError(RuntimeError):
    def __init__(self, fn: str, status: int, hip_err: int = 0):
        msg = f"{fn}: {STATUS.get(status, status)}"
        if status == 4:
            msg += f" (hipError {hip_err})"
        super().__init__(msg)
        self.status = status


class CacheDesc(ctypes.Structure):
    _fields_ = [("ratio", ctypes.c_int32), ("window", ctypes.c_int32), ("dim", ctypes.c_int32),
                ("rope_dims", ctypes.c_int32), ("dtype", ctypes.c_int32), ("pages", ctypes.c_void_p),
                ("scales", ctypes.c_void_p), ("block_table", ctypes.c_void_p), ("batch", ctypes.c_int32),
                ("bt_stride", ctypes.c_int32), ("n_phys", ctypes.c_int32)]


class RawDesc(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("dim", ctypes.c_int32), ("roles", ctypes.c_int32),
                ("kv_pages", ctypes.c_void_p), ("logit_pages", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("batch", ctypes.c_int32), ("bt_stride", ctypes.c_int32),
                ("n_phys", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libcsa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m long_context_compressed_compress_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, F, D, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double, ctypes.c_size_t
        CP, RP = ctypes.POINTER(CacheDesc), ctypes.POINTER(RawDesc)
        sig = {
            "csa_compress_insert": (I32, [CP, RP, I32, P, P, I32, I32, P, P, P, F, P, I32, P, I32, P, P]),
            "csa_compress_insert_pair": (I32, [CP, RP, P, P, P, P, I32, CP, RP, P, P, P, P, I32, I32, P, P, I32, I32, F,
                                               P]),
            "csa_compress_index_score": (I32, [CP, RP, P, P, P, P, I32, CP, RP, P, P, P, P, I32, I32, P, P, I32, I32, F,
                                               I32, P, P, I64, P, I32, I32, P, I32, I32, P, SZ, P]),
            "csa_index_topk_workspace": (SZ, [I32, I64, I32, I32]),
            "csa_index_topk": (I32, [CP, I32, P, P, I64, P, I32, I32, P, I32, I32, P, P, P, P, SZ, P]),
            "csa_index_workspace_clear": (I32, [P, SZ, I32, P]),
            "csa_index_topk_noalloc": (I32, [CP, I32, P, P, I64, P, I32, I32, P, I32, I32, P, P, P, P]),
            "csa_index_score": (I32, [CP, I32, P, P, I64, P, I32, I32, P, I32, I32, P, SZ, P]),
            "csa_index_select": (I32, [CP, I32, P, P, I64, I32, P, P, P, P, SZ, P]),
            "csa_attend_workspace": (SZ, [I32, I32, I32, I32]),
            "csa_attend": (I32, [CP, RP, I32, I32, P, P, P, I32, I32, P, I32, I64, F, I32, P, I32, P, P, P, SZ, P]),
            "csa_inv_rope": (I32, [I32, I32, I32, I32, P, P, I32, P, P]),
            "csa_rope_table": (I32, [I32, I32, D, P, P]),
            "csa_inv_rope_quant_fp8": (I32, [I32, I32, I32, I32, P, P, I32, P, I32, P, P, P]),
            "csa_attend_quant_fp8": (I32, [CP, RP, I32, I32, P, P, P, I32, I32, P, I32, I64, F, P, I32, I32, P, P, P, P,
                                           SZ, P]),
            "csa_prepare_qk": (I32, [I32, I32, P, P, P, I32, P, F, P, RP, I32, P, I32, P, P]),
            "csa_num_entries": (I64, [I64, I32, I32]),
            "csa_num_eligible": (I64, [I64, I32, I32]),
            "csa_entry_slot": (I64, [P, I64, I32]),
            "csa_raw_slot": (I64, [P, I64]),
            "csa_status_string": (ctypes.c_char_p, [I32]),
            "csa_last_hip_error": (I32, []),
            "csa_version": (I32, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise CsaError(fn, status, lib().csa_last_hip_error())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


_DT = {torch.float32: F32, torch.bfloat16: BF16, torch.int16: BF16, torch.uint16: BF16, torch.uint8: FP8,
       torch.float8_e4m3fn: FP8, torch.float4_e2m1fn_x2: FP4}


def dtype_code(t: torch.Tensor) -> int:
    return _DT[t.dtype]


# ------------------------------------------------------------------ descriptors
@dataclass
class Cache:
    """A compressed cache: pages [n_phys*256/ratio][dim], optional fp8 scales, block table [batch][bt_stride].

    An MXFP4 cache holds pages as torch.float4_e2m1fn_x2 [rows][dim/2] (two codes per byte) and scales as
    uint8 [rows][dim/32] E8M0 block exponents."""
    ratio: int
    window: int
    dim: int
    rope_dims: int
    pages: torch.Tensor
    block_table: torch.Tensor
    scales: Optional[torch.Tensor] = None

    @property
    def dtype(self) -> int:
        return dtype_code(self.pages)

    def desc(self) -> CacheDesc:
        per = 256 // self.ratio if self.ratio in (4, 128) else 1
        return CacheDesc(self.ratio, self.window, self.dim, self.rope_dims, self.dtype, _ptr(self.pages),
                         _ptr(self.scales), _ptr(self.block_table), self.block_table.shape[0],
                         self.block_table.shape[1], self.pages.shape[0] // per)


@dataclass
class Raw:
    """Raw per-position pages: compressor state (roles = window/ratio, with logits) or window K=V rows (roles = 0)."""
    dim: int
    roles: int
    kv_pages: torch.Tensor
    block_table: torch.Tensor
    logit_pages: Optional[torch.Tensor] = None
    scales: Optional[torch.Tensor] = None

    def desc(self) -> RawDesc:
        return RawDesc(dtype_code(self.kv_pages), self.dim, self.roles, _ptr(self.kv_pages), _ptr(self.logit_pages),
                       _ptr(self.scales), _ptr(self.block_table), self.block_table.shape[0],
                       self.block_table.shape[1], self.kv_pages.shape[0] // 256)


# ------------------------------------------------------------------ calls
def compress_insert(cache: Cache, state: Raw, start_pos: torch.Tensor, cu_new: torch.Tensor, kv_new: torch.Tensor,
                    logit_new: torch.Tensor, gamma: torch.Tensor, rms_eps: float, rope_cs: torch.Tensor,
                    max_new_per_seq: int, out_slots: Optional[torch.Tensor] = None,
                    out_new_entries: Optional[torch.Tensor] = None, stream=None) -> None:
    cd, sd = cache.desc(), state.desc()
    batch = start_pos.shape[0]
    _check("csa_compress_insert", lib().csa_compress_insert(
        ctypes.byref(cd), ctypes.byref(sd), batch, _ptr(start_pos), _ptr(cu_new), kv_new.shape[0], max_new_per_seq,
        _ptr(kv_new), _ptr(logit_new), _ptr(gamma), rms_eps, _ptr(rope_cs), rope_cs.shape[0],
        _ptr(out_slots), 0 if out_slots is None else out_slots.shape[1], _ptr(out_new_entries), _stream(stream)))


def compress_insert_pair(cache_a: Cache, state_a: Raw, kv_a: torch.Tensor, logit_a: torch.Tensor,
                         gamma_a: torch.Tensor, rope_a: torch.Tensor, cache_b: Cache, state_b: Raw,
                         kv_b: torch.Tensor, logit_b: torch.Tensor, gamma_b: torch.Tensor, rope_b: torch.Tensor,
                         start_pos: torch.Tensor, cu_new: torch.Tensor, rms_eps: float, max_new_per_seq: int,
                         stream=None) -> None:
    """compress_insert of two caches taking the same new tokens (main + indexer of a c4a layer) in one call."""
    ca, sa, cb, sb = cache_a.desc(), state_a.desc(), cache_b.desc(), state_b.desc()
    _check("csa_compress_insert_pair", lib().csa_compress_insert_pair(
        ctypes.byref(ca), ctypes.byref(sa), _ptr(kv_a), _ptr(logit_a), _ptr(gamma_a), _ptr(rope_a), rope_a.shape[0],
        ctypes.byref(cb), ctypes.byref(sb), _ptr(kv_b), _ptr(logit_b), _ptr(gamma_b), _ptr(rope_b), rope_b.shape[0],
        start_pos.shape[0], _ptr(start_pos), _ptr(cu_new), kv_a.shape[0], max_new_per_seq, rms_eps, _stream(stream)))


def compress_index_score(cache_a: Cache, state_a: Raw, kv_a: torch.Tensor, logit_a: torch.Tensor,
                         gamma_a: torch.Tensor, rope_a: torch.Tensor, cache_b: Cache, state_b: Raw,
                         kv_b: torch.Tensor, logit_b: torch.Tensor, gamma_b: torch.Tensor, rope_b: torch.Tensor,
                         start_pos: torch.Tensor, cu_new: torch.Tensor, rms_eps: float, q_seq: torch.Tensor,
                         q_pos: torch.Tensor, max_elig: int, q_idx: torch.Tensor, head_w: Optional[torch.Tensor],
                         mode: int, k: int, workspace: torch.Tensor, stream=None) -> None:
    """A decode step's compress_insert_pair (main cache a, indexer cache b; one new token per sequence) followed by
    index_score over cache b for query q = sequence q's token, in one launch where the configuration allows."""
    ca, sa, cb, sb = cache_a.desc(), state_a.desc(), cache_b.desc(), state_b.desc()
    n_q, n_heads = q_idx.shape[0], q_idx.shape[1]
    _check("csa_compress_index_score", lib().csa_compress_index_score(
        ctypes.byref(ca), ctypes.byref(sa), _ptr(kv_a), _ptr(logit_a), _ptr(gamma_a), _ptr(rope_a), rope_a.shape[0],
        ctypes.byref(cb), ctypes.byref(sb), _ptr(kv_b), _ptr(logit_b), _ptr(gamma_b), _ptr(rope_b), rope_b.shape[0],
        start_pos.shape[0], _ptr(start_pos), _ptr(cu_new), kv_a.shape[0], 1, rms_eps, n_q, _ptr(q_seq), _ptr(q_pos),
        max_elig, _ptr(q_idx), dtype_code(q_idx), n_heads, _ptr(head_w), mode, k, _ptr(workspace), workspace.numel(),
        _stream(stream)))


def index_topk_workspace(n_q: int, max_elig: int, k: int, n_heads: int) -> int:
    return int(lib().csa_index_topk_workspace(n_q, max_elig, k, n_heads))


def index_workspace(n_q: int, max_elig: int, k: int, n_heads: int = 1, device="cuda") -> torch.Tensor:
    """A zero-filled index workspace (the select pass keeps its histogram region zeroed afterwards)."""
    return torch.zeros(index_topk_workspace(n_q, max_elig, k, n_heads), dtype=torch.uint8, device=device)


def index_workspace_clear(workspace: torch.Tensor, n_q: int, stream=None) -> None:
    _check("csa_index_workspace_clear", lib().csa_index_workspace_clear(
        _ptr(workspace), workspace.numel(), n_q, _stream(stream)))


def index_topk(cache: Cache, q_seq: torch.Tensor, q_pos: torch.Tensor, max_elig: int, q_idx: torch.Tensor,
               head_w: Optional[torch.Tensor], mode: int, k: int, out_idx: torch.Tensor,
               out_count: Optional[torch.Tensor] = None, out_scores: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    n_q, n_heads = q_idx.shape[0], q_idx.shape[1]
    if workspace is None:
        workspace = index_workspace(n_q, max_elig, k, n_heads, q_idx.device)
    cd = cache.desc()
    _check("csa_index_topk", lib().csa_index_topk(
        ctypes.byref(cd), n_q, _ptr(q_seq), _ptr(q_pos), max_elig, _ptr(q_idx), dtype_code(q_idx), n_heads,
        _ptr(head_w), mode, k, _ptr(out_idx), _ptr(out_count), _ptr(out_scores), _ptr(workspace),
        workspace.numel(), _stream(stream)))


def index_topk_noalloc(cache: Cache, q_seq: torch.Tensor, q_pos: torch.Tensor, max_elig: int, q_idx: torch.Tensor,
                       head_w: Optional[torch.Tensor], mode: int, k: int, out_idx: torch.Tensor,
                       out_count: Optional[torch.Tensor] = None, out_scores: Optional[torch.Tensor] = None,
                       stream=None) -> None:
    """csa_index_topk_noalloc: index_topk on the library's fixed per-GPU scratch; allocates nothing (the caller
    passes inputs and outputs)."""
    n_q, n_heads = q_idx.shape[0], q_idx.shape[1]
    cd = cache.desc()
    _check("csa_index_topk_noalloc", lib().csa_index_topk_noalloc(
        ctypes.byref(cd), n_q, _ptr(q_seq), _ptr(q_pos), max_elig, _ptr(q_idx), dtype_code(q_idx), n_heads,
        _ptr(head_w), mode, k, _ptr(out_idx), _ptr(out_count), _ptr(out_scores), _stream(stream)))


def index_score(cache: Cache, q_seq: torch.Tensor, q_pos: torch.Tensor, max_elig: int, q_idx: torch.Tensor,
                head_w: Optional[torch.Tensor], mode: int, k: int, workspace: torch.Tensor, stream=None) -> None:
    n_q, n_heads = q_idx.shape[0], q_idx.shape[1]
    cd = cache.desc()
    _check("csa_index_score", lib().csa_index_score(
        ctypes.byref(cd), n_q, _ptr(q_seq), _ptr(q_pos), max_elig, _ptr(q_idx), dtype_code(q_idx), n_heads,
        _ptr(head_w), mode, k, _ptr(workspace), workspace.numel(), _stream(stream)))


def index_select(cache: Cache, q_seq: torch.Tensor, q_pos: torch.Tensor, max_elig: int, k: int,
                 out_idx: torch.Tensor, workspace: torch.Tensor, out_count: Optional[torch.Tensor] = None,
                 out_scores: Optional[torch.Tensor] = None, stream=None) -> None:
    cd = cache.desc()
    _check("csa_index_select", lib().csa_index_select(
        ctypes.byref(cd), q_seq.shape[0], _ptr(q_seq), _ptr(q_pos), max_elig, k, _ptr(out_idx), _ptr(out_count),
        _ptr(out_scores), _ptr(workspace), workspace.numel(), _stream(stream)))


def attend(cache: Cache, swa: Raw, swa_window: int, q_seq: torch.Tensor, q_pos: torch.Tensor, q: torch.Tensor,
           topk_idx: Optional[torch.Tensor], max_elig: int, softmax_scale: float, fuse_inv_rope: bool,
           rope_cs: torch.Tensor, out: torch.Tensor, out_lse: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    n_q, n_heads = q.shape[0], q.shape[1]
    cd, sd = cache.desc(), swa.desc()
    k = 0 if topk_idx is None else topk_idx.shape[1]
    if workspace is None:
        need = attend_workspace(n_q, n_heads, q.shape[2], (k if topk_idx is not None else max_elig) + swa_window)
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device) if need else None
    _check("csa_attend", lib().csa_attend(
        ctypes.byref(cd), ctypes.byref(sd), swa_window, n_q, _ptr(q_seq), _ptr(q_pos), _ptr(q), dtype_code(q),
        n_heads, _ptr(topk_idx), k, max_elig, softmax_scale, int(fuse_inv_rope), _ptr(rope_cs), rope_cs.shape[0],
        _ptr(out), _ptr(out_lse), _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream(stream)))


def attend_quant_fp8(cache: Cache, swa: Raw, swa_window: int, q_seq: torch.Tensor, q_pos: torch.Tensor,
                     q: torch.Tensor, topk_idx: Optional[torch.Tensor], max_elig: int, softmax_scale: float,
                     rope_cs: torch.Tensor, group: int, out_codes: torch.Tensor, out_scales: torch.Tensor,
                     out_lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                     stream=None) -> None:
    """csa_attend_quant_fp8: attention with the inverse RoPE + grouped fp8 output epilogue fused in."""
    n_q, n_heads = q.shape[0], q.shape[1]
    cd, sd = cache.desc(), swa.desc()
    k = 0 if topk_idx is None else topk_idx.shape[1]
    if workspace is None:
        need = attend_workspace(n_q, n_heads, q.shape[2], (k if topk_idx is not None else max_elig) + swa_window)
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device) if need else None
    _check("csa_attend_quant_fp8", lib().csa_attend_quant_fp8(
        ctypes.byref(cd), ctypes.byref(sd), swa_window, n_q, _ptr(q_seq), _ptr(q_pos), _ptr(q), dtype_code(q),
        n_heads, _ptr(topk_idx), k, max_elig, softmax_scale, _ptr(rope_cs), rope_cs.shape[0], group, _ptr(out_codes),
        _ptr(out_scales), _ptr(out_lse), _ptr(workspace), 0 if workspace is None else workspace.numel(),
        _stream(stream)))


def attend_workspace(n_q: int, n_heads: int, dim: int, max_keys: int) -> int:
    return int(lib().csa_attend_workspace(n_q, n_heads, dim, max_keys))


def inv_rope(io: torch.Tensor, q_pos: torch.Tensor, rope_dims: int, rope_cs: torch.Tensor, stream=None) -> None:
    n_q, n_heads, dim = io.shape
    _check("csa_inv_rope", lib().csa_inv_rope(n_q, n_heads, dim, rope_dims, _ptr(q_pos), _ptr(rope_cs),
                                              rope_cs.shape[0], _ptr(io), _stream(stream)))


def prepare_qk(q: torch.Tensor, kv: torch.Tensor, tok_seq: torch.Tensor, tok_pos: torch.Tensor, q_gamma: torch.Tensor,
               rms_eps: float, swa: Raw, rope_dims: int, rope_cs: torch.Tensor, q_out: Optional[torch.Tensor] = None,
               stream=None) -> torch.Tensor:
    """Query norm + RoPE into q_out (same shape and dtype as q [n][H][D]); the window key of every token (kv [n][D],
    RoPE'd at its position) is written into swa's pages. Returns q_out."""
    n_tok, n_heads, _ = q.shape
    if q_out is None:
        q_out = torch.empty_like(q)
    sd = swa.desc()
    _check("csa_prepare_qk", lib().csa_prepare_qk(
        n_tok, n_heads, _ptr(tok_seq), _ptr(tok_pos), _ptr(q), dtype_code(q), _ptr(q_gamma), rms_eps, _ptr(kv),
        ctypes.byref(sd), rope_dims, _ptr(rope_cs), rope_cs.shape[0], _ptr(q_out), _stream(stream)))
    return q_out


def inv_rope_quant_fp8(x: torch.Tensor, q_pos: torch.Tensor, rope_dims: int, rope_cs: torch.Tensor, group: int,
                       out_codes: Optional[torch.Tensor] = None, out_scales: Optional[torch.Tensor] = None,
                       stream=None):
    """Inverse RoPE + fp8 quantisation of an attention output x [n_q][H][D] fp32 (not inverse-rotated yet).
    Returns (codes uint8 [n_q][H][D], scales fp32 [n_q][H][D // group])."""
    n_q, n_heads, dim = x.shape
    if out_codes is None:
        out_codes = torch.empty((n_q, n_heads, dim), dtype=torch.uint8, device=x.device)
    if out_scales is None:
        out_scales = torch.empty((n_q, n_heads, dim // group), dtype=torch.float32, device=x.device)
    _check("csa_inv_rope_quant_fp8", lib().csa_inv_rope_quant_fp8(
        n_q, n_heads, dim, rope_dims, _ptr(q_pos), _ptr(rope_cs), rope_cs.shape[0], _ptr(x), group,
        _ptr(out_codes), _ptr(out_scales), _stream(stream)))
    return out_codes, out_scales


def rope_table(rows: int, rope_dims: int, theta: float = 10000.0, device="cuda", stream=None) -> torch.Tensor:
    out = torch.empty((rows, rope_dims // 2, 2), dtype=torch.float32, device=device)
    _check("csa_rope_table", lib().csa_rope_table(rows, rope_dims, theta, _ptr(out), _stream(stream)))
    return out


def num_entries(n_raw: int, ratio: int, window: int) -> int:
    return int(lib().csa_num_entries(n_raw, ratio, window))


def num_eligible(q_pos: int, ratio: int, window: int) -> int:
    return int(lib().csa_num_eligible(q_pos, ratio, window))
