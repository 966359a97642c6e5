"""ctypes binding of the C ABI in include/tpla.h (argument marshalling only).

Every function takes torch tensors that already live on the GPU, passes their
device pointers and the current HIP stream to the library, and raises
``TplaError`` on a non-OK status.  Nothing is computed here; when the shared
library has not been built the first call raises instead of falling back to
anything else.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

from .build import LIB_PATH

TPLA_OK = 0
STATUS_NAMES = {0: "TPLA_OK", 1: "TPLA_ERR_INVALID_ARGUMENT", 2: "TPLA_ERR_UNSUPPORTED",
                3: "TPLA_ERR_WORKSPACE_TOO_SMALL", 4: "TPLA_ERR_HIP"}
DTYPES = {"f32": 0, "bf16": 1}
TRANSFORMS = {"identity": 0, "wht": 1}
KERNELS = {"auto": 0, "generic": 1, "mfma": 2}
SCHEDULES = {"auto": 0, "chunked": 1, "balanced": 2}

EXPORTED = ["tpla_abi_version", "tpla_status_string", "tpla_last_error", "tpla_workspace_size",
            "latent_cache_append", "tpla_decode_sharded", "tpla_decode_sharded_ex", "mla_decode_absorbed",
            "tpla_value_up_projection", "tpla_merge_context_parts", "latent_cache_append_normed",
            "mla_prefill_workspace_size", "mla_prefill_absorbed", "mla_prefill_absorbed_ex",
            "tpla_decode_sharded_noalloc", "tpla_decode_sharded_projected"]


class TplaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class CacheDesc(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("d_latent", ctypes.c_int32), ("d_rope", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("max_pages_per_seq", ctypes.c_int32), ("transform", ctypes.c_int32)]


class DecodeOpts(ctypes.Structure):
    _fields_ = [("chunk_tokens", ctypes.c_int32), ("kernel", ctypes.c_int32),
                ("decode_begin", ctypes.c_void_p), ("decode_end", ctypes.c_void_p), ("schedule", ctypes.c_int32)]


@dataclass(frozen=True)
class Desc:
    """Python view of tpla_cache_desc_t."""

    dtype: str
    d_latent: int
    d_rope: int
    page_size: int
    num_pages: int
    max_pages_per_seq: int = 0
    transform: str = "identity"

    def c(self) -> CacheDesc:
        return CacheDesc(DTYPES[self.dtype], self.d_latent, self.d_rope, self.page_size, self.num_pages,
                         self.max_pages_per_seq, TRANSFORMS[self.transform])


_LIB = None
_P = ctypes.c_void_p
_I32 = ctypes.c_int32


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load (once) the built shared library; raises if it is missing."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library {path} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    lib.tpla_abi_version.restype = _I32
    lib.tpla_status_string.restype = ctypes.c_char_p
    lib.tpla_status_string.argtypes = [_I32]
    lib.tpla_last_error.restype = ctypes.c_char_p
    lib.tpla_workspace_size.restype = _I32
    lib.tpla_workspace_size.argtypes = [ctypes.POINTER(CacheDesc), _I32, _I32, _I32, _I32, _I32,
                                        ctypes.POINTER(DecodeOpts), ctypes.POINTER(ctypes.c_size_t)]
    lib.latent_cache_append.restype = _I32
    lib.latent_cache_append.argtypes = [ctypes.POINTER(CacheDesc), _P, _P, _P, ctypes.c_int64, _P]
    decode_args = [ctypes.POINTER(CacheDesc), _P, _P, _P, _I32, _I32, _I32, _P, _P, ctypes.c_float,
                   _I32, _I32, _I32, _P, _P, _P, ctypes.c_size_t]
    lib.tpla_decode_sharded.restype = _I32
    lib.tpla_decode_sharded.argtypes = decode_args + [_P]
    lib.tpla_decode_sharded_ex.restype = _I32
    lib.tpla_decode_sharded_ex.argtypes = decode_args + [ctypes.POINTER(DecodeOpts), _P]
    lib.tpla_decode_sharded_noalloc.restype = _I32
    lib.tpla_decode_sharded_noalloc.argtypes = decode_args[:-2] + [_P]
    lib.tpla_decode_sharded_projected.restype = _I32
    lib.tpla_decode_sharded_projected.argtypes = (decode_args[:13] + [_I32, _P, _I32] + decode_args[13:]
                                                  + [ctypes.POINTER(DecodeOpts), _P])
    lib.mla_decode_absorbed.restype = _I32
    lib.mla_decode_absorbed.argtypes = [ctypes.POINTER(CacheDesc), _P, _P, _P, _I32, _I32, _I32, _P, _P,
                                        ctypes.c_float, _P, _P, _P, ctypes.c_size_t, _P]
    lib.latent_cache_append_normed.restype = _I32
    lib.latent_cache_append_normed.argtypes = [ctypes.POINTER(CacheDesc), _P, _P, _P, ctypes.c_int64, _I32,
                                               ctypes.c_float, _P]
    lib.tpla_merge_context_parts.restype = _I32
    lib.tpla_merge_context_parts.argtypes = [_I32] * 8 + [_P, _P, _P, _P, _P]
    lib.tpla_value_up_projection.restype = _I32
    lib.tpla_value_up_projection.argtypes = [_I32, _P, _P, _I32, _I32, _I32, _I32, _P, _P]
    lib.mla_prefill_workspace_size.restype = _I32
    lib.mla_prefill_workspace_size.argtypes = [ctypes.POINTER(CacheDesc), _I32, _I32, _I32, ctypes.POINTER(DecodeOpts),
                                               ctypes.POINTER(ctypes.c_size_t)]
    prefill_args = [ctypes.POINTER(CacheDesc), _P, _P, _P, _P, _I32, _I32, _I32, _I32, _P, _P, ctypes.c_float,
                    _P, _P, _P, ctypes.c_size_t]
    lib.mla_prefill_absorbed.restype = _I32
    lib.mla_prefill_absorbed.argtypes = prefill_args + [_P]
    lib.mla_prefill_absorbed_ex.restype = _I32
    lib.mla_prefill_absorbed_ex.argtypes = prefill_args + [ctypes.POINTER(DecodeOpts), _P]
    _LIB = lib
    return lib


def _check(status: int) -> None:
    if status != TPLA_OK:
        raise TplaError(status, load_library().tpla_last_error().decode())


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("the library takes device tensors only")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _event_handle(ev):
    """Raw hipEvent_t of a torch.cuda.Event (recorded once so that it exists)."""
    if ev is None:
        return None
    if not ev.cuda_event:
        ev.record()
    return ctypes.c_void_p(ev.cuda_event)


def _opts(chunk_tokens: int = 0, kernel: str = "auto", events=None, schedule: str = "auto"):
    if not chunk_tokens and kernel == "auto" and events is None and schedule == "auto":
        return None
    begin, end = events if events is not None else (None, None)
    return ctypes.byref(DecodeOpts(int(chunk_tokens), KERNELS[kernel], _event_handle(begin), _event_handle(end),
                                   SCHEDULES[schedule]))


def abi_version() -> int:
    return int(load_library().tpla_abi_version())


def workspace_size(desc: Desc, batch: int, heads: int, num_shards: int, shard_count: int, max_seq_len: int,
                   chunk_tokens: int = 0, kernel: str = "auto", schedule: str = "auto") -> int:
    lib = load_library()
    out = ctypes.c_size_t(0)
    cdesc = desc.c()
    _check(lib.tpla_workspace_size(ctypes.byref(cdesc), batch, heads, num_shards, shard_count, max_seq_len,
                                   _opts(chunk_tokens, kernel, None, schedule), ctypes.byref(out)))
    return int(out.value)


def latent_cache_append(desc: Desc, cache: torch.Tensor, rows: torch.Tensor, slots: torch.Tensor,
                        stream=None) -> None:
    """Store rows [n, d_latent + d_rope] at slots (int64 [n]) of the cache pool."""
    if slots.dtype != torch.int64:
        raise ValueError("slots must be int64")
    lib = load_library()
    cdesc = desc.c()
    _check(lib.latent_cache_append(ctypes.byref(cdesc), _ptr(cache), _ptr(rows), _ptr(slots), int(slots.numel()),
                                   _stream(stream)))


def latent_cache_append_normed(desc: Desc, cache: torch.Tensor, rows: torch.Tensor, slots: torch.Tensor,
                               norm_slices: int, eps: float = 1e-6, stream=None) -> None:
    """latent_cache_append with the latent RMS-normalised (unit gain) over norm_slices equal slices."""
    if slots.dtype != torch.int64:
        raise ValueError("slots must be int64")
    lib = load_library()
    cdesc = desc.c()
    _check(lib.latent_cache_append_normed(ctypes.byref(cdesc), _ptr(cache), _ptr(rows), _ptr(slots),
                                          int(slots.numel()), norm_slices, ctypes.c_float(eps), _stream(stream)))


def alloc_workspace(nbytes: int, device) -> torch.Tensor:
    """Device workspace (torch allocations are 256-byte aligned)."""
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def tpla_decode_sharded(desc: Desc, cache: torch.Tensor, block_table: torch.Tensor | None, seq_lens: torch.Tensor,
                        q_latent: torch.Tensor, q_rope: torch.Tensor, scale: float, num_shards: int,
                        max_seq_len: int, shard_begin: int = 0, shard_count: int | None = None,
                        out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                        workspace: torch.Tensor | None = None, want_lse: bool = True,
                        chunk_tokens: int = 0, kernel: str = "auto", events=None, stream=None, schedule: str = "auto"):
    """TPLA decode; returns (out [B, H, d_latent] fp32, lse [B, shard_count, H] fp32 or None).

    ``events=(begin, end)`` (torch.cuda.Event with timing) are recorded around the split-K
    decode kernel alone."""
    if shard_count is None:
        shard_count = num_shards - shard_begin
    batch, heads = int(q_latent.shape[0]), int(q_latent.shape[1])
    dev = q_latent.device
    if seq_lens.dtype != torch.int32 or (block_table is not None and block_table.dtype != torch.int32):
        raise ValueError("seq_lens and block_table must be int32")
    if out is None:
        out = torch.empty((batch, heads, desc.d_latent), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((batch, shard_count, heads), dtype=torch.float32, device=dev)
    need = workspace_size(desc, batch, heads, num_shards, shard_count, max_seq_len, chunk_tokens, kernel, schedule)
    if workspace is None:
        workspace = alloc_workspace(need, dev)
    lib = load_library()
    cdesc = desc.c()
    _check(lib.tpla_decode_sharded_ex(ctypes.byref(cdesc), _ptr(cache), _ptr(block_table), _ptr(seq_lens), batch, heads,
                                      max_seq_len, _ptr(q_latent), _ptr(q_rope), ctypes.c_float(scale), num_shards,
                                      shard_begin, shard_count, _ptr(out), _ptr(lse), _ptr(workspace),
                                      workspace.numel(), _opts(chunk_tokens, kernel, events, schedule), _stream(stream)))
    return out, lse


def tpla_decode_sharded_noalloc(desc: Desc, cache: torch.Tensor, block_table: torch.Tensor | None,
                                seq_lens: torch.Tensor, q_latent: torch.Tensor, q_rope: torch.Tensor, scale: float,
                                num_shards: int, max_seq_len: int, out: torch.Tensor, lse: torch.Tensor | None,
                                shard_begin: int = 0, shard_count: int | None = None, stream=None):
    """TPLA decode through the allocation-free entry point (the library's static scratch); the
    caller passes the outputs, nothing is allocated.  Returns (out, lse)."""
    if shard_count is None:
        shard_count = num_shards - shard_begin
    batch, heads = int(q_latent.shape[0]), int(q_latent.shape[1])
    if seq_lens.dtype != torch.int32 or (block_table is not None and block_table.dtype != torch.int32):
        raise ValueError("seq_lens and block_table must be int32")
    lib = load_library()
    cdesc = desc.c()
    _check(lib.tpla_decode_sharded_noalloc(ctypes.byref(cdesc), _ptr(cache), _ptr(block_table), _ptr(seq_lens), batch,
                                           heads, max_seq_len, _ptr(q_latent), _ptr(q_rope), ctypes.c_float(scale),
                                           num_shards, shard_begin, shard_count, _ptr(out), _ptr(lse), _stream(stream)))
    return out, lse


def tpla_decode_sharded_projected(desc: Desc, cache: torch.Tensor, block_table: torch.Tensor | None,
                                  seq_lens: torch.Tensor, q_latent: torch.Tensor, q_rope: torch.Tensor, scale: float,
                                  num_shards: int, max_seq_len: int, w_uv: torch.Tensor, shard_begin: int = 0,
                                  shard_count: int | None = None, out_v: torch.Tensor | None = None,
                                  lse: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                                  want_lse: bool = True, chunk_tokens: int = 0, kernel: str = "auto", events=None,
                                  stream=None, schedule: str = "auto"):
    """TPLA decode with the value up-projection fused into the merge; w_uv bf16 [H, d_v, d_latent].
    Returns (out_v [B, H, d_v] fp32, lse [B, shard_count, H] fp32 or None)."""
    if shard_count is None:
        shard_count = num_shards - shard_begin
    batch, heads = int(q_latent.shape[0]), int(q_latent.shape[1])
    dev = q_latent.device
    if seq_lens.dtype != torch.int32 or (block_table is not None and block_table.dtype != torch.int32):
        raise ValueError("seq_lens and block_table must be int32")
    if w_uv.dim() != 3 or int(w_uv.shape[0]) != heads or int(w_uv.shape[2]) != desc.d_latent:
        raise ValueError("w_uv must be [heads, d_v, d_latent]")
    d_v = int(w_uv.shape[1])
    w_dtype = DTYPES["bf16"] if w_uv.dtype == torch.bfloat16 else DTYPES["f32"]
    if out_v is None:
        out_v = torch.empty((batch, heads, d_v), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((batch, shard_count, heads), dtype=torch.float32, device=dev)
    need = workspace_size(desc, batch, heads, num_shards, shard_count, max_seq_len, chunk_tokens, kernel, schedule)
    if workspace is None:
        workspace = alloc_workspace(need, dev)
    lib = load_library()
    cdesc = desc.c()
    _check(lib.tpla_decode_sharded_projected(ctypes.byref(cdesc), _ptr(cache), _ptr(block_table), _ptr(seq_lens),
                                             batch, heads, max_seq_len, _ptr(q_latent), _ptr(q_rope),
                                             ctypes.c_float(scale), num_shards, shard_begin, shard_count, w_dtype,
                                             _ptr(w_uv), d_v, _ptr(out_v), _ptr(lse), _ptr(workspace),
                                             workspace.numel(), _opts(chunk_tokens, kernel, events, schedule),
                                             _stream(stream)))
    return out_v, lse


def mla_decode_absorbed(desc: Desc, cache: torch.Tensor, block_table: torch.Tensor | None, seq_lens: torch.Tensor,
                        q_latent: torch.Tensor, q_rope: torch.Tensor, scale: float, max_seq_len: int,
                        out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                        workspace: torch.Tensor | None = None, want_lse: bool = True, stream=None):
    """Exact absorbed MLA decode; returns (out [B, H, d_latent], lse [B, H] or None)."""
    batch, heads = int(q_latent.shape[0]), int(q_latent.shape[1])
    dev = q_latent.device
    if out is None:
        out = torch.empty((batch, heads, desc.d_latent), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((batch, heads), dtype=torch.float32, device=dev)
    need = workspace_size(desc, batch, heads, 1, 1, max_seq_len)
    if workspace is None:
        workspace = alloc_workspace(need, dev)
    lib = load_library()
    cdesc = desc.c()
    _check(lib.mla_decode_absorbed(ctypes.byref(cdesc), _ptr(cache), _ptr(block_table), _ptr(seq_lens), batch, heads,
                                   max_seq_len, _ptr(q_latent), _ptr(q_rope), ctypes.c_float(scale), _ptr(out),
                                   _ptr(lse), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out, lse


def prefill_workspace_size(desc: Desc, num_queries: int, heads: int, max_seq_len: int, chunk_tokens: int = 0,
                           kernel: str = "auto", schedule: str = "auto") -> int:
    lib = load_library()
    out = ctypes.c_size_t(0)
    cdesc = desc.c()
    _check(lib.mla_prefill_workspace_size(ctypes.byref(cdesc), num_queries, heads, max_seq_len,
                                          _opts(chunk_tokens, kernel, None, schedule), ctypes.byref(out)))
    return int(out.value)


def mla_prefill_absorbed(desc: Desc, cache: torch.Tensor, block_table: torch.Tensor | None, seq_lens: torch.Tensor,
                         query_start: torch.Tensor, q_latent: torch.Tensor, q_rope: torch.Tensor, scale: float,
                         max_seq_len: int, out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                         workspace: torch.Tensor | None = None, want_lse: bool = True, chunk_tokens: int = 0,
                         kernel: str = "auto", events=None, stream=None, schedule: str = "auto"):
    """Exact absorbed MLA prefill over the cache; returns (out [Nq, H, d_latent], lse [Nq, H] or None).

    ``query_start`` (int32 [batch + 1]) gives each sequence's query rows; the new tokens' rows
    must already be in the cache (they are the last of seq_lens[b])."""
    num_queries, heads = int(q_latent.shape[0]), int(q_latent.shape[1])
    batch = int(query_start.numel()) - 1
    dev = q_latent.device
    if seq_lens.dtype != torch.int32 or query_start.dtype != torch.int32 or (
            block_table is not None and block_table.dtype != torch.int32):
        raise ValueError("seq_lens, query_start and block_table must be int32")
    if out is None:
        out = torch.empty((num_queries, heads, desc.d_latent), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((num_queries, heads), dtype=torch.float32, device=dev)
    need = prefill_workspace_size(desc, num_queries, heads, max_seq_len, chunk_tokens, kernel, schedule)
    if workspace is None:
        workspace = alloc_workspace(need, dev)
    lib = load_library()
    cdesc = desc.c()
    _check(lib.mla_prefill_absorbed_ex(ctypes.byref(cdesc), _ptr(cache), _ptr(block_table), _ptr(seq_lens),
                                       _ptr(query_start), batch, num_queries, heads, max_seq_len, _ptr(q_latent),
                                       _ptr(q_rope), ctypes.c_float(scale), _ptr(out), _ptr(lse), _ptr(workspace),
                                       workspace.numel(), _opts(chunk_tokens, kernel, events, schedule),
                                       _stream(stream)))
    return out, lse


def tpla_value_up_projection(o: torch.Tensor, w_uv: torch.Tensor, out_v: torch.Tensor | None = None, stream=None):
    """out_v[b, h] = w_uv[h] @ o[b, h]; o fp32 [B, H, d_latent], w_uv [H, d_v, d_latent] (fp32 or bf16).
    Returns out_v fp32 [B, H, d_v]."""
    if o.dtype != torch.float32 or w_uv.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("o must be fp32 and w_uv fp32 or bf16")
    batch, heads, d_latent = (int(x) for x in o.shape)
    if tuple(w_uv.shape[::2]) != (heads, d_latent):
        raise ValueError("w_uv must be [heads, d_v, d_latent]")
    d_v = int(w_uv.shape[1])
    if out_v is None:
        out_v = torch.empty((batch, heads, d_v), dtype=torch.float32, device=o.device)
    w_dtype = DTYPES["bf16"] if w_uv.dtype == torch.bfloat16 else DTYPES["f32"]
    lib = load_library()
    _check(lib.tpla_value_up_projection(w_dtype, _ptr(o), _ptr(w_uv), batch, heads, d_latent, d_v, _ptr(out_v),
                                        _stream(stream)))
    return out_v


def tpla_merge_context_parts(out_parts: torch.Tensor, lse_parts: torch.Tensor, num_shards: int,
                             shard_begin: int = 0, transform: str = "identity", out: torch.Tensor | None = None,
                             lse: torch.Tensor | None = None, want_lse: bool = True, stream=None):
    """Merge P decode results over disjoint context parts: out_parts fp32 [P, B, H, d_latent],
    lse_parts fp32 [P, B, n, H] -> (out [B, H, d_latent], lse [B, n, H] or None)."""
    if out_parts.dtype != torch.float32 or lse_parts.dtype != torch.float32:
        raise ValueError("out_parts and lse_parts must be fp32")
    parts, batch, heads, d_latent = (int(x) for x in out_parts.shape)
    shard_count = int(lse_parts.shape[2])
    if tuple(lse_parts.shape) != (parts, batch, shard_count, heads):
        raise ValueError("lse_parts must be [parts, batch, shard_count, heads]")
    if out is None:
        out = torch.empty((batch, heads, d_latent), dtype=torch.float32, device=out_parts.device)
    if lse is None and want_lse:
        lse = torch.empty((batch, shard_count, heads), dtype=torch.float32, device=out_parts.device)
    lib = load_library()
    _check(lib.tpla_merge_context_parts(TRANSFORMS[transform], num_shards, shard_begin, shard_count, parts, batch,
                                        heads, d_latent, _ptr(out_parts), _ptr(lse_parts), _ptr(out), _ptr(lse),
                                        _stream(stream)))
    return out, lse
