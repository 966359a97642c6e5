"""Seeded synthetic inputs for latent-cache decode, shared by the tests and the benchmark.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic, so both the HIP path and the CPU oracle can consume its
arrays without sharing any computation.

Recipe (one generator per tensor, ``np.random.default_rng([case_seed, tensor_id])``):

  tensor 0  q_lat      [B, H, d_c]  standard normal
  tensor 1  q_rope     [B, H, d_r]  standard normal
  tensor 2  latent     per sequence b = 0..B-1 in order, [T_b, d_c] standard normal
  tensor 3  rope key   per sequence b in order, [T_b, d_r] standard normal
  tensor 4  per-channel log-scale of the latent, [d_c] ~ N(0, sigma); the
            latent is multiplied by exp(log-scale) (Kimi-K2-shaped case)
  tensor 5  context lengths, integers uniform in [lo, hi] inclusive
  tensor 6  page permutation for the paged layout

Context-merge inputs (``make_context_parts``, its own seed): tensor 0 the parts' outputs
[P, B, H, d_c] (float32 normals), tensor 1 their log-sum-exps [P, B, n, H] (normals times 3),
tensor 2 which of those are -inf (a part with no tokens), each with probability ``empty``.

Value up-projection inputs (``make_value_projection``, its own seed): tensor 0 the latent-frame
attention output o [B, H, d_c] (float32 normals), tensor 1 the per-head value weights
W_UV [H, d_v, d_c], normals scaled by 1/sqrt(d_c) (the spread of a trained projection's
rows), in the weight dtype.

Normals are drawn as float32.  bf16 cases round them to bfloat16 with
round-to-nearest-even and keep the raw 16-bit patterns (uint16).  Rows of a
page beyond a sequence's length, and pool pages no sequence uses, are filled
with NaN so that any read of them would show up in the result.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

BF16_NAN = np.uint16(0x7FC0)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact)."""
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def stored_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of a stored array (bf16 bit patterns or float32)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


@dataclass
class Case:
    """One decode problem: queries, cache layout and the rows that fill it."""

    name: str
    dtype: str              # "bf16" (uint16 bit patterns) or "f32"
    batch: int
    heads: int
    d_latent: int
    d_rope: int
    shards: int
    scale: float            # float32 value passed to the library
    transform: str          # "identity" or "wht"
    page_size: int
    num_pages: int
    max_seq_len: int
    paged: bool
    q_lat: np.ndarray
    q_rope: np.ndarray
    seq_lens: np.ndarray    # int32 [B]
    block_table: np.ndarray | None  # int32 [B, max_pages_per_seq], -1 where unused
    rows: np.ndarray        # [n, d_c + d_r] raw rows in (b, t) order
    slots: np.ndarray       # int64 [n], page * page_size + offset of each row
    pool: np.ndarray | None = None  # [num_pages, page_size, d_c + d_r]: rows placed, NaN elsewhere
    meta: dict = field(default_factory=dict)

    @property
    def width(self) -> int:
        return self.d_latent + self.d_rope

    @property
    def max_pages_per_seq(self) -> int:
        return 0 if self.block_table is None else self.block_table.shape[1]

    @property
    def total_tokens(self) -> int:
        return int(self.seq_lens.astype(np.int64).sum())

    def empty_pool(self) -> np.ndarray:
        shape = (self.num_pages, self.page_size, self.width)
        if self.dtype == "bf16":
            return np.full(shape, BF16_NAN, dtype=np.uint16)
        return np.full(shape, np.nan, dtype=np.float32)


def _normal(rng, shape, dtype):
    return rng.standard_normal(shape, dtype=np.float32)


def _to_dtype(x32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x32) if dtype == "bf16" else x32.astype(np.float32)


def make_case(seed: int, *, batch: int, heads: int, d_latent: int, d_rope: int, shards: int,
              lens=None, len_range=None, dtype: str = "bf16", scale: float | None = None,
              transform: str = "identity", paged: bool = False, page_size: int = 64,
              max_seq_len: int | None = None, extra_pages: int = 0,
              channel_sigma: float | None = None, token_gain: float | None = None,
              place_rows: bool = True, name: str = "custom") -> Case:
    """Build a seeded case.

    ``lens`` gives the context length of every sequence (int or list);
    otherwise ``len_range=(lo, hi)`` draws them uniformly (inclusive).
    A contiguous layout (``paged=False``) gives each sequence its own page of
    ``max_seq_len`` rows and no block table.  A paged layout uses
    ``page_size``-row pages, assigned by a seeded random permutation, plus
    ``extra_pages`` NaN-filled pages that no sequence uses.
    ``token_gain`` scales the rows of each sequence geometrically along its
    tokens, from 1 at the first token to ``token_gain`` at the last (before the
    rounding to the stored dtype), so that later tiles hold much larger logits
    than the first: a decode then has to raise its running maximum mid-sequence.
    """
    if lens is not None:
        seq_lens = np.broadcast_to(np.asarray(lens, dtype=np.int64), (batch,)).astype(np.int32).copy()
    else:
        lo, hi = len_range
        seq_lens = np.random.default_rng([seed, 5]).integers(lo, hi, size=batch, endpoint=True).astype(np.int32)
    if max_seq_len is None:
        max_seq_len = int(max(1, seq_lens.max()))
    if int(seq_lens.max()) > max_seq_len:
        raise ValueError("a context length exceeds max_seq_len")
    if scale is None:
        scale = 1.0 / math.sqrt(d_latent // shards + d_rope)
    scale = float(np.float32(scale))

    q_lat = _to_dtype(_normal(np.random.default_rng([seed, 0]), (batch, heads, d_latent), dtype), dtype)
    q_rope = _to_dtype(_normal(np.random.default_rng([seed, 1]), (batch, heads, d_rope), dtype), dtype)

    total = int(seq_lens.astype(np.int64).sum())
    width = d_latent + d_rope
    rows32 = np.empty((total, width), dtype=np.float32)
    rng_lat = np.random.default_rng([seed, 2])
    rng_rope = np.random.default_rng([seed, 3])
    chan = None
    if channel_sigma is not None:
        chan = np.exp(np.random.default_rng([seed, 4]).normal(0.0, channel_sigma, size=d_latent).astype(np.float32))
    off = 0
    for b in range(batch):
        t_b = int(seq_lens[b])
        lat = rng_lat.standard_normal((t_b, d_latent), dtype=np.float32)
        if chan is not None:
            lat = lat * chan[None, :]
        rows32[off:off + t_b, :d_latent] = lat
        rows32[off:off + t_b, d_latent:] = rng_rope.standard_normal((t_b, d_rope), dtype=np.float32)
        if token_gain is not None and t_b > 1:
            ramp = np.float32(token_gain) ** (np.arange(t_b, dtype=np.float32) / np.float32(t_b - 1))
            rows32[off:off + t_b] *= ramp[:, None]
        off += t_b
    rows = _to_dtype(rows32, dtype)
    del rows32

    if paged:
        pages_per_seq = [(int(t) + page_size - 1) // page_size for t in seq_lens]
        used = sum(pages_per_seq)
        num_pages = used + extra_pages
        perm = np.random.default_rng([seed, 6]).permutation(num_pages)
        max_pages = (max_seq_len + page_size - 1) // page_size
        block_table = np.full((batch, max_pages), -1, dtype=np.int32)
        k = 0
        for b in range(batch):
            block_table[b, :pages_per_seq[b]] = perm[k:k + pages_per_seq[b]]
            k += pages_per_seq[b]
        page_of = block_table
        psize = page_size
    else:
        num_pages = batch
        block_table = None
        psize = max_seq_len
        page_of = None

    slots = np.empty(total, dtype=np.int64)
    off = 0
    for b in range(batch):
        t = np.arange(int(seq_lens[b]), dtype=np.int64)
        page = (np.full_like(t, b) if page_of is None else page_of[b][t // psize].astype(np.int64))
        slots[off:off + t.size] = page * psize + t % psize
        off += t.size

    case = Case(name=name, dtype=dtype, batch=batch, heads=heads, d_latent=d_latent, d_rope=d_rope,
                shards=shards, scale=scale, transform=transform, page_size=psize, num_pages=num_pages,
                max_seq_len=max_seq_len, paged=paged, q_lat=q_lat, q_rope=q_rope, seq_lens=seq_lens,
                block_table=block_table, rows=rows, slots=slots,
                meta=dict(seed=seed, channel_sigma=channel_sigma, token_gain=token_gain, extra_pages=extra_pages))
    if place_rows:
        pool = case.empty_pool()
        pool.reshape(num_pages * psize, width)[slots] = rows
        case.pool = pool
    return case


# The five benchmark workloads (synthetic stand-ins with DeepSeek-V3 / Kimi-K2 shapes).
WORKLOADS = {
    1: dict(name="tiny-tpla-g2-f32", batch=1, heads=4, d_latent=64, d_rope=16, shards=2, lens=128,
            dtype="f32", scale=1.0 / math.sqrt(48)),
    2: dict(name="dsv3-mla-g1-ctx4k-bf16", batch=32, heads=128, d_latent=512, d_rope=64, shards=1,
            lens=4096, dtype="bf16", scale=1.0 / math.sqrt(192)),
    3: dict(name="dsv3-tpla-g2-ctx32k-bf16", batch=16, heads=128, d_latent=512, d_rope=64, shards=2,
            lens=32768, dtype="bf16", scale=1.0 / math.sqrt(192)),
    4: dict(name="kimik2-tpla-g4-ctx32k-bf16", batch=32, heads=64, d_latent=512, d_rope=64, shards=4,
            lens=32768, dtype="bf16", scale=1.0 / math.sqrt(192), channel_sigma=0.5),
    5: dict(name="paged-wht-tpla-g2-ctx1k-64k-bf16", batch=64, heads=128, d_latent=512, d_rope=64,
            shards=2, len_range=(1024, 65536), max_seq_len=65536, paged=True, page_size=64,
            dtype="bf16", scale=1.0 / math.sqrt(192), transform="wht"),
}


def make_config(cfg: int, *, place_rows: bool | None = None) -> Case:
    """The seeded case for benchmark workload ``cfg`` (1..5); seed = cfg."""
    kw = dict(WORKLOADS[cfg])
    if place_rows is None:
        place_rows = kw.get("transform", "identity") == "identity"
    return make_case(cfg, place_rows=place_rows, **kw)


def make_value_projection(seed: int, *, batch: int, heads: int, d_latent: int, d_v: int, dtype: str = "bf16"):
    """Seeded (o [B, H, d_c] float32, W_UV [H, d_v, d_c] in ``dtype``) for the value up-projection."""
    o = np.random.default_rng([seed, 0]).standard_normal((batch, heads, d_latent), dtype=np.float32)
    w = np.random.default_rng([seed, 1]).standard_normal((heads, d_v, d_latent), dtype=np.float32)
    w = (w * np.float32(1.0 / math.sqrt(d_latent))).astype(np.float32)
    return o, _to_dtype(w, dtype)


def make_context_parts(seed: int, *, parts: int, batch: int, heads: int, d_latent: int, shard_count: int,
                       empty: float = 0.2):
    """Seeded (out_parts [P, B, H, d_c], lse_parts [P, B, n, H]) float32 for the context merge."""
    out = np.random.default_rng([seed, 0]).standard_normal((parts, batch, heads, d_latent), dtype=np.float32)
    lse = np.random.default_rng([seed, 1]).standard_normal((parts, batch, shard_count, heads), dtype=np.float32)
    lse = (lse * np.float32(3.0)).astype(np.float32)
    lse[np.random.default_rng([seed, 2]).random(lse.shape) < empty] = -np.inf
    return out, lse


def make_prefill_queries(seed: int, *, new_tokens, heads: int, d_latent: int, d_rope: int, dtype: str = "bf16"):
    """Seeded query rows of a prefill call: sequence b has new_tokens[b] new tokens (the last of
    its cached rows).  Returns (query_start int32 [B + 1], q_lat [Nq, H, d_c], q_rope [Nq, H, d_r])
    in ``dtype``; the values are N(0, 1) drawn as float32 and stored like decode queries."""
    query_start = np.concatenate([[0], np.cumsum(np.asarray(new_tokens, dtype=np.int64))]).astype(np.int32)
    nq = int(query_start[-1])
    q_lat = np.random.default_rng([seed, 0]).standard_normal((nq, heads, d_latent), dtype=np.float32)
    q_rope = np.random.default_rng([seed, 1]).standard_normal((nq, heads, d_rope), dtype=np.float32)
    return query_start, _to_dtype(q_lat, dtype), _to_dtype(q_rope, dtype)
