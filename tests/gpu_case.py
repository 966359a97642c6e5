"""Helpers for the GPU tests: move a seeded case to the device, run the library through the
C ABI, and run the fp64 oracle on the same arrays (or on a sample of sequences)."""

from __future__ import annotations

import numpy as np
import torch

import oracle
from mla_latent_kv_13_amd import binding, inputs

DEV = "cuda:0"

# Parity bar: relative L2 error and max-abs error relative to max|ref| over the whole output.
TOL = {"bf16": 2e-2, "f32": 1e-5}
# lse, relative to max(1, |lse|).  With an unrotated cache the bf16 path forms its logits
# exactly from the stored bf16 inputs in fp32, and the one bf16 rounding it adds (of the
# probabilities fed to the value product) does not enter lse.  With the Hadamard-rotated
# cache the rotated query is rounded to bf16 for the matrix cores: each logit then moves by
# about scale * 2^-9 / sqrt(3) * sqrt(w) (unit-variance entries), ~1e-3 at w = 256, scale
# 1/sqrt(192), and lse by as much.
LSE_TOL = {("bf16", "identity"): 1e-4, ("bf16", "wht"): 1e-2, ("f32", "identity"): 1e-5, ("f32", "wht"): 1e-5}


def to_torch(a: np.ndarray, dtype: str, device=DEV) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def desc_of(case: inputs.Case) -> binding.Desc:
    return binding.Desc(case.dtype, case.d_latent, case.d_rope, case.page_size, case.num_pages,
                        case.max_pages_per_seq, case.transform)


class DeviceCase:
    """Device copies of a case.  The pool is filled by the library's append for rotated caches,
    and also for plain ones when ``via_append`` is set (or the case carries no host pool);
    otherwise a plain pool is copied from the host."""

    def __init__(self, case: inputs.Case, device=DEV, via_append: bool = False):
        self.case = case
        self.desc = desc_of(case)
        self.q_lat = to_torch(case.q_lat, case.dtype, device)
        self.q_rope = to_torch(case.q_rope, case.dtype, device)
        self.seq_lens = torch.from_numpy(case.seq_lens).to(device)
        self.block_table = None if case.block_table is None else torch.from_numpy(case.block_table).to(device)
        if case.transform == "identity" and case.pool is not None and not via_append:
            self.pool = to_torch(case.pool, case.dtype, device)
        else:
            self.pool = to_torch(case.empty_pool(), case.dtype, device)
            rows = to_torch(case.rows, case.dtype, device)
            slots = torch.from_numpy(case.slots).to(device)
            binding.latent_cache_append(self.desc, self.pool, rows, slots)
            del rows, slots

    def decode(self, shard_begin=0, shard_count=None, **kw):
        c = self.case
        return binding.tpla_decode_sharded(self.desc, self.pool, self.block_table, self.seq_lens, self.q_lat,
                                           self.q_rope, c.scale, c.shards, c.max_seq_len, shard_begin=shard_begin,
                                           shard_count=shard_count, **kw)


def oracle_pool(case: inputs.Case, seqs):
    """(pool [len(seqs), T_max, width] float64, lens): a compact contiguous pool of sequences `seqs`
    built from the case's raw rows (the oracle's own append builds rotated caches)."""
    starts = np.concatenate([[0], np.cumsum(case.seq_lens.astype(np.int64))])
    lens = case.seq_lens[seqs]
    tmax = int(max(1, lens.max()))
    pool = np.full((len(seqs), tmax, case.width), np.nan)
    rows, slots = [], []
    for i, b in enumerate(seqs):
        r = inputs.stored_to_f64(case.rows[starts[b]:starts[b + 1]], case.dtype)
        if case.transform == "identity":
            pool[i, :r.shape[0]] = r
        else:
            rows.append(r)
            slots.append(i * tmax + np.arange(r.shape[0]))
    if case.transform != "identity" and rows:
        pool = oracle.latent_cache_append(pool, np.concatenate(rows), np.concatenate(slots), case.d_latent,
                                          case.transform, case.dtype)
    return pool, lens


def oracle_decode(case: inputs.Case, seqs=None, shard_begin=0, shard_count=None, heads=None):
    """Oracle output for sequences `seqs` (all by default) and query heads `heads` (all by
    default; heads are independent, so a subset is exact) on a compact contiguous pool built
    from the case's raw rows."""
    if seqs is None:
        seqs = list(range(case.batch))
    seqs = list(seqs)
    pool, lens = oracle_pool(case, seqs)
    q_lat = inputs.stored_to_f64(case.q_lat, case.dtype)[seqs]
    q_rope = inputs.stored_to_f64(case.q_rope, case.dtype)[seqs]
    if heads is not None:
        q_lat, q_rope = q_lat[:, list(heads)], q_rope[:, list(heads)]
    return oracle.tpla_decode_sharded(pool, None, lens, q_lat, q_rope, float(np.float32(case.scale)), case.shards,
                                      shard_begin, shard_count, transform=case.transform)


def oracle_decode_grouped(case: inputs.Case, seqs=None, group: int = 4, shard_begin=0, shard_count=None):
    """oracle_decode over `seqs` (all by default), `group` sequences at a time, so that the
    oracle's fp64 copies of a large cache never exist whole; returns (out, lse) for `seqs`."""
    seqs = list(range(case.batch)) if seqs is None else list(seqs)
    outs, lses = [], []
    for k in range(0, len(seqs), group):
        o, l = oracle_decode(case, seqs[k:k + group], shard_begin, shard_count)
        outs.append(o)
        lses.append(l)
    return np.concatenate(outs), np.concatenate(lses)


def parity(got, ref):
    """(relative L2 error, max-abs error / max|ref|) of got against ref."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = np.max(np.abs(ref))
    if scale == 0.0:
        return (0.0 if np.all(got == 0) else np.inf), (0.0 if np.all(got == 0) else np.inf)
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref)), float(np.max(np.abs(got - ref)) / scale)


def assert_parity(got, ref, dtype, what=""):
    rel, mx = parity(got, ref)
    tol = TOL[dtype]
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert rel <= tol and mx <= tol, f"{what}: rel L2 {rel:.3e}, max-abs/max|ref| {mx:.3e} (tol {tol})"
    return rel, mx


def assert_lse(got, ref, dtype, what="", transform="identity"):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    same_inf = np.isneginf(got) == np.isneginf(ref)
    assert np.all(same_inf), f"{what}: -inf pattern of lse differs"
    fin = ~np.isneginf(ref)
    if np.any(fin):
        err = np.max(np.abs(got[fin] - ref[fin]) / np.maximum(1.0, np.abs(ref[fin])))
        assert err <= LSE_TOL[(dtype, transform)], f"{what}: lse error {err:.3e}"
