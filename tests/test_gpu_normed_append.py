"""GPU parity of latent_cache_append_normed (RMS normalisation with unit gain over the whole latent
or over G slices, after the optional Hadamard rotation) against the fp64 oracle, and a decode over
a cache written that way."""

import numpy as np
import pytest
import torch

import oracle
from gpu_case import DEV, assert_lse, assert_parity, desc_of, parity, to_torch
from mla_latent_kv_13_amd import binding, inputs

pytestmark = pytest.mark.gpu

# (name, d_latent, d_rope, dtype, transform, norm_slices, eps)
CASES = [
    ("plain_whole_latent", 512, 64, "bf16", "identity", 1, 1e-6),
    ("plain_four_slices", 512, 64, "bf16", "identity", 4, 1e-6),
    ("rotated_whole_latent", 512, 64, "bf16", "wht", 1, 1e-6),
    ("rotated_two_slices", 512, 64, "bf16", "wht", 2, 1e-2),
    ("rotated_1024_eight_slices_fp32", 1024, 32, "f32", "wht", 8, 1e-6),
    ("rotated_32_two_slices", 32, 16, "bf16", "wht", 2, 1e-6),
    ("plain_64_sixty_four_slices_fp32", 64, 8, "f32", "identity", 64, 1e-3),
]


def _append_both(name, d_latent, d_rope, dtype, transform, norm, eps, lens):
    case = inputs.make_case(500 + len(name), batch=len(lens), heads=32, d_latent=d_latent, d_rope=d_rope, shards=1,
                            lens=lens, dtype=dtype, transform=transform, paged=True, page_size=16, extra_pages=2,
                            channel_sigma=0.7, place_rows=False)
    pool = to_torch(case.empty_pool(), dtype)
    binding.latent_cache_append_normed(desc_of(case), pool, to_torch(case.rows, dtype),
                                       torch.from_numpy(case.slots).to(DEV), norm, eps)
    torch.cuda.synchronize()
    if dtype == "bf16":
        got = inputs.stored_to_f64(pool.view(torch.int16).cpu().numpy().view(np.uint16), dtype)
    else:
        got = pool.cpu().numpy().astype(np.float64)
    raw = inputs.stored_to_f64(case.rows, dtype)
    empty = np.full((1, raw.shape[0], d_latent + d_rope), np.nan)
    ref = oracle.latent_cache_append(empty, raw, np.arange(raw.shape[0]), d_latent, transform, dtype,
                                     norm_slices=norm, eps=eps)[0]
    return case, pool, got.reshape(-1, d_latent + d_rope), ref


@pytest.mark.parametrize("name,d_latent,d_rope,dtype,transform,norm,eps", CASES, ids=[c[0] for c in CASES])
def test_normed_append_matches_oracle(name, d_latent, d_rope, dtype, transform, norm, eps):
    print(f"case {name}", flush=True)
    case, _, flat, ref = _append_both(name, d_latent, d_rope, dtype, transform, norm, eps, [40, 7, 1])
    mine = flat[case.slots]
    if dtype == "bf16":  # one bf16 rounding of an fp32 value: at most one unit apart, nearly always equal
        ulp = np.ldexp(1.0, np.frexp(ref[:, :d_latent])[1] - 8)
        assert np.all(np.abs(mine[:, :d_latent] - ref[:, :d_latent]) <= ulp)
        assert np.mean(mine[:, :d_latent] == ref[:, :d_latent]) > 0.98
    else:
        rel, mx = parity(mine[:, :d_latent], ref[:, :d_latent])
        assert rel <= 1e-5 and mx <= 1e-5, (rel, mx)
    assert np.array_equal(mine[:, d_latent:], ref[:, d_latent:])  # rope unchanged
    untouched = np.ones(flat.shape[0], dtype=bool)
    untouched[case.slots] = False
    assert np.all(np.isnan(flat[untouched]))


def test_decode_over_shard_normed_rotated_cache():
    """G = 2 decode over a cache whose rotated latent was normalised per shard slice, against the
    oracle's decode over the oracle's own normalised cache."""
    case, pool, _, ref_rows = _append_both("decode_normed", 512, 64, "bf16", "wht", 2, 1e-6, [300, 65])
    case.shards = 2
    q_lat, q_rope = to_torch(case.q_lat, "bf16"), to_torch(case.q_rope, "bf16")
    out, lse = binding.tpla_decode_sharded(desc_of(case), pool, torch.from_numpy(case.block_table).to(DEV),
                                           torch.from_numpy(case.seq_lens).to(DEV), q_lat, q_rope, case.scale, 2,
                                           case.max_seq_len)
    torch.cuda.synchronize()
    # the oracle's normalised rotated rows, in a compact contiguous pool per sequence
    starts = np.concatenate([[0], np.cumsum(case.seq_lens)])
    tmax = int(case.seq_lens.max())
    opool = np.full((case.batch, tmax, 576), np.nan)
    for b in range(case.batch):
        opool[b, :case.seq_lens[b]] = ref_rows[starts[b]:starts[b + 1]]
    ref, ref_lse = oracle.tpla_decode_sharded(opool, None, case.seq_lens, inputs.stored_to_f64(case.q_lat, "bf16"),
                                              inputs.stored_to_f64(case.q_rope, "bf16"), case.scale, 2,
                                              transform="wht")
    assert_parity(out.cpu().numpy(), ref, "bf16", "decode over a shard-normalised cache")
    assert_lse(lse.cpu().numpy(), ref_lse, "bf16", "decode over a shard-normalised cache", "wht")
