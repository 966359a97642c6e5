"""GPU parity of the value up-projection (tpla_value_up_projection) against the fp64 oracle,
alone and after a decode call (a device's shard share projects to its operand of the all-reduce)."""

import numpy as np
import pytest
import torch

import oracle
from gpu_case import DeviceCase, assert_parity, oracle_decode, parity, to_torch
from mla_latent_kv_13_amd import binding, inputs

pytestmark = pytest.mark.gpu

# Bar for the projection alone: the weights are used exactly as stored and o enters with about
# 16 significant bits (bf16 value plus bf16 remainder), accumulated in fp32: the fp32 bar.
TOL = 1e-5

# (name, batch, heads, d_latent, d_v, weight dtype): matrix-core tiles with whole and ragged
# 32-row / 32-column blocks (batches of 32 and 64 at DeepSeek-V3 shapes; value widths up to 600;
# latent widths up to 2064), a single element, and the fp32 path (fp32 weights, or a latent width
# that is not a multiple of 16).
SHAPES = [
    ("dsv3_shape", 32, 128, 512, 128, "bf16"),
    ("paged_headline_batch", 64, 128, 512, 128, "bf16"),
    ("two_kparts_dv256", 40, 4, 512, 256, "bf16"),
    ("one_kpart_dv300", 19, 3, 256, 300, "bf16"),
    ("latent_1024_lds_over_64k", 33, 2, 1024, 128, "bf16"),
    ("dv600_tile_kernel", 5, 2, 128, 600, "bf16"),
    ("latent_2064_tile_kernel", 3, 1, 2064, 64, "bf16"),
    ("ragged_rows_and_columns", 37, 3, 64, 45, "bf16"),
    ("one_output", 1, 1, 16, 1, "bf16"),
    ("two_row_blocks_g4_width", 70, 5, 128, 96, "bf16"),
    ("fp32_weights", 5, 4, 48, 7, "f32"),
    ("bf16_width_not_multiple_of_16", 6, 2, 40, 9, "bf16"),
]


@pytest.mark.parametrize("name,batch,heads,d_latent,d_v,dtype", SHAPES, ids=[s[0] for s in SHAPES])
def test_projection_matches_oracle(name, batch, heads, d_latent, d_v, dtype):
    print(f"case {name}", flush=True)
    o, w = inputs.make_value_projection(200 + len(name), batch=batch, heads=heads, d_latent=d_latent, d_v=d_v,
                                        dtype=dtype)
    got = binding.tpla_value_up_projection(torch.from_numpy(o).cuda(), to_torch(w, dtype))
    torch.cuda.synchronize()
    ref = oracle.value_up_projection(o.astype(np.float64), inputs.stored_to_f64(w, dtype))
    rel, mx = parity(got.cpu().numpy(), ref)
    print(f"  rel L2 {rel:.2e} max {mx:.2e}", flush=True)
    assert rel <= TOL and mx <= TOL, (name, rel, mx)


def test_projection_overwrites_output_and_empty_batch():
    o, w = inputs.make_value_projection(301, batch=3, heads=2, d_latent=32, d_v=33)
    out = torch.full((3, 2, 33), float("nan"), device="cuda:0")
    binding.tpla_value_up_projection(torch.from_numpy(o).cuda(), to_torch(w, "bf16"), out_v=out)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    empty = torch.empty((0, 2, 32), dtype=torch.float32, device="cuda:0")
    assert binding.tpla_value_up_projection(empty, to_torch(w, "bf16")).shape == (0, 2, 33)


@pytest.mark.parametrize("transform", ["identity", "wht"])
def test_shard_shares_project_to_allreduce_operands(transform):
    """Each shard's decode share, projected, is one device's all-reduce operand: their fp32 sum
    equals the projection of the full call, and both match the oracle chain."""
    case = inputs.make_case(17, batch=3, heads=64, d_latent=512, d_rope=64, shards=2, lens=[700, 45, 1],
                            paged=True, page_size=64, transform=transform, scale=1.0 / np.sqrt(192))
    _, w = inputs.make_value_projection(18, batch=1, heads=64, d_latent=512, d_v=128)
    wt = to_torch(w, "bf16")
    dc = DeviceCase(case)
    full, _ = dc.decode()
    proj_full = binding.tpla_value_up_projection(full, wt)
    total = torch.zeros_like(proj_full)
    for s in range(2):
        part, _ = dc.decode(shard_begin=s, shard_count=1)
        total += binding.tpla_value_up_projection(part, wt)
    torch.cuda.synchronize()
    rel, mx = parity(total.cpu().numpy(), proj_full.cpu().numpy())
    assert rel < 1e-5 and mx < 1e-5, (rel, mx)
    ref_lat, _ = oracle_decode(case)
    ref = oracle.value_up_projection(ref_lat, inputs.stored_to_f64(w, "bf16"))
    assert_parity(proj_full.cpu().numpy(), ref, "bf16", f"projected decode ({transform})")
