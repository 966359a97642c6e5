"""GPU parity on a seeded sweep of random small configurations: batch, heads, shard count and
subset, context lengths (empty ones included), layout and page size, transform, dtype, schedule.
Each configuration is checked against the fp64 oracle at the bar of its dtype."""

import numpy as np
import pytest
import torch

from gpu_case import DeviceCase, assert_lse, assert_parity, oracle_decode
from mla_latent_kv_13_amd import inputs

pytestmark = pytest.mark.gpu


def _config(i):
    rng = np.random.default_rng([7919, i])
    dtype = "f32" if rng.random() < 0.15 else "bf16"
    mfma_shape = dtype == "bf16" and rng.random() < 0.7
    if mfma_shape:  # shapes the matrix-core kernel takes: slices of 128/256/512, rope 64, heads % 32 == 0
        d_latent, d_rope = 512, 64
        shards = int(rng.choice([1, 2, 4]))
        heads = int(32 * rng.integers(1, 5))
    else:
        d_latent = int(rng.choice([64, 128, 256]))
        d_rope = int(rng.choice([8, 16, 32]))
        shards = int(rng.choice([s for s in (1, 2, 4, 8) if d_latent % s == 0]))
        heads = int(rng.integers(1, 9))
    batch = int(rng.integers(1, 7))
    lens = [int(x) for x in rng.integers(0, 1500, size=batch)]
    if rng.random() < 0.3:
        lens[int(rng.integers(0, batch))] = 0
    paged = bool(rng.random() < 0.6)
    page_size = int(rng.choice([1, 8, 16, 32, 64, 128])) if paged else 64
    transform = "wht" if rng.random() < 0.4 else "identity"
    shard_begin = int(rng.integers(0, shards))
    shard_count = int(rng.integers(1, shards - shard_begin + 1))
    schedule = str(rng.choice(["auto", "chunked", "balanced"])) if mfma_shape else "auto"
    scale = float(rng.uniform(-0.2, 0.2)) if rng.random() < 0.1 else 1.0 / np.sqrt(d_latent // shards + d_rope)
    return dict(batch=batch, heads=heads, d_latent=d_latent, d_rope=d_rope, shards=shards, lens=lens,
                dtype=dtype, paged=paged, page_size=page_size, transform=transform, scale=scale,
                channel_sigma=0.5 if rng.random() < 0.3 else None,
                extra_pages=int(rng.integers(1, 3)) if paged else 0), shard_begin, shard_count, schedule


@pytest.mark.parametrize("i", range(100))
def test_random_configuration(i):
    kw, s0, n, schedule = _config(i)
    print(f"config {i}: {kw} shards [{s0}, {s0 + n}) schedule {schedule}", flush=True)
    case = inputs.make_case(9000 + i, name=f"random-{i}", **kw)
    dc = DeviceCase(case)
    out, lse = dc.decode(shard_begin=s0, shard_count=n, schedule=schedule)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_decode(case, shard_begin=s0, shard_count=n)
    got = out.detach().cpu().numpy()
    if np.max(np.abs(ref)) == 0.0:  # every sequence empty
        assert np.all(got == 0.0)
    else:
        assert_parity(got, ref, case.dtype, f"config {i}")
    assert_lse(lse.detach().cpu().numpy(), ref_lse, case.dtype, f"config {i}", case.transform)
