"""GPU: the allocation-free decode entry point (tpla_decode_sharded_noalloc, for callers that
cannot allocate device memory) against tpla_decode_sharded with a caller workspace, on calls in a
row through the C ABI: a larger paged Hadamard-rotated call, then a smaller plain one (the static
scratch still holds the first call's partials), then the first again.  Both entry points run the
same plan and kernels, so the outputs must agree bit for bit (and lie within the parity bar of the
oracle's bf16 tolerance of each other)."""

import numpy as np
import pytest
import torch

from gpu_case import DeviceCase, assert_parity, desc_of
from mla_latent_kv_13_amd import binding, inputs

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 64 << 20


def _cases():
    big = inputs.make_case(501, batch=8, heads=128, d_latent=512, d_rope=64, shards=2,
                           lens=[20000, 1, 777, 0, 9000, 64, 31, 15000], paged=True, page_size=64,
                           transform="wht", extra_pages=3, scale=1.0 / np.sqrt(192), place_rows=False)
    small = inputs.make_case(502, batch=3, heads=64, d_latent=512, d_rope=64, shards=4, lens=[500, 33, 1],
                             scale=1.0 / np.sqrt(192))
    return big, small


def _noalloc(dc, out, lse):
    c = dc.case
    return binding.tpla_decode_sharded_noalloc(dc.desc, dc.pool, dc.block_table, dc.seq_lens, dc.q_lat, dc.q_rope,
                                               c.scale, c.shards, c.max_seq_len, out, lse)


def test_noalloc_matches_workspace_entry_on_calls_in_a_row():
    big, small = _cases()
    for c in (big, small):
        need = binding.workspace_size(desc_of(c), c.batch, c.heads, c.shards, c.shards, c.max_seq_len)
        assert 0 < need <= SCRATCH_BYTES, need
    dcs = [DeviceCase(big), DeviceCase(small)]
    for step, dc in enumerate([dcs[0], dcs[1], dcs[0]]):
        c = dc.case
        print(f"no-alloc call {step}: batch {c.batch} heads {c.heads} G {c.shards} {c.transform}", flush=True)
        ref_out, ref_lse = dc.decode()
        out = torch.full_like(ref_out, float("nan"))
        lse = torch.full_like(ref_lse, float("nan"))
        _noalloc(dc, out, lse)
        torch.cuda.synchronize()
        assert_parity(out.cpu().numpy(), ref_out.cpu().numpy(), "bf16", f"no-alloc call {step}")
        assert torch.equal(out, ref_out), f"call {step}: outputs differ from the workspace entry point"
        assert torch.equal(lse, ref_lse), f"call {step}: lse differs from the workspace entry point"


def test_noalloc_rejects_calls_beyond_the_scratch():
    # 4096 sequences of up to 64K tokens at 128 heads: the partials alone are far beyond 64 MiB
    desc = binding.Desc("bf16", 512, 64, 64, 1 << 20, 1024, "identity")
    need = binding.workspace_size(desc, 4096, 128, 2, 2, 65536)
    assert need > SCRATCH_BYTES
    dev = "cuda:0"
    cache = torch.empty(16, dtype=torch.bfloat16, device=dev)
    seq_lens = torch.zeros(4096, dtype=torch.int32, device=dev)
    bt = torch.zeros((4096, 1024), dtype=torch.int32, device=dev)
    q = torch.zeros((4096, 128, 512), dtype=torch.bfloat16, device=dev)
    qr = torch.zeros((4096, 128, 64), dtype=torch.bfloat16, device=dev)
    out = torch.empty((4096, 128, 512), dtype=torch.float32, device=dev)
    with pytest.raises(binding.TplaError, match="WORKSPACE_TOO_SMALL"):
        binding.tpla_decode_sharded_noalloc(desc, cache, bt, seq_lens, q, qr, 0.1, 2, 65536, out, None)
