"""GPU parity of the decode with the value up-projection fused into its merge
(tpla_decode_sharded_projected).

Checked three ways on the same seeded inputs:
* against the oracle chain -- the fp64 decode, then the fp64 per-head projection -- at the bf16
  bar (the fp32 bar for an fp32 cache);
* against the library's unfused pair (tpla_decode_sharded, then tpla_value_up_projection): the
  same sums, so only the rounding order of the merge's normaliser may differ: 1e-5 of max|ref|;
* lse against the unfused call's.
Shapes cover every wave layout of the product (d_v of 1, 96, 128, 256 and 512: one to sixteen
value tiles, four, two or one k-part), batch tiles with a ragged tail, empty and one-token
sequences, both transforms, shard subsets, the generic kernel (fp32 cache), a 1024-wide latent
(more than 64 KiB of LDS per workgroup) and the full-size paged Hadamard workload."""

import numpy as np
import pytest
import torch

import oracle
from gpu_case import DeviceCase, assert_lse, assert_parity, oracle_decode, parity, to_torch
from mla_latent_kv_13_amd import binding, inputs

pytestmark = pytest.mark.gpu

CHAIN_TOL = 1e-5

# (name, make_case kwargs, d_v, shard_begin, shard_count)
CASES = [
    ("g1_identity_contiguous", dict(batch=5, heads=32, d_latent=512, d_rope=64, shards=1, lens=[300, 0, 1, 97, 1000]),
     128, 0, None),
    ("g2_wht_paged_ragged_batch_tile", dict(batch=19, heads=64, d_latent=512, d_rope=64, shards=2,
                                            len_range=(1, 700), paged=True, page_size=64, transform="wht"),
     128, 0, None),
    ("g4_identity_paged_dv96", dict(batch=3, heads=64, d_latent=512, d_rope=64, shards=4, lens=[513, 64, 2],
                                    paged=True, page_size=16), 96, 0, None),
    ("g2_wht_second_shard_only", dict(batch=4, heads=32, d_latent=512, d_rope=64, shards=2, lens=[900, 33, 0, 64],
                                      paged=True, page_size=32, transform="wht"), 128, 1, 1),
    ("g2_identity_dv256", dict(batch=17, heads=32, d_latent=512, d_rope=64, shards=2, len_range=(0, 400)),
     256, 0, None),
    ("g1_wht_dv512", dict(batch=2, heads=32, d_latent=512, d_rope=64, shards=1, lens=[257, 31], transform="wht"),
     512, 0, None),
    ("g2_identity_dv1", dict(batch=3, heads=32, d_latent=256, d_rope=64, shards=2, lens=[100, 1, 50]), 1, 0, None),
    ("f32_cache_generic_kernel", dict(batch=3, heads=4, d_latent=64, d_rope=16, shards=2, lens=[128, 5, 0],
                                      dtype="f32"), 32, 0, None),
    ("latent_1024_g2", dict(batch=2, heads=32, d_latent=1024, d_rope=64, shards=2, lens=[300, 70]), 128, 0, None),
]


def _run(case, w, shard_begin=0, shard_count=None, **kw):
    dc = DeviceCase(case)
    wt = to_torch(w, "bf16")
    got, lse = binding.tpla_decode_sharded_projected(dc.desc, dc.pool, dc.block_table, dc.seq_lens, dc.q_lat,
                                                     dc.q_rope, case.scale, case.shards, case.max_seq_len, wt,
                                                     shard_begin=shard_begin, shard_count=shard_count, **kw)
    lat, lse_ref = dc.decode(shard_begin=shard_begin, shard_count=shard_count, **kw)
    chain = binding.tpla_value_up_projection(lat, wt)
    torch.cuda.synchronize()
    return got.cpu().numpy(), lse.cpu().numpy(), chain.cpu().numpy(), lse_ref.cpu().numpy()


@pytest.mark.parametrize("name,kw,d_v,sb,sc", CASES, ids=[c[0] for c in CASES])
def test_fused_projection_matches_oracle_chain(name, kw, d_v, sb, sc):
    print(f"case {name}", flush=True)
    seed = 900 + sum(map(ord, name)) % 97
    case = inputs.make_case(seed, **kw)
    _, w = inputs.make_value_projection(seed + 1, batch=1, heads=case.heads, d_latent=case.d_latent, d_v=d_v)
    got, lse, chain, lse_chain = _run(case, w, sb, sc)
    rel, mx = parity(got, chain)
    print(f"  fused vs unfused pair: rel L2 {rel:.2e} max {mx:.2e}; bit-equal {np.mean(got == chain):.3f}", flush=True)
    assert rel <= CHAIN_TOL and mx <= CHAIN_TOL, (name, rel, mx)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lse_chain))
    fin = np.isfinite(lse_chain)
    assert np.max(np.abs(lse[fin] - lse_chain[fin]), initial=0.0) <= 1e-5
    ref_lat, ref_lse = oracle_decode(case, shard_begin=sb, shard_count=sc)
    ref = oracle.value_up_projection(ref_lat, inputs.stored_to_f64(w, "bf16"))
    r = assert_parity(got, ref, case.dtype, f"{name}: fused projection vs oracle chain")
    print(f"  vs oracle chain: rel L2 {r[0]:.2e} max {r[1]:.2e}", flush=True)
    assert_lse(lse, ref_lse, case.dtype, name, case.transform)
    empty = case.seq_lens == 0
    assert np.all(got[empty] == 0.0), "an empty sequence projects to zero"


@pytest.mark.parametrize("cfg", [2, 5])
def test_fused_projection_full_size(cfg):
    """The full-size MLA and paged Hadamard workloads with DeepSeek-V3's value head (d_v 128):
    the whole output against the unfused pair, sampled sequences against the oracle chain."""
    print(f"workload {cfg}", flush=True)
    case = inputs.make_config(cfg, place_rows=False)
    _, w = inputs.make_value_projection(40 + cfg, batch=1, heads=case.heads, d_latent=case.d_latent, d_v=128)
    dc = DeviceCase(case, via_append=True)
    wt = to_torch(w, "bf16")
    got, lse = binding.tpla_decode_sharded_projected(dc.desc, dc.pool, dc.block_table, dc.seq_lens, dc.q_lat,
                                                     dc.q_rope, case.scale, case.shards, case.max_seq_len, wt)
    lat, lse_ref = dc.decode()
    chain = binding.tpla_value_up_projection(lat, wt)
    torch.cuda.synchronize()
    got, chain = got.cpu().numpy(), chain.cpu().numpy()
    del dc, lat
    rel, mx = parity(got, chain)
    print(f"  fused vs unfused pair: rel L2 {rel:.2e} max {mx:.2e}; bit-equal {np.mean(got == chain):.3f}", flush=True)
    assert rel <= CHAIN_TOL and mx <= CHAIN_TOL
    assert np.max(np.abs(lse.cpu().numpy() - lse_ref.cpu().numpy())) <= 1e-5
    seqs = [0, 17, case.batch - 1]
    ref_lat, _ = oracle_decode(case, seqs)
    ref = oracle.value_up_projection(ref_lat, inputs.stored_to_f64(w, "bf16"))
    r = assert_parity(got[seqs], ref, "bf16", f"workload {cfg}: sampled sequences vs oracle chain")
    print(f"  sampled vs oracle chain: rel L2 {r[0]:.2e} max {r[1]:.2e}", flush=True)


def test_fused_projection_errors():
    case = inputs.make_case(5, batch=2, heads=32, d_latent=512, d_rope=64, shards=2, lens=[10, 20])
    dc = DeviceCase(case)

    def call(w):
        return binding.tpla_decode_sharded_projected(dc.desc, dc.pool, dc.block_table, dc.seq_lens, dc.q_lat,
                                                     dc.q_rope, case.scale, case.shards, case.max_seq_len, w)

    with pytest.raises(binding.TplaError) as e:
        call(torch.zeros((32, 128, 512), dtype=torch.float32, device="cuda:0"))
    assert e.value.status == 2  # fp32 weights: the two-call path
    with pytest.raises(binding.TplaError) as e:
        call(torch.zeros((32, 513, 512), dtype=torch.bfloat16, device="cuda:0"))
    assert e.value.status == 2  # d_v above 512
    with pytest.raises(binding.TplaError) as e:
        call(torch.zeros((32, 0, 512), dtype=torch.bfloat16, device="cuda:0"))
    assert e.value.status == 1  # d_v = 0
    odd = inputs.make_case(6, batch=1, heads=4, d_latent=40, d_rope=8, shards=1, lens=[9])
    do = DeviceCase(odd)
    with pytest.raises(binding.TplaError) as e:
        binding.tpla_decode_sharded_projected(do.desc, do.pool, do.block_table, do.seq_lens, do.q_lat, do.q_rope,
                                              odd.scale, 1, odd.max_seq_len,
                                              torch.zeros((4, 8, 40), dtype=torch.bfloat16, device="cuda:0"))
    assert e.value.status == 2  # d_latent not a multiple of 16
    torch.cuda.synchronize()


def test_fused_projection_replays_from_a_hip_graph():
    """The fused call (query rotation with the tile prefix, decode kernel, merge with the projection)
    enqueues no memset, allocation or synchronisation, so it can be captured in a HIP graph: every
    replay, with eager work and synchronisations between the replays, equals the eager call bit for bit."""
    case = inputs.make_case(33, batch=20, heads=64, d_latent=512, d_rope=64, shards=2, len_range=(0, 900), paged=True,
                            page_size=64, transform="wht", scale=1.0 / np.sqrt(192))
    _, w = inputs.make_value_projection(34, batch=1, heads=64, d_latent=512, d_v=128)
    dc = DeviceCase(case)
    wt = to_torch(w, "bf16")

    def call(**kw):
        return binding.tpla_decode_sharded_projected(dc.desc, dc.pool, dc.block_table, dc.seq_lens, dc.q_lat, dc.q_rope,
                                                     case.scale, case.shards, case.max_seq_len, wt, **kw)

    eager_out, eager_lse = call()
    out, lse = torch.empty_like(eager_out), torch.empty_like(eager_lse)
    ws = binding.alloc_workspace(binding.workspace_size(dc.desc, case.batch, case.heads, 2, 2, case.max_seq_len),
                                 "cuda:0")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(out_v=out, lse=lse, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(out_v=out, lse=lse, workspace=ws)
    for _ in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager_out) and torch.equal(lse, eager_lse)
