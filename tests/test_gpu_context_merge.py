"""GPU parity of the context merge (tpla_merge_context_parts): alone against the fp64 oracle, and
after decoding disjoint parts of every sequence's context, against the oracle's decode of the whole
context (the exact context-parallel alternative)."""

import numpy as np
import pytest
import torch

import oracle
from gpu_case import DEV, DeviceCase, assert_lse, assert_parity, oracle_decode, parity
from mla_latent_kv_13_amd import binding, inputs

pytestmark = pytest.mark.gpu

# (name, parts, batch, heads, d_latent, transform, G, shard_begin, shard_count): both layouts of the
# kernel (rows rotated in registers, V values per lane; plain rows), shard subsets, parts with no
# tokens (lse -inf, about one in five), a single part.
MERGE_ALONE = [
    ("plain_g2", 3, 4, 8, 512, "identity", 2, 0, 2),
    ("plain_width_96_subset", 2, 3, 5, 96, "identity", 3, 1, 2),
    ("wht_512_g2", 4, 3, 6, 512, "wht", 2, 0, 2),
    ("wht_1024_g4_subset", 3, 2, 4, 1024, "wht", 4, 1, 2),
    ("wht_32_under_a_wave", 3, 2, 3, 32, "wht", 2, 1, 1),
    ("single_part", 1, 2, 4, 256, "wht", 1, 0, 1),
]


@pytest.mark.parametrize("name,P,B,H,d,transform,G,s0,n", MERGE_ALONE, ids=[m[0] for m in MERGE_ALONE])
def test_merge_matches_oracle(name, P, B, H, d, transform, G, s0, n):
    print(f"case {name}", flush=True)
    out_p, lse_p = inputs.make_context_parts(400 + len(name), parts=P, batch=B, heads=H, d_latent=d, shard_count=n)
    got, got_lse = binding.tpla_merge_context_parts(torch.from_numpy(out_p).to(DEV), torch.from_numpy(lse_p).to(DEV),
                                                    G, s0, transform)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.merge_context_parts(out_p, lse_p, G, s0, n, transform=transform)
    rel, mx = parity(got.cpu().numpy(), ref)
    print(f"  rel L2 {rel:.2e} max {mx:.2e}", flush=True)
    assert rel <= 1e-5 and mx <= 1e-5, (name, rel, mx)
    assert_lse(got_lse.cpu().numpy(), ref_lse, "f32", name)


def _part_inputs(case, a, e):
    """Block table and lengths of tokens [a, e) of every sequence (a, e page-aligned)."""
    ps = case.page_size
    bt = np.full_like(case.block_table, -1)
    lens = np.zeros_like(case.seq_lens)
    for b in range(case.batch):
        t1 = min(e, int(case.seq_lens[b]))
        if t1 <= a:
            continue
        pages = (t1 - a + ps - 1) // ps
        bt[b, :pages] = case.block_table[b, a // ps:a // ps + pages]
        lens[b] = t1 - a
    return torch.from_numpy(bt).to(DEV), torch.from_numpy(lens).to(DEV), int(max(1, lens.max()))


@pytest.mark.parametrize("transform,G,s0,n", [("identity", 1, 0, 1), ("wht", 2, 0, 2), ("identity", 4, 1, 2)])
def test_split_context_decode_then_merge(transform, G, s0, n):
    """Tokens [0, 256), [256, 256) (empty), [256, 640), [640, end) of each sequence decoded as four
    parts, merged, against the oracle's decode of the whole context; and against the library's own
    whole-context decode."""
    case = inputs.make_case(23, batch=4, heads=64, d_latent=512, d_rope=64, shards=G, lens=[1000, 300, 0, 257],
                            paged=True, page_size=64, transform=transform, scale=1.0 / np.sqrt(192))
    dc = DeviceCase(case)
    cuts = [(0, 256), (256, 256), (256, 640), (640, case.max_seq_len)]
    outs, lses = [], []
    for a, e in cuts:
        bt, lens, max_len = _part_inputs(case, a, e)
        o, l = binding.tpla_decode_sharded(dc.desc, dc.pool, bt, lens, dc.q_lat, dc.q_rope, case.scale, G, max_len,
                                           shard_begin=s0, shard_count=n)
        outs.append(o)
        lses.append(l)
    got, got_lse = binding.tpla_merge_context_parts(torch.stack(outs), torch.stack(lses), G, s0, transform)
    whole, whole_lse = dc.decode(shard_begin=s0, shard_count=n)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_decode(case, shard_begin=s0, shard_count=n)
    assert_parity(got.cpu().numpy(), ref, "bf16", f"merged parts ({transform}, G={G})")
    assert_lse(got_lse.cpu().numpy(), ref_lse, "bf16", f"merged parts ({transform}, G={G})", transform)
    rel, _ = parity(got.cpu().numpy(), whole.cpu().numpy())
    assert rel < 5e-3, rel  # two bf16-weighted decodes of the same context
    assert np.array_equal(np.isneginf(got_lse.cpu().numpy()), np.isneginf(whole_lse.cpu().numpy()))
