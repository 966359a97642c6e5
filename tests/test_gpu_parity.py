"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle on the same seeded inputs."""

import numpy as np
import pytest
import torch

from gpu_case import DeviceCase, assert_lse, assert_parity, oracle_decode, oracle_decode_grouped, parity
from mla_latent_kv_13_amd import binding, inputs

pytestmark = pytest.mark.gpu


def _np(t):
    return None if t is None else t.detach().float().cpu().numpy()


def _say(msg):
    print(msg, flush=True)


# (name, make_case kwargs, decode kwargs) -- small enough for the oracle, several 32-token
# tiles, ragged tails, empty and single-token sequences, both layouts, both transforms.
SMALL = [
    ("g1_h128_contig", dict(batch=4, heads=128, shards=1, lens=[1000, 1, 64, 333]), {}),
    ("g1_h128_chunk64", dict(batch=3, heads=128, shards=1, lens=[700, 0, 129]), dict(chunk_tokens=64)),
    ("g2_h128_contig", dict(batch=4, heads=128, shards=2, lens=[777, 32, 0, 2049]), dict(chunk_tokens=128)),
    ("g2_h128_paged_wht", dict(batch=3, heads=128, shards=2, lens=[3000, 1, 700], paged=True, page_size=64,
                               transform="wht", extra_pages=5), {}),
    ("g4_h64_contig", dict(batch=3, heads=64, shards=4, lens=[1500, 65, 31], channel_sigma=0.5), {}),
    ("g4_h64_paged", dict(batch=2, heads=64, shards=4, lens=[513, 2000], paged=True, page_size=64), dict(chunk_tokens=256)),
    ("g4_h128_contig", dict(batch=2, heads=128, shards=4, lens=[900, 70]), {}),
    ("g4_h128_paged32", dict(batch=2, heads=128, shards=4, lens=[1300, 33], paged=True, page_size=32), {}),
    ("g4_h32_paged8", dict(batch=3, heads=32, shards=4, lens=[400, 9, 64], paged=True, page_size=8), {}),
    ("g2_h32_paged_wht_chunk64", dict(batch=3, heads=32, shards=2, lens=[900, 100, 5], paged=True, page_size=16,
                                      transform="wht"), dict(chunk_tokens=64)),
    ("g1_h96_paged", dict(batch=2, heads=96, shards=1, lens=[300, 41], paged=True, page_size=32), {}),
    ("g2_h128_generic_kernel", dict(batch=2, heads=128, shards=2, lens=[260, 77]), dict(kernel="generic")),
    ("odd_shape_generic_bf16", dict(batch=3, heads=3, d_latent=64, d_rope=16, shards=2, lens=[50, 0, 130]), {}),
    ("odd_shape_generic_g1_wht", dict(batch=2, heads=5, d_latent=128, d_rope=8, shards=1, lens=[40, 9],
                                      transform="wht", paged=True, page_size=8), {}),
    ("f32_g2_wht_paged", dict(batch=2, heads=4, d_latent=64, d_rope=16, shards=2, lens=[200, 17], dtype="f32",
                              transform="wht", paged=True, page_size=16), {}),
    ("zero_scale_uniform_weights", dict(batch=2, heads=128, shards=2, lens=[100, 33], scale=0.0), {}),
    ("negative_scale", dict(batch=2, heads=64, shards=4, lens=[250, 64], scale=-0.1), {}),
    ("single_tile_and_one_token", dict(batch=3, heads=128, shards=1, lens=[32, 1, 31]), {}),
    ("more_than_64_chunks", dict(batch=2, heads=32, shards=2, lens=[5000, 4100]), dict(chunk_tokens=64)),
    # eight and sixteen shards: 64- and 32-wide slices (the generic kernel), plain and rotated
    ("g8_w64_generic", dict(batch=2, heads=16, shards=8, lens=[333, 65]), {}),
    ("g16_w32_generic_wht", dict(batch=2, heads=8, shards=16, lens=[200, 31], transform="wht", paged=True,
                                 page_size=16), {}),
    # 256 heads: two 128-head groups at w = 256, four 64-head groups at w = 512
    ("g2_h256_two_head_groups", dict(batch=2, heads=256, shards=2, lens=[700, 90]), {}),
    ("g1_h256_four_head_groups_paged", dict(batch=2, heads=256, shards=1, lens=[400, 129], paged=True,
                                            page_size=32), {}),
    # Hadamard row widths 256 and 1024 (4 and 16 values per lane) and 32 (fp32, half the lanes idle)
    ("g2_wht_dl256", dict(batch=2, heads=64, d_latent=256, shards=2, lens=[300, 45], transform="wht"), {}),
    ("g4_wht_dl1024_paged", dict(batch=2, heads=32, d_latent=1024, shards=4, lens=[200, 70], transform="wht",
                                 paged=True, page_size=32), {}),
    ("f32_wht_dl32", dict(batch=2, heads=3, d_latent=32, d_rope=8, shards=2, lens=[40, 7], dtype="f32",
                          transform="wht"), {}),
    # Rows growing 8-fold along each sequence: later tiles' logits exceed the first tile's maximum
    # by 12-26 (base 2), so the running maximum is raised mid-segment (O and l rescaled) on every
    # tile width, and the 128-wide slices refit tiles whose weights would overflow
    ("g4_h64_rising_logits", dict(batch=2, heads=64, shards=4, lens=[1500, 300], token_gain=8.0), {}),
    ("g4_h128_rising_logits_balanced", dict(batch=3, heads=128, shards=4, lens=[900, 40, 2100], token_gain=8.0),
     dict(schedule="balanced")),
    ("g2_h128_rising_logits_paged_wht", dict(batch=2, heads=128, shards=2, lens=[2000, 200], paged=True, page_size=64,
                                             transform="wht", token_gain=8.0), {}),
    ("g1_h128_rising_logits", dict(batch=2, heads=128, shards=1, lens=[1200, 90], token_gain=8.0),
     dict(chunk_tokens=512)),
    ("g2_h32_rising_logits_generic", dict(batch=2, heads=32, shards=2, lens=[700, 64], token_gain=8.0),
     dict(kernel="generic")),
    # page sizes that are not powers of two: page and offset of a token by division, on every kernel
    ("g2_h128_paged48", dict(batch=3, heads=128, shards=2, lens=[700, 47, 1000], paged=True, page_size=48), {}),
    ("g4_h64_paged96_balanced", dict(batch=3, heads=64, shards=4, lens=[500, 96, 1], paged=True, page_size=96),
     dict(schedule="balanced")),
    ("g1_h128_paged100_wht", dict(batch=2, heads=128, shards=1, lens=[640, 99], paged=True, page_size=100,
                                  transform="wht"), {}),
    ("f32_g2_paged24_generic", dict(batch=2, heads=4, d_latent=64, d_rope=16, shards=2, lens=[100, 23], dtype="f32",
                                    paged=True, page_size=24), {}),
]


@pytest.mark.parametrize("name,kw,dkw", SMALL, ids=[s[0] for s in SMALL])
def test_small_cases_match_oracle(name, kw, dkw):
    _say(f"case {name}")
    args = dict(d_latent=512, d_rope=64, dtype="bf16", scale=1.0 / np.sqrt(192))
    args.update(kw)
    case = inputs.make_case(100 + len(name), name=name, **args)
    dc = DeviceCase(case)
    out, lse = dc.decode(**dkw)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_decode(case)
    rel, mx = assert_parity(_np(out), ref_out, case.dtype, name)
    assert_lse(_np(lse), ref_lse, case.dtype, name, case.transform)
    _say(f"  rel L2 {rel:.2e} max {mx:.2e}")


def test_config1_tiny_fp32():
    case = inputs.make_config(1)
    dc = DeviceCase(case)
    out, lse = dc.decode()
    ref_out, ref_lse = oracle_decode(case)
    assert_parity(_np(out), ref_out, "f32", "config 1")
    assert_lse(_np(lse), ref_lse, "f32", "config 1")


def test_shard_subsets_are_additive_and_match_oracle():
    case = inputs.make_case(7, batch=3, heads=64, d_latent=512, d_rope=64, shards=4, lens=[600, 3, 250],
                            paged=True, page_size=64, transform="wht", scale=1.0 / np.sqrt(192))
    dc = DeviceCase(case)
    full, full_lse = dc.decode()
    acc = torch.zeros_like(full)
    for s in range(4):
        part, part_lse = dc.decode(shard_begin=s, shard_count=1)
        ref, ref_lse = oracle_decode(case, shard_begin=s, shard_count=1)
        assert_parity(_np(part), ref, "bf16", f"shard {s}")
        assert_lse(_np(part_lse), ref_lse, "bf16", f"shard {s}", "wht")
        assert torch.equal(part_lse[:, 0], full_lse[:, s])
        acc += part
    rel, mx = parity(_np(acc), _np(full))
    assert rel < 1e-6 and mx < 1e-6
    mid, _ = dc.decode(shard_begin=1, shard_count=2)
    ref, _ = oracle_decode(case, shard_begin=1, shard_count=2)
    assert_parity(_np(mid), ref, "bf16", "shards 1-2")


def test_shard_subset_without_rotation_leaves_other_columns_zero():
    case = inputs.make_case(8, batch=2, heads=128, d_latent=512, d_rope=64, shards=2, lens=[300, 90])
    dc = DeviceCase(case)
    out, _ = dc.decode(shard_begin=1, shard_count=1)
    out = _np(out)
    assert np.all(out[:, :, :256] == 0.0)
    ref, _ = oracle_decode(case, shard_begin=1, shard_count=1)
    assert_parity(out, ref, "bf16", "shard 1")


def test_mla_entry_point_equals_single_shard_call():
    case = inputs.make_case(9, batch=2, heads=128, d_latent=512, d_rope=64, shards=1, lens=[400, 1000],
                            scale=1.0 / np.sqrt(192))
    dc = DeviceCase(case)
    a, a_lse = dc.decode()
    b, b_lse = binding.mla_decode_absorbed(dc.desc, dc.pool, None, dc.seq_lens, dc.q_lat, dc.q_rope, case.scale,
                                           case.max_seq_len)
    assert torch.equal(a, b) and torch.equal(a_lse[:, 0], b_lse)


def test_bitwise_deterministic():
    case = inputs.make_case(10, batch=3, heads=128, d_latent=512, d_rope=64, shards=2, lens=[2000, 513, 64],
                            paged=True, page_size=64, transform="wht")
    dc = DeviceCase(case)
    first, first_lse = dc.decode()
    for _ in range(9):
        again, again_lse = dc.decode()
        assert torch.equal(first, again) and torch.equal(first_lse, again_lse)


LAYOUTS = [
    # (name, case kwargs, dtype, call kwargs): page sizes 64 (whole tiles per page) and 16 (tiles
    # straddle pages), against the contiguous layout of the same seeded rows
    ("g2_wht_chunked", dict(heads=128, shards=2, transform="wht"), "bf16", dict(schedule="chunked", chunk_tokens=512)),
    ("g2_wht_balanced", dict(heads=128, shards=2, transform="wht"), "bf16", dict(schedule="balanced")),
    ("g1_identity_chunked", dict(heads=64, shards=1), "bf16", dict(schedule="chunked", chunk_tokens=256)),
    ("g4_identity_balanced", dict(heads=64, shards=4), "bf16", dict(schedule="balanced")),
    ("generic_f32", dict(heads=4, shards=2, d_latent=64, d_rope=16), "f32", dict(chunk_tokens=256)),
]


@pytest.mark.parametrize("name,kw,dtype,call", LAYOUTS, ids=[x[0] for x in LAYOUTS])
def test_paged_and_contiguous_layouts_agree_bitwise(name, kw, dtype, call):
    """The same seeded rows stored contiguously and in permuted pages (NaN-filled spare pages) give
    the same bits: the layout changes where a row is read from, never the arithmetic."""
    base = dict(batch=4, d_latent=512, d_rope=64, lens=[1500, 33, 0, 700], dtype=dtype)
    base.update(kw)
    outs = []
    for paged, page_size in ((False, 64), (True, 64), (True, 16)):
        case = inputs.make_case(14, paged=paged, page_size=page_size, extra_pages=2 if paged else 0,
                                name=f"{name}-{paged}-{page_size}", **base)
        out, lse = DeviceCase(case).decode(**call)
        torch.cuda.synchronize()
        outs.append((out.cpu(), lse.cpu()))
    ref, ref_lse = oracle_decode(case)
    assert_parity(outs[0][0].numpy(), ref, dtype, name)
    for out, lse in outs[1:]:
        assert torch.equal(out, outs[0][0]) and torch.equal(lse, outs[0][1])


def test_calls_on_two_streams_at_once():
    """The library keeps no state between calls: calls enqueued on two streams at once, each with its
    own outputs and workspace (a paged rotated G = 2 decode with the balanced schedule, a contiguous
    G = 1 decode with chunks), give the same bits as the same calls one after the other."""
    ca = inputs.make_case(12, batch=4, heads=128, d_latent=512, d_rope=64, shards=2, lens=[3000, 70, 0, 1500],
                          paged=True, page_size=64, transform="wht", extra_pages=2)
    cb = inputs.make_case(13, batch=3, heads=64, d_latent=512, d_rope=64, shards=1, lens=[2048, 1, 777])
    da, db = DeviceCase(ca), DeviceCase(cb)
    ref_a, ref_b = da.decode(), db.decode()
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    sa.wait_stream(torch.cuda.current_stream())
    sb.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        with torch.cuda.stream(sa):
            oa = da.decode()
        with torch.cuda.stream(sb):
            ob = db.decode()
        outs.append((oa, ob))
    torch.cuda.synchronize()
    for oa, ob in outs:
        assert torch.equal(oa[0], ref_a[0]) and torch.equal(oa[1], ref_a[1])
        assert torch.equal(ob[0], ref_b[0]) and torch.equal(ob[1], ref_b[1])


BALANCED = [
    ("contig_ragged_g2", dict(batch=5, heads=128, shards=2, lens=[1000, 0, 1, 4097, 33])),
    ("paged_ragged_g1", dict(batch=4, heads=128, shards=1, lens=[2500, 31, 0, 700], paged=True, page_size=64,
                             extra_pages=3)),
    ("paged16_ragged_g4_wht", dict(batch=3, heads=64, shards=4, lens=[900, 64, 3], paged=True, page_size=16,
                                   transform="wht")),
    ("more_workers_than_tiles", dict(batch=6, heads=32, shards=1, lens=[5, 0, 40, 1, 0, 70])),
    ("all_empty", dict(batch=3, heads=64, shards=2, lens=[0, 0, 0])),
]


@pytest.mark.parametrize("name,kw", BALANCED, ids=[b[0] for b in BALANCED])
def test_balanced_and_chunked_schedules_match_oracle(name, kw):
    """Both work schedules of the MFMA kernel on ragged batches (empty, single-token, multi-page
    sequences; shares of tiles crossing sequence boundaries) against the oracle."""
    _say(f"case {name}")
    args = dict(d_latent=512, d_rope=64, dtype="bf16", scale=1.0 / np.sqrt(192))
    args.update(kw)
    case = inputs.make_case(300 + len(name), name=name, **args)
    dc = DeviceCase(case)
    ref_out, ref_lse = oracle_decode(case)
    outs = {}
    for sched in ("chunked", "balanced"):
        out, lse = dc.decode(schedule=sched, chunk_tokens=128 if sched == "chunked" else 0)
        torch.cuda.synchronize()
        assert_parity(_np(out), ref_out, "bf16", f"{name} {sched}")
        assert_lse(_np(lse), ref_lse, "bf16", f"{name} {sched}", case.transform)
        outs[sched] = _np(out)
    rel, _ = parity(outs["balanced"], outs["chunked"])
    assert rel < 5e-3


def test_split_count_invariance():
    case = inputs.make_case(11, batch=2, heads=128, d_latent=512, d_rope=64, shards=2, lens=[4096, 1500])
    dc = DeviceCase(case)
    ref, ref_lse = oracle_decode(case)
    outs = []
    for ct in (64, 512, 4096):
        out, lse = dc.decode(chunk_tokens=ct)
        assert_parity(_np(out), ref, "bf16", f"chunk {ct}")
        assert_lse(_np(lse), ref_lse, "bf16", f"chunk {ct}")
        outs.append(_np(out))
    rel, _ = parity(outs[0], outs[2])
    assert rel < 5e-3


def test_append_matches_oracle_rounding():
    import oracle

    case = inputs.make_case(12, batch=2, heads=4, d_latent=512, d_rope=64, shards=2, lens=[300, 200], paged=True,
                            page_size=64, transform="wht", extra_pages=2)
    dc = DeviceCase(case)
    got = inputs.stored_to_f64(dc.pool.view(torch.int16).cpu().numpy().view(np.uint16), "bf16")
    flat = got.reshape(-1, case.width)
    raw = inputs.stored_to_f64(case.rows, "bf16")
    empty = np.full((1, case.rows.shape[0], case.width), np.nan)
    ref = oracle.latent_cache_append(empty, raw, np.arange(case.rows.shape[0]), 512, "wht", "bf16")[0]
    mine = flat[case.slots]
    ulp = np.ldexp(1.0, np.frexp(ref[:, :512])[1] - 8)
    assert np.all(np.abs(mine[:, :512] - ref[:, :512]) <= ulp)
    assert np.mean(mine[:, :512] == ref[:, :512]) > 0.99
    assert np.array_equal(mine[:, 512:], raw[:, 512:])
    untouched = np.ones(flat.shape[0], dtype=bool)
    untouched[case.slots] = False
    assert np.all(np.isnan(flat[untouched]))


def test_errors_surface_as_status():
    case = inputs.make_case(13, batch=2, heads=3, d_latent=64, d_rope=16, shards=2, lens=[10, 20])
    dc = DeviceCase(case)
    with pytest.raises(binding.TplaError, match="UNSUPPORTED"):
        dc.decode(kernel="mfma")
    small = torch.empty(16, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(binding.TplaError, match="WORKSPACE_TOO_SMALL"):
        dc.decode(workspace=small)
    with pytest.raises(binding.TplaError, match="INVALID_ARGUMENT"):
        dc.decode(shard_begin=1, shard_count=2)


# Full-size workloads in the launch configuration the benchmark times, compared with the oracle
# over the whole output (every sequence, head and column) at the bf16 bar.  The plain caches are
# written by the library's own append (a plain copy), as the rotated one is; the oracle builds its
# caches from the raw rows.  The paged workload's 64 sequences are checked in four groups of 16
# after one decode, so that each test stays within a couple of minutes of oracle time.
_full_cache = {}


def _full_decode(cfg):
    if cfg not in _full_cache:
        _full_cache.clear()
        torch.cuda.empty_cache()
        _say(f"config {cfg}: generating")
        case = inputs.make_config(cfg, place_rows=False)
        dc = DeviceCase(case, via_append=True)
        _say(f"config {cfg}: decoding")
        out, lse = dc.decode()
        torch.cuda.synchronize()
        _full_cache[cfg] = (case, _np(out), _np(lse))
        del dc, out, lse
    return _full_cache[cfg]


FULL = [(2, None), (3, None), (4, None)] + [(5, (k * 16, (k + 1) * 16)) for k in range(4)]


@pytest.mark.parametrize("cfg,rng", FULL, ids=[f"c{c}" + (f"_seq{r[0]}-{r[1] - 1}" if r else "_all") for c, r in FULL])
def test_full_size_workloads_whole_output(cfg, rng):
    case, out_np, lse_np = _full_decode(cfg)
    seqs = list(range(case.batch)) if rng is None else list(range(*rng))
    assert np.all(np.isfinite(out_np[seqs])) and np.all(np.isfinite(lse_np[seqs]))
    _say(f"config {cfg}: oracle on sequences {seqs[0]}..{seqs[-1]}")
    ref, ref_lse = oracle_decode_grouped(case, seqs)
    rel, mx = assert_parity(out_np[seqs], ref, "bf16", f"config {cfg}")
    assert_lse(lse_np[seqs], ref_lse, "bf16", f"config {cfg}", case.transform)
    _say(f"config {cfg}: rel L2 {rel:.2e} max {mx:.2e}")


# Long contexts: a 17-token sequence beside one of 1,000,003 tokens (a ragged last tile).  In
# the contiguous layout the long sequence owns page 1 of the pool, so its rows lie 1.15 to 2.3 GB
# into it (past 2^31 bytes from token 864,133 on); with 1-row pages every token sits on a page of
# its own and the balanced schedule needs over a thousand workers.  Four tokens of the long
# sequence are replaced by one head's own query, which then dominates that head's softmax: a
# lost, doubled or misplaced row moves that head's output by far more than the tolerance.
LONG_LENS = [17, 1_000_003]
LONG_PLANTS = [(0, 0), (524_287, 38), (900_000, 63), (1_000_002, 13)]  # (token, head)
LONG_HEADS = [0, 7, 13, 38, 63]
LONG_LAYOUTS = {"contig": dict(paged=False), "paged64": dict(paged=True, page_size=64),
                "paged1": dict(paged=True, page_size=1)}
LONG = [("contig", 1, {}), ("contig", 2, {}), ("contig", 4, {}), ("contig", 2, dict(schedule="balanced")),
        ("contig", 2, dict(kernel="generic")), ("paged64", 2, {}), ("paged64", 4, dict(schedule="chunked")),
        ("paged1", 2, {})]
_long_cache = {}


def _plant(case, b, picks):
    """Set token t of sequence b to head h's own query (same stored type), for (t, h) in picks."""
    start = int(case.seq_lens[:b].astype(np.int64).sum())
    flat = case.pool.reshape(-1, case.width)
    for t, h in picks:
        i = start + t
        case.rows[i, :case.d_latent] = case.q_lat[b, h]
        case.rows[i, case.d_latent:] = case.q_rope[b, h]
        flat[case.slots[i]] = case.rows[i]


def _long_case(layout):
    if layout not in _long_cache:
        _long_cache.clear()  # one layout's host and device copies at a time
        torch.cuda.empty_cache()
        _say(f"long {layout}: generating")
        case = inputs.make_case(1234, batch=2, heads=64, d_latent=512, d_rope=64, shards=2, lens=LONG_LENS,
                                scale=1.0 / np.sqrt(192), name=f"long-{layout}", **LONG_LAYOUTS[layout])
        _plant(case, 1, LONG_PLANTS)
        _long_cache[layout] = (case, DeviceCase(case))
    return _long_cache[layout]


@pytest.mark.parametrize("layout,g,dkw", LONG, ids=[f"{l}_g{g}_{'_'.join(d.values()) or 'auto'}" for l, g, d in LONG])
def test_million_token_context_sampled(layout, g, dkw):
    import dataclasses
    base, dc = _long_case(layout)
    case = dataclasses.replace(base, shards=g)
    dc.case = case
    _say(f"long {layout} G={g} {dkw}: decoding")
    out, lse = dc.decode(**dkw)
    torch.cuda.synchronize()
    out_np, lse_np = _np(out), _np(lse)
    assert np.all(np.isfinite(out_np)) and np.all(np.isfinite(lse_np))
    _say(f"long {layout} G={g}: oracle")
    ref, ref_lse = oracle_decode(case, [0])
    assert_parity(out_np[[0]], ref, "bf16", f"long {layout} G={g} short sequence")
    assert_lse(lse_np[[0]], ref_lse, "bf16", f"long {layout} G={g} short sequence")
    ref, ref_lse = oracle_decode(case, [1], heads=LONG_HEADS)
    for k, h in enumerate(LONG_HEADS):
        rel, mx = assert_parity(out_np[1, h], ref[0, k], "bf16", f"long {layout} G={g} head {h}")
        _say(f"  head {h}: rel L2 {rel:.2e} max {mx:.2e}")
    assert_lse(lse_np[1][:, LONG_HEADS], ref_lse[0], "bf16", f"long {layout} G={g} long sequence")


def test_decode_call_replays_from_a_hip_graph():
    """A decode call (query rotation, tile-prefix scan, decode kernel, merge) enqueues no memset,
    allocation or synchronisation, so it can be captured in a HIP graph; every replay, with eager
    work and synchronisations between replays, equals the eager call bit for bit."""
    case = inputs.make_case(31, batch=3, heads=64, d_latent=512, d_rope=64, shards=2, lens=[900, 1, 300], paged=True,
                            page_size=64, transform="wht", scale=1.0 / np.sqrt(192))
    dc = DeviceCase(case)
    eager_out, eager_lse = dc.decode()
    out, lse = torch.empty_like(eager_out), torch.empty_like(eager_lse)
    ws = binding.alloc_workspace(binding.workspace_size(dc.desc, case.batch, case.heads, 2, 2, case.max_seq_len),
                                 "cuda:0")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dc.decode(out=out, lse=lse, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dc.decode(out=out, lse=lse, workspace=ws)
    for _ in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager_out) and torch.equal(lse, eager_lse)


def test_five_thousand_short_ragged_sequences():
    """Many short sequences (0..40 tokens, 64-token pages): the tile-prefix scan over 5000 lengths,
    worker shares crossing hundreds of sequence boundaries, a 5000-row merge grid."""
    case = inputs.make_case(41, batch=5000, heads=32, d_latent=512, d_rope=64, shards=2, len_range=(0, 40),
                            paged=True, page_size=64, scale=1.0 / np.sqrt(192))
    dc = DeviceCase(case)
    ref, ref_lse = oracle_decode(case)
    for sched in ("balanced", "chunked"):
        out, lse = dc.decode(schedule=sched)
        torch.cuda.synchronize()
        rel, mx = assert_parity(_np(out), ref, "bf16", f"5000 sequences, {sched}")
        assert_lse(_np(lse), ref_lse, "bf16", f"5000 sequences, {sched}")
        _say(f"5000 sequences {sched}: rel L2 {rel:.2e} max {mx:.2e}")
