"""GPU parity of the absorbed MLA prefill (mla_prefill_absorbed) against the fp64 oracle: every new
token attends to its causal prefix of the cache.  Both kernels, both schedules, contiguous and
paged caches, the Hadamard-rotated cache, fresh prompts and continued contexts, sequences without
new tokens, rows with no visible token, and sampled rows of a full-size chunked-prefill step."""

import numpy as np
import pytest
import torch

import oracle
from gpu_case import DEV, DeviceCase, assert_lse, assert_parity, oracle_pool, to_torch
from mla_latent_kv_13_amd import binding, inputs

pytestmark = pytest.mark.gpu


def _queries(case, seed, new):
    query_start, q_lat, q_rope = inputs.make_prefill_queries(seed, new_tokens=new, heads=case.heads,
                                                             d_latent=case.d_latent, d_rope=case.d_rope,
                                                             dtype=case.dtype)
    return query_start, q_lat, q_rope


def _prefill(dc, query_start, q_lat, q_rope, **kw):
    c = dc.case
    return binding.mla_prefill_absorbed(dc.desc, dc.pool, dc.block_table, dc.seq_lens,
                                        torch.from_numpy(query_start).to(DEV), to_torch(q_lat, c.dtype),
                                        to_torch(q_rope, c.dtype), c.scale, c.max_seq_len, **kw)


def _oracle(case, query_start, q_lat, q_rope):
    pool, lens = oracle_pool(case, list(range(case.batch)))
    return oracle.mla_prefill_absorbed(pool, None, lens, query_start, inputs.stored_to_f64(q_lat, case.dtype),
                                       inputs.stored_to_f64(q_rope, case.dtype), float(np.float32(case.scale)),
                                       transform=case.transform)


# (name, case kwargs, new tokens per sequence, call kwargs)
CASES = [
    ("dsv3_contiguous_continue_and_fresh",
     dict(batch=3, heads=128, d_latent=512, d_rope=64, lens=[700, 300, 64]), [40, 300, 1], {}),
    ("dsv3_paged_wht_balanced",
     dict(batch=3, heads=128, d_latent=512, d_rope=64, lens=[1000, 513, 90], paged=True, page_size=64,
          transform="wht", extra_pages=2), [70, 0, 90], {}),
    ("dsv3_paged_wht_chunked",
     dict(batch=3, heads=128, d_latent=512, d_rope=64, lens=[1000, 513, 90], paged=True, page_size=64,
          transform="wht", extra_pages=2), [70, 0, 90], dict(schedule="chunked")),
    ("h64_pages_of_16",
     dict(batch=2, heads=64, d_latent=512, d_rope=64, lens=[200, 37], paged=True, page_size=16, extra_pages=1),
     [33, 37], {}),
    ("generic_kernel_f32",
     dict(batch=2, heads=4, d_latent=64, d_rope=16, lens=[100, 5], dtype="f32"), [20, 5], {}),
    ("generic_kernel_bf16_wht",
     dict(batch=2, heads=3, d_latent=64, d_rope=8, lens=[130, 17], transform="wht"), [9, 17], {}),
    ("rows_without_prefix",
     dict(batch=2, heads=32, d_latent=512, d_rope=64, lens=[2, 10]), [3, 4], {}),
]


@pytest.mark.parametrize("name,kw,new,call", CASES, ids=[c[0] for c in CASES])
def test_prefill_matches_oracle(name, kw, new, call):
    print(f"case {name}", flush=True)
    scale = 1.0 / np.sqrt(192) if kw["d_latent"] == 512 else 1.0 / np.sqrt(kw["d_latent"] + kw["d_rope"])
    case = inputs.make_case(500 + len(name), shards=1, scale=scale, name=name, **kw)
    dc = DeviceCase(case)
    query_start, q_lat, q_rope = _queries(case, 600 + len(name), new)
    out, lse = _prefill(dc, query_start, q_lat, q_rope, **call)
    torch.cuda.synchronize()
    ref, ref_lse = _oracle(case, query_start, q_lat, q_rope)
    got = out.cpu().numpy()
    rel, mx = assert_parity(got, ref, case.dtype, name)
    print(f"  rel L2 {rel:.2e} max {mx:.2e}", flush=True)
    assert_lse(lse.cpu().numpy(), ref_lse, case.dtype, name, case.transform)
    empty = np.all(np.isneginf(ref_lse), axis=1)
    assert np.all(got[empty] == 0.0)


def test_last_new_token_is_the_decode_of_the_whole_sequence():
    """The last new token of every sequence sees the whole cache: its row is the decode result of
    that token's query (the library's decode call on the same cache, same bar against each other)."""
    case = inputs.make_case(77, batch=3, heads=128, d_latent=512, d_rope=64, shards=1, lens=[900, 65, 300],
                            paged=True, page_size=64, transform="wht", scale=1.0 / np.sqrt(192), extra_pages=1)
    dc = DeviceCase(case)
    new = [10, 65, 1]
    query_start, q_lat, q_rope = _queries(case, 78, new)
    out, lse = _prefill(dc, query_start, q_lat, q_rope)
    last = query_start[1:] - 1
    dec, dec_lse = binding.mla_decode_absorbed(dc.desc, dc.pool, dc.block_table, dc.seq_lens,
                                               to_torch(q_lat[last], "bf16"), to_torch(q_rope[last], "bf16"),
                                               case.scale, case.max_seq_len)
    torch.cuda.synchronize()
    got, want = out.cpu().numpy()[last], dec.cpu().numpy()
    rel = np.linalg.norm(got - want) / np.linalg.norm(want)
    assert rel < 5e-3, rel
    assert np.max(np.abs(lse.cpu().numpy()[last] - dec_lse.cpu().numpy())) < 1e-2


def test_full_size_chunked_prefill_step_sampled():
    """The prefill workload the benchmark times (4 sequences of 4096 cached tokens whose last 1024
    are new, 128 heads, paged 64-token pages, Hadamard-rotated cache), in the benchmark's launch
    configuration; sampled rows against the oracle one by one, and every row finite."""
    case = inputs.make_case(91, batch=4, heads=128, d_latent=512, d_rope=64, shards=1, lens=4096, paged=True,
                            page_size=64, transform="wht", scale=1.0 / np.sqrt(192), name="prefill-4x1024-of-4096")
    dc = DeviceCase(case)
    new = [1024] * 4
    query_start, q_lat, q_rope = _queries(case, 92, new)
    print("prefill 4 x 1024 new of 4096", flush=True)
    out, lse = _prefill(dc, query_start, q_lat, q_rope)
    torch.cuda.synchronize()
    got, got_lse = out.cpu().numpy(), lse.cpu().numpy()
    assert np.all(np.isfinite(got)) and np.all(np.isfinite(got_lse))
    rng = np.random.default_rng(93)
    rows = sorted({0, 1023, 1024, 4095, *rng.integers(0, 4096, size=4).tolist()})
    pools = {}
    for r in rows:
        b = int(np.searchsorted(query_start, r, side="right") - 1)
        j = r - int(query_start[b])
        visible = int(case.seq_lens[b]) - new[b] + j + 1
        if b not in pools:
            pools[b] = oracle_pool(case, [b])[0]
        ref, ref_lse = oracle.mla_prefill_absorbed(pools[b], None, [visible], [0, 1],
                                                   inputs.stored_to_f64(q_lat[r:r + 1], "bf16"),
                                                   inputs.stored_to_f64(q_rope[r:r + 1], "bf16"),
                                                   float(np.float32(case.scale)), transform="wht")
        assert_parity(got[r:r + 1], ref, "bf16", f"row {r}")
        assert_lse(got_lse[r:r + 1], ref_lse, "bf16", f"row {r}", "wht")


@pytest.mark.parametrize("transform", ["wht", "identity"])
def test_prefill_rows_finished_whole_and_merged(transform):
    """Under the balanced schedule a row whose tiles all fall in one workgroup's share is finished by
    the decode kernel itself (normalised, rotated back, written), and the merge combines the others.
    One sequence gives a single row over 20,000 tokens, longer than any share, so it is split and
    merged; the other gives 400 short rows, most of them inside one share.  Every row against the
    oracle, and the chunked schedule (every row merged) on the same inputs against it too."""
    case = inputs.make_case(131, batch=2, heads=64, d_latent=512, d_rope=64, shards=1, lens=[20000, 400],
                            paged=True, page_size=64, transform=transform, scale=1.0 / np.sqrt(192), extra_pages=1,
                            name=f"prefill-whole-and-split-{transform}")
    dc = DeviceCase(case)
    query_start, q_lat, q_rope = _queries(case, 132, [1, 400])
    ref, ref_lse = _oracle(case, query_start, q_lat, q_rope)
    for schedule in ("balanced", "chunked"):
        print(f"prefill {transform} {schedule}", flush=True)
        out, lse = _prefill(dc, query_start, q_lat, q_rope, schedule=schedule)
        torch.cuda.synchronize()
        assert_parity(out.cpu().numpy(), ref, "bf16", f"{transform} {schedule}")
        assert_lse(lse.cpu().numpy(), ref_lse, "bf16", f"{transform} {schedule}", transform)


def _random_prefill(i):
    rng = np.random.default_rng([4241, i])
    dtype = "f32" if rng.random() < 0.15 else "bf16"
    if dtype == "bf16" and rng.random() < 0.7:  # shapes the matrix-core kernel takes
        d_latent, d_rope, heads = 512, 64, int(32 * rng.integers(1, 5))
    else:
        d_latent, d_rope, heads = int(rng.choice([64, 128, 256])), int(rng.choice([8, 16, 32])), int(rng.integers(1, 9))
    batch = int(rng.integers(1, 6))
    lens = [int(x) for x in rng.integers(0, 700, size=batch)]
    new = []
    for t in lens:
        u = rng.random()
        new.append(t if u < 0.25 else (0 if u < 0.35 else (t + 2 if u < 0.4 else int(rng.integers(0, t + 1)))))
    paged = bool(rng.random() < 0.6)
    kw = dict(batch=batch, heads=heads, d_latent=d_latent, d_rope=d_rope, shards=1, lens=lens, dtype=dtype,
              paged=paged, page_size=int(rng.choice([1, 8, 16, 32, 64])) if paged else 64,
              transform="wht" if rng.random() < 0.4 else "identity", scale=1.0 / np.sqrt(d_latent + d_rope),
              extra_pages=1 if paged else 0)
    schedule = str(rng.choice(["auto", "chunked", "balanced"])) if dtype == "bf16" and d_latent == 512 else "auto"
    return kw, new, schedule


@pytest.mark.parametrize("i", range(60))
def test_random_prefill_configuration(i):
    kw, new, schedule = _random_prefill(i)
    print(f"prefill config {i}: {kw} new {new} schedule {schedule}", flush=True)
    case = inputs.make_case(7000 + i, name=f"prefill-random-{i}", **kw)
    dc = DeviceCase(case)
    query_start, q_lat, q_rope = _queries(case, 7100 + i, new)
    if int(query_start[-1]) == 0:
        return  # no new tokens: the call enqueues nothing (checked in the host tests)
    out, lse = _prefill(dc, query_start, q_lat, q_rope, schedule=schedule)
    torch.cuda.synchronize()
    ref, ref_lse = _oracle(case, query_start, q_lat, q_rope)
    got = out.cpu().numpy()
    if np.max(np.abs(ref)) == 0.0:
        assert np.all(got == 0.0)
    else:
        assert_parity(got, ref, case.dtype, f"prefill config {i}")
    assert_lse(lse.cpu().numpy(), ref_lse, case.dtype, f"prefill config {i}", case.transform)


def test_prefill_at_the_row_limit():
    """The most query rows one call takes (65,535): a single fresh prompt of 65,535 tokens, 32 heads,
    paged 64-token pages.  Its context is longer than the pages one workgroup stages, so the
    balanced schedule cuts shares at that bound.  Every output is finite; rows at the tile edges
    and the far end against the oracle one by one."""
    n = 65535
    case = inputs.make_case(95, batch=1, heads=32, d_latent=512, d_rope=64, shards=1, lens=n, paged=True,
                            page_size=64, scale=1.0 / np.sqrt(192), extra_pages=1, name="prefill-row-limit")
    dc = DeviceCase(case)
    query_start, q_lat, q_rope = _queries(case, 96, [n])
    print("prefill of 65535 new tokens", flush=True)
    out, lse = _prefill(dc, query_start, q_lat, q_rope)
    torch.cuda.synchronize()
    got_lse = lse.cpu().numpy()
    assert torch.isfinite(out).all().item() and np.all(np.isfinite(got_lse))
    pool = oracle_pool(case, [0])[0]
    rng = np.random.default_rng(97)
    for r in sorted({0, 1, 31, 32, 33, 4095, 32767, n - 2, n - 1, *rng.integers(0, n, size=3).tolist()}):
        ref, ref_lse = oracle.mla_prefill_absorbed(pool, None, [r + 1], [0, 1],
                                                   inputs.stored_to_f64(q_lat[r:r + 1], "bf16"),
                                                   inputs.stored_to_f64(q_rope[r:r + 1], "bf16"),
                                                   float(np.float32(case.scale)))
        assert_parity(out[r:r + 1].cpu().numpy(), ref, "bf16", f"row {r}")
        assert_lse(got_lse[r:r + 1], ref_lse, "bf16", f"row {r}")


def test_prefill_call_replays_from_a_hip_graph():
    """A prefill call (row map, tile-prefix scan, query rotation, decode kernel, merge) enqueues no
    memset, allocation or synchronisation, so it can be captured in a HIP graph; every replay, with
    eager work and synchronisations between replays, equals the eager call bit for bit."""
    case = inputs.make_case(33, batch=3, heads=128, d_latent=512, d_rope=64, shards=1, lens=[700, 90, 300],
                            paged=True, page_size=64, transform="wht", scale=1.0 / np.sqrt(192), extra_pages=1)
    dc = DeviceCase(case)
    query_start, q_lat, q_rope = _queries(case, 34, [50, 90, 1])
    qs_t, ql_t, qr_t = torch.from_numpy(query_start).to(DEV), to_torch(q_lat, "bf16"), to_torch(q_rope, "bf16")

    def call(**kw):
        return binding.mla_prefill_absorbed(dc.desc, dc.pool, dc.block_table, dc.seq_lens, qs_t, ql_t, qr_t, case.scale,
                                            case.max_seq_len, **kw)

    eager_out, eager_lse = call()
    out, lse = torch.empty_like(eager_out), torch.empty_like(eager_lse)
    ws = binding.alloc_workspace(binding.prefill_workspace_size(dc.desc, int(query_start[-1]), case.heads,
                                                                case.max_seq_len), DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(out=out, lse=lse, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(out=out, lse=lse, workspace=ws)
    for _ in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager_out) and torch.equal(lse, eager_lse)
