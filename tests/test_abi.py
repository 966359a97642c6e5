"""The C-ABI library on the CPU: it loads, exports every entry point include/tpla.h declares,
and rejects bad arguments on the host before touching the GPU (no compute calls here)."""

import ctypes
import os
import re

import pytest

from mla_latent_kv_13_amd import binding
from mla_latent_kv_13_amd import build as build_mod

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tpla.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(build_mod.LIB_PATH):
        build_mod.build()
    return binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^(?:int32_t|const char\*)\s+(\w+)\s*\(", text, flags=re.M)


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("latent_cache_append", "tpla_decode_sharded", "mla_decode_absorbed", "tpla_workspace_size",
                     "tpla_value_up_projection", "tpla_merge_context_parts", "latent_cache_append_normed"):
        assert required in names
    assert set(names) == set(binding.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert binding.abi_version() == 5
    assert lib.tpla_status_string(3) == b"TPLA_ERR_WORKSPACE_TOO_SMALL"


DSV3 = binding.Desc("bf16", 512, 64, 64, 1000, 1024, "identity")


def test_workspace_size_host_only(lib):
    n = binding.workspace_size(DSV3, 16, 128, 2, 2, 32768)
    assert n > 16 * 2 * 128 * 256 * 4  # at least one chunk of partials per sequence and shard
    rot = binding.Desc("bf16", 512, 64, 64, 1000, 1024, "wht")
    assert binding.workspace_size(rot, 16, 128, 2, 2, 32768) > n  # room for the rotated query
    # a paged cache uses the balanced schedule by default, which ignores chunk_tokens
    assert binding.workspace_size(DSV3, 16, 128, 2, 2, 32768, chunk_tokens=64) == n
    chunked = binding.workspace_size(DSV3, 16, 128, 2, 2, 32768, schedule="chunked")
    assert binding.workspace_size(DSV3, 16, 128, 2, 2, 32768, chunk_tokens=64, schedule="chunked") > chunked
    assert binding.workspace_size(DSV3, 16, 128, 2, 2, 32768, schedule="balanced") == n


def _ru(n):
    return (n + 255) // 256 * 256


def test_workspace_size_long_contexts(lib):
    """Past 4096 chunks a sequence's chunks grow, but never beyond what the kernel takes: 960
    tokens for the MFMA kernel on 1-row pages (1021 staged pages), 2048 for the generic kernel."""
    g, w = 2, 256
    paged1 = binding.Desc("bf16", 512, 64, 1, 8_000_000, 8_000_000, "identity")
    nc, heads = -(-8_000_000 // 960), 128
    assert binding.workspace_size(paged1, 1, heads, g, g, 8_000_000, schedule="chunked") == \
        _ru(nc * g * heads * w * 4) + _ru(nc * g * heads * 4)
    f32 = binding.Desc("f32", 512, 64, 16_000_000, 1, 0, "identity")
    nc, heads = -(-16_000_000 // 2048), 4
    assert binding.workspace_size(f32, 1, heads, g, g, 16_000_000) == _ru(nc * g * heads * w * 4) + _ru(nc * g * heads * 4)
    # an explicit chunk length is taken as given or refused
    with pytest.raises(binding.TplaError, match="UNSUPPORTED"):
        binding.workspace_size(f32, 1, heads, g, g, 16_000_000, chunk_tokens=4096)
    with pytest.raises(binding.TplaError, match="UNSUPPORTED"):
        binding.workspace_size(paged1, 1, 128, g, g, 8_000_000, chunk_tokens=1024, schedule="chunked")


@pytest.mark.parametrize("kw,msg", [
    (dict(num_shards=3), "INVALID_ARGUMENT"),            # 3 does not divide 512
    (dict(num_shards=2, shard_count=3), "INVALID_ARGUMENT"),
    (dict(heads=0), "INVALID_ARGUMENT"),
    (dict(chunk_tokens=100), "INVALID_ARGUMENT"),
    (dict(kernel="mfma", heads=40), "UNSUPPORTED"),
    (dict(kernel="generic", schedule="balanced"), "UNSUPPORTED"),  # balanced needs the MFMA kernel
])
def test_workspace_size_rejects(lib, kw, msg):
    args = dict(batch=2, heads=128, num_shards=2, shard_count=None, max_seq_len=4096, chunk_tokens=0, kernel="auto",
                schedule="auto")
    args.update(kw)
    if args["shard_count"] is None:
        args["shard_count"] = args["num_shards"]
    with pytest.raises(binding.TplaError, match=msg):
        binding.workspace_size(DSV3, args["batch"], args["heads"], args["num_shards"], args["shard_count"],
                               args["max_seq_len"], args["chunk_tokens"], args["kernel"], args["schedule"])


def _decode_raw(lib, desc, **kw):
    """Call tpla_decode_sharded with fake (never dereferenced) device addresses; only for
    arguments that validation rejects before anything is enqueued."""
    a = dict(cache=0x10000, block_table=0x20000, seq_lens=0x30000, batch=2, heads=128, max_seq_len=4096,
             q_latent=0x40000, q_rope=0x50000, scale=0.1, num_shards=2, shard_begin=0, shard_count=2,
             out=0x60000, lse=0, workspace=0x70000, workspace_bytes=1 << 40)
    a.update(kw)
    cdesc = desc.c()
    p = ctypes.c_void_p
    st = lib.tpla_decode_sharded(ctypes.byref(cdesc), p(a["cache"]), p(a["block_table"] or None), p(a["seq_lens"]),
                                 a["batch"], a["heads"], a["max_seq_len"], p(a["q_latent"]), p(a["q_rope"]),
                                 ctypes.c_float(a["scale"]), a["num_shards"], a["shard_begin"], a["shard_count"],
                                 p(a["out"]), p(a["lse"] or None), p(a["workspace"]), a["workspace_bytes"], None)
    return st, lib.tpla_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(cache=0), 1),
    (dict(out=0x60004), 1),                      # misaligned output
    (dict(shard_begin=1, shard_count=2), 1),     # shard range beyond G
    (dict(num_shards=5, shard_count=5), 1),      # G does not divide d_latent
    (dict(workspace_bytes=16), 3),
    (dict(scale=float("nan")), 1),
    (dict(block_table=0, max_seq_len=4096), 1),  # no block table needs page_size >= max_seq_len
])
def test_decode_validation_before_launch(lib, kw, status):
    st, msg = _decode_raw(lib, DSV3, **kw)
    assert st == status, (st, msg)
    assert msg


def _projected_raw(lib, desc, **kw):
    """tpla_decode_sharded_projected with fake (never dereferenced) device addresses; only for
    arguments that validation rejects before anything is enqueued."""
    a = dict(cache=0x10000, block_table=0x20000, seq_lens=0x30000, batch=2, heads=128, max_seq_len=4096,
             q_latent=0x40000, q_rope=0x50000, scale=0.1, num_shards=2, shard_begin=0, shard_count=2,
             w_dtype=1, w_uv=0x80000, d_v=128, out_v=0x60000, lse=0, workspace=0x70000, workspace_bytes=1 << 40)
    a.update(kw)
    cdesc = desc.c()
    p = ctypes.c_void_p
    st = lib.tpla_decode_sharded_projected(
        ctypes.byref(cdesc), p(a["cache"]), p(a["block_table"] or None), p(a["seq_lens"]), a["batch"], a["heads"],
        a["max_seq_len"], p(a["q_latent"]), p(a["q_rope"]), ctypes.c_float(a["scale"]), a["num_shards"],
        a["shard_begin"], a["shard_count"], a["w_dtype"], p(a["w_uv"] or None), a["d_v"], p(a["out_v"] or None),
        p(a["lse"] or None), p(a["workspace"]), a["workspace_bytes"], None, None)
    return st, lib.tpla_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(w_dtype=0), 2),                        # fp32 weights: the two-call path
    (dict(d_v=513), 2),
    (dict(d_v=0), 1),
    (dict(w_uv=0), 1),
    (dict(out_v=0), 1),
    (dict(w_uv=0x80008), 1),                     # misaligned weights
    (dict(out_v=0x60004), 1),                    # misaligned output
    (dict(workspace_bytes=16), 3),
    (dict(shard_begin=1, shard_count=2), 1),
])
def test_projected_decode_validation_before_launch(lib, kw, status):
    st, msg = _projected_raw(lib, DSV3, **kw)
    assert st == status, (st, msg)
    assert msg


def test_projected_decode_needs_latent_multiple_of_16(lib):
    d40 = binding.Desc("bf16", 40, 8, 64, 10, 16, "identity")
    st, msg = _projected_raw(lib, d40, num_shards=1, shard_count=1, heads=4)
    assert st == 2 and "multiple of 16" in msg


def test_bad_descriptor(lib):
    bad = binding.Desc("bf16", 768, 64, 64, 10, 16, "wht")  # Hadamard needs a power of two
    st, msg = _decode_raw(lib, bad)
    assert st == 2 and "power of two" in msg
    odd = binding.Desc("bf16", 512, 60, 64, 10, 16, "identity")  # 60 is not a multiple of 8
    st, msg = _decode_raw(lib, odd)
    assert st == 2


def _up_raw(lib, **kw):
    """tpla_value_up_projection with fake (never dereferenced) device addresses; only for
    arguments that validation settles before anything is enqueued."""
    a = dict(w_dtype=1, o=0x10000, w=0x20000, batch=4, heads=8, d_latent=512, d_v=128, out=0x30000)
    a.update(kw)
    p = ctypes.c_void_p
    st = lib.tpla_value_up_projection(a["w_dtype"], p(a["o"] or None), p(a["w"] or None), a["batch"], a["heads"],
                                      a["d_latent"], a["d_v"], p(a["out"] or None), None)
    return st, lib.tpla_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(w_dtype=7), 2),
    (dict(batch=-1), 1),
    (dict(d_v=0), 1),
    (dict(d_latent=0), 1),
    (dict(o=0), 1),
    (dict(w=0x20008), 1),          # misaligned weights
    (dict(heads=70000), 2),
])
def test_up_projection_validation_before_launch(lib, kw, status):
    st, msg = _up_raw(lib, **kw)
    assert st == status, (st, msg)
    assert msg


def test_up_projection_empty_is_a_no_op(lib):
    # nothing is enqueued, so no device is touched: fine without a GPU
    assert _up_raw(lib, batch=0, o=0, w=0, out=0)[0] == 0
    assert _up_raw(lib, heads=0, o=0, w=0, out=0)[0] == 0


def _merge_raw(lib, **kw):
    """tpla_merge_context_parts with fake (never dereferenced) device addresses; only for
    arguments that validation settles before anything is enqueued."""
    a = dict(transform=0, G=2, s0=0, n=2, parts=3, batch=4, heads=8, d=512, op=0x10000, lp=0x20000, out=0x30000,
             lse=0x40000)
    a.update(kw)
    p = ctypes.c_void_p
    st = lib.tpla_merge_context_parts(a["transform"], a["G"], a["s0"], a["n"], a["parts"], a["batch"], a["heads"],
                                      a["d"], p(a["op"] or None), p(a["lp"] or None), p(a["out"] or None),
                                      p(a["lse"] or None), None)
    return st, lib.tpla_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(transform=5), 1),
    (dict(parts=0), 1),
    (dict(G=3), 1),                 # 3 does not divide 512
    (dict(s0=1, n=2), 1),           # shard range beyond G
    (dict(d=2048, G=2), 2),
    (dict(G=128, n=128), 2),        # more than 64 shards in one call
    (dict(transform=1, d=96, G=1, n=1), 2),  # Hadamard needs a power of two
    (dict(op=0), 1),
    (dict(out=0x30008), 1),         # misaligned output
    (dict(batch=70000), 2),
])
def test_context_merge_validation_before_launch(lib, kw, status):
    st, msg = _merge_raw(lib, **kw)
    assert st == status, (st, msg)
    assert msg


def test_context_merge_empty_is_a_no_op(lib):
    assert _merge_raw(lib, batch=0, op=0, lp=0, out=0, lse=0)[0] == 0


@pytest.mark.parametrize("desc,norm,eps,status", [
    (DSV3, 0, 1e-6, 1),             # at least one slice
    (DSV3, 3, 1e-6, 1),             # 3 does not divide 512
    (DSV3, 2, -1.0, 1),             # negative eps
    (DSV3, 2, float("inf"), 1),
    (DSV3, 128, 1e-6, 2),           # more than 64 slices
    (binding.Desc("bf16", 576, 64, 64, 1000, 1024, "identity"), 1, 1e-6, 2),  # not a power of two
])
def test_normed_append_validation(lib, desc, norm, eps, status):
    cdesc = desc.c()
    p = ctypes.c_void_p
    st = lib.latent_cache_append_normed(ctypes.byref(cdesc), p(0x10000), p(0x20000), p(0x30000), 4, norm,
                                        ctypes.c_float(eps), None)
    assert st == status, (st, lib.tpla_last_error().decode())


def test_normed_append_zero_rows_is_a_no_op(lib):
    cdesc = DSV3.c()
    assert lib.latent_cache_append_normed(ctypes.byref(cdesc), None, None, None, 0, 2, ctypes.c_float(1e-6),
                                          None) == 0


def _prefill_raw(lib, desc, **kw):
    """Call mla_prefill_absorbed with fake (never dereferenced) device addresses; only for
    arguments that validation rejects, or that make the call a no-op, before anything is enqueued."""
    a = dict(cache=0x10000, block_table=0x20000, seq_lens=0x30000, query_start=0x38000, batch=2, num_queries=64,
             heads=128, max_seq_len=4096, q_latent=0x40000, q_rope=0x50000, scale=0.1, out=0x60000, lse=0,
             workspace=0x70000, workspace_bytes=1 << 40)
    a.update(kw)
    cdesc = desc.c()
    p = ctypes.c_void_p
    st = lib.mla_prefill_absorbed(ctypes.byref(cdesc), p(a["cache"]), p(a["block_table"] or None),
                                  p(a["seq_lens"] or None), p(a["query_start"] or None), a["batch"],
                                  a["num_queries"], a["heads"], a["max_seq_len"], p(a["q_latent"]), p(a["q_rope"]),
                                  ctypes.c_float(a["scale"]), p(a["out"]), p(a["lse"] or None), p(a["workspace"]),
                                  a["workspace_bytes"], None)
    return st, lib.tpla_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(query_start=0), 1),
    (dict(seq_lens=0), 1),
    (dict(batch=0), 1),
    (dict(num_queries=-1), 1),
    (dict(num_queries=70000), 2),               # more query rows than the merge grid takes
    (dict(workspace_bytes=16), 3),
    (dict(out=0x60004), 1),                     # misaligned output
    (dict(scale=float("nan")), 1),
    (dict(block_table=0, batch=2000), 1),       # without a block table each sequence owns a page
])
def test_prefill_validation_before_launch(lib, kw, status):
    st, msg = _prefill_raw(lib, DSV3, **kw)
    assert st == status, (st, msg)
    assert msg
    if kw.get("num_queries", 0) > 65535:
        assert "num_queries" in msg, msg


def test_prefill_without_new_tokens_is_a_no_op(lib):
    st, msg = _prefill_raw(lib, DSV3, num_queries=0)
    assert st == 0 and msg == ""
    assert binding.prefill_workspace_size(DSV3, 0, 128, 4096) == 0


def test_prefill_workspace_holds_the_row_map(lib):
    # the same rows as a decode call, plus the row map (prefix length and sequence per row)
    rows = 1000
    dec = binding.workspace_size(DSV3, rows, 128, 1, 1, 4096)
    pre = binding.prefill_workspace_size(DSV3, rows, 128, 4096)
    assert pre == dec + 2 * _ru(rows * 4)
    contiguous = binding.Desc("bf16", 512, 64, 4096, 8, 0, "identity")
    assert binding.prefill_workspace_size(contiguous, rows, 128, 4096) == \
        binding.workspace_size(contiguous, rows, 128, 1, 1, 4096) + 2 * _ru(rows * 4)


def test_balanced_workers_only_grow_past_the_staged_page_bound(lib):
    """Balanced schedule (paged cache): one worker per CU slot unless a context is longer than the
    pages a workgroup stages (1021 pages of 64 rows here, 2041 tiles); workspace sizes show the
    worker count (partial slots = rows + workers)."""
    g1 = binding.Desc("bf16", 512, 64, 64, 100_000, 2048, "identity")
    heads, w = 128, 512  # w = 512: two head groups of 64 per unit, one workgroup per CU -> 128 workers

    def partials(slots):
        return _ru(slots * heads * w * 4) + _ru(slots * heads * 4)

    # prefill of 4096 rows over contexts of 4096: within the bound, so 128 workers
    rows = 4096
    assert binding.prefill_workspace_size(g1, rows, heads, 4096) == 2 * _ru(rows * 4) + _ru((rows + 1) * 4) + \
        partials(rows + 128)
    # decode of 64 sequences up to 131072 tokens (4096 tiles > 2041): shares must stay under the bound,
    # ceil(64 * 4096 / 2041) = 129 workers
    assert binding.workspace_size(g1, 64, heads, 1, 1, 131072) == _ru(65 * 4) + partials(64 + 129)


def test_header_compiles_as_c99(tmp_path):
    """include/tpla.h is a C interface: a C99 translation unit that includes it and takes the
    address of every declared function compiles with gcc, warnings as errors."""
    import shutil
    import subprocess

    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    names = declared_functions()
    src = tmp_path / "abi_check.c"
    src.write_text('#include "tpla.h"\ntypedef void (*any_fn)(void);\nany_fn all_entry_points[] = {\n'
                   + "".join(f"  (any_fn)&{n},\n" for n in names) + "};\n")
    res = subprocess.run([gcc, "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror", "-fsyntax-only",
                          "-I", os.path.join(ROOT, "include"), str(src)], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
