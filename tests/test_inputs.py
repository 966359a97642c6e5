"""Seeded input generator: determinism, layout validity, workload shapes (CPU)."""

import hashlib

import numpy as np

from mla_latent_kv_13_amd import inputs


def _digest(case):
    h = hashlib.sha256()
    for a in (case.q_lat, case.q_rope, case.rows, case.slots, case.seq_lens):
        h.update(np.ascontiguousarray(a).tobytes())
    if case.block_table is not None:
        h.update(case.block_table.tobytes())
    return h.hexdigest()


def test_deterministic():
    kw = dict(batch=3, heads=8, d_latent=64, d_rope=16, shards=2, len_range=(1, 200), paged=True, page_size=16)
    assert _digest(inputs.make_case(7, **kw)) == _digest(inputs.make_case(7, **kw))
    assert _digest(inputs.make_case(7, **kw)) != _digest(inputs.make_case(8, **kw))


def test_bf16_conversion_round_trip_and_ties():
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 0.0], dtype=np.float32)
    bits = inputs.f32_to_bf16_bits(x)
    back = inputs.bf16_bits_to_f32(bits)
    assert back.tolist() == [1.0, 1.0, 1.0 + 2.0 ** -6, -2.5, 0.0]


def test_paged_layout_is_valid():
    case = inputs.make_case(3, batch=5, heads=4, d_latent=32, d_rope=8, shards=2, lens=[0, 1, 63, 64, 130],
                            paged=True, page_size=64, extra_pages=3)
    bt = case.block_table
    used = bt[bt >= 0]
    assert len(np.unique(used)) == len(used)  # no page shared between sequences
    for b, t in enumerate(case.seq_lens):
        n = (int(t) + 63) // 64
        assert np.all(bt[b, :n] >= 0) and np.all(bt[b, n:] == -1)
    assert case.num_pages == len(used) + 3
    flat = case.pool.reshape(-1, case.width)
    assert np.array_equal(flat[case.slots], case.rows)
    mask = np.ones(flat.shape[0], dtype=bool)
    mask[case.slots] = False
    assert np.all(flat[mask] == inputs.BF16_NAN)  # page tails and unused pages are NaN


def test_workload_shapes():
    c1 = inputs.make_config(1)
    assert c1.pool.shape == (1, 128, 80) and c1.dtype == "f32" and c1.shards == 2
    assert abs(c1.scale - 1 / np.sqrt(48)) < 1e-7
    c2 = inputs.make_config(2)
    assert c2.pool.shape == (32, 4096, 576) and c2.q_lat.shape == (32, 128, 512) and c2.total_tokens == 131072
    lens = np.random.default_rng([5, 5]).integers(1024, 65536, size=64, endpoint=True)
    assert int(lens.sum()) == 2085650
    assert sum((int(t) + 63) // 64 for t in lens) == 32624


def test_prefill_queries_layout_and_determinism():
    qs, q_lat, q_rope = inputs.make_prefill_queries(5, new_tokens=[3, 0, 7], heads=4, d_latent=64, d_rope=16)
    assert qs.dtype == np.int32 and list(qs) == [0, 3, 3, 10]
    assert q_lat.shape == (10, 4, 64) and q_rope.shape == (10, 4, 16)
    assert q_lat.dtype == np.uint16 and q_rope.dtype == np.uint16  # bf16 bit patterns
    again = inputs.make_prefill_queries(5, new_tokens=[3, 0, 7], heads=4, d_latent=64, d_rope=16)
    assert np.array_equal(again[1], q_lat) and np.array_equal(again[2], q_rope)
    f32 = inputs.make_prefill_queries(5, new_tokens=[2], heads=1, d_latent=8, d_rope=8, dtype="f32")
    assert f32[1].dtype == np.float32 and np.isfinite(f32[1]).all()
    none = inputs.make_prefill_queries(1, new_tokens=[0, 0], heads=2, d_latent=8, d_rope=8)
    assert list(none[0]) == [0, 0, 0] and none[1].shape == (0, 2, 8)


def test_token_gain_scales_rows_along_each_sequence():
    """The same draws as without the gain, row t of a T-token sequence times gain ** (t / (T - 1));
    one-token sequences are left as drawn."""
    kw = dict(batch=3, heads=4, d_latent=64, d_rope=16, shards=2, lens=[100, 1, 33], dtype="f32")
    plain = inputs.make_case(11, **kw)
    grown = inputs.make_case(11, token_gain=8.0, **kw)
    off = 0
    for t_b in plain.seq_lens:
        t_b = int(t_b)
        a, g = plain.rows[off:off + t_b], grown.rows[off:off + t_b]
        ramp = 8.0 ** (np.arange(t_b) / max(t_b - 1, 1)) if t_b > 1 else np.ones(1)
        np.testing.assert_allclose(g, a * ramp[:, None], rtol=1e-6)
        off += t_b
    assert np.array_equal(plain.q_lat, grown.q_lat) and np.array_equal(plain.slots, grown.slots)
