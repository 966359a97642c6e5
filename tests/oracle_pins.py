"""Pins that tie the fp64 oracle to something other than itself.

Each ``pin_*`` function takes a module with the oracle's API and raises
AssertionError when the module disagrees with what the pages or the
mathematics fix.  ``test_oracle_pins.py`` runs them on the real oracle;
``test_oracle_mutations.py`` runs them on deliberately broken copies of it
and expects at least one pin to fail for each planted mistake.

Sources for the definitions (by page title and part):
 [FR]  "[Feature Request] Bandwidth-optimal tensor-parallel sharding of MLA
       (latent-cache sharding / TPLA)"
 [ABS] "TPLA: Tensor Parallel Latent Attention for Efficient Disaggregated
       Prefill & Decode Inference", abstract
 [REV] automated review of arXiv 2508.15881 (pith.science verdict)
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import scipy.linalg
import scipy.special
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = max(np.linalg.norm(b), 1e-300)
    return float(np.linalg.norm(a - b) / den)


def _pool(lat_rows, rope_rows, max_len=None):
    """Contiguous float64 pool [B, max_len, d_c + d_r] with NaN beyond each length."""
    B = len(lat_rows)
    d_c = lat_rows[0].shape[1]
    d_r = rope_rows[0].shape[1]
    lens = [x.shape[0] for x in lat_rows]
    max_len = max_len or max(1, max(lens))
    pool = np.full((B, max_len, d_c + d_r), np.nan)
    for b in range(B):
        pool[b, :lens[b], :d_c] = lat_rows[b]
        pool[b, :lens[b], d_c:] = rope_rows[b]
    return pool, np.array(lens, dtype=np.int32)


def _random_problem(seed, B=3, H=4, d_c=32, d_r=8, lens=(9, 1, 17), chan=None):
    rng = np.random.default_rng(seed)
    lat = [rng.standard_normal((t, d_c)) * (1.0 if chan is None else chan) for t in lens]
    rope = [rng.standard_normal((t, d_r)) for t in lens]
    pool, seq_lens = _pool(lat, rope)
    q_lat = rng.standard_normal((B, H, d_c))
    q_rope = rng.standard_normal((B, H, d_r))
    return pool, seq_lens, q_lat, q_rope


# ---------------------------------------------------------------- P1
def pin_p1_absorbed_equals_unabsorbed(orc):
    """G = 1 equals MLA with K and V expanded through W_UK / W_UV ([FR] Tests /
    validation: G = 1 must match head-parallel MLA exactly; [REV] referee
    report, significance: matrix absorption).  Brute force by explicit loops."""
    rng = np.random.default_rng(11)
    B, H, d_c, d_r, d_nope, d_v = 2, 3, 16, 8, 6, 5
    lens = (7, 4)
    scale = 0.37
    lat = [rng.standard_normal((t, d_c)) for t in lens]
    rope = [rng.standard_normal((t, d_r)) for t in lens]
    pool, seq_lens = _pool(lat, rope)
    q_nope = rng.standard_normal((B, H, d_nope))
    q_rope = rng.standard_normal((B, H, d_r))
    w_uk = rng.standard_normal((H, d_nope, d_c))
    w_uv = rng.standard_normal((H, d_v, d_c))
    # absorbed query of head h: W_UK[h]^T q_nope  (a [d_c] vector)
    q_lat = np.stack([np.stack([w_uk[h].T @ q_nope[b, h] for h in range(H)]) for b in range(B)])
    out, lse = orc.mla_decode_absorbed(pool, None, seq_lens, q_lat, q_rope, scale)
    assert out.shape == (B, H, d_c) and lse.shape == (B, H)
    # then the value up-projection the absorbed form applies afterwards
    projected = orc.value_up_projection(out, w_uv)
    assert projected.shape == (B, H, d_v)
    for b in range(B):
        ref = orc.mla_unabsorbed_bruteforce(lat[b], rope[b], q_nope[b], q_rope[b], w_uk, w_uv, scale)
        assert _rel(projected[b], ref) <= 1e-12, ("P1", b, _rel(projected[b], ref))


def pin_p1b_bruteforce_closed_form(orc):
    """The brute force itself: one token gives its value row exactly, and two
    tokens with a logit gap of ln 3 give weights 1/4, 3/4."""
    H, d_c, d_r, d_nope, d_v = 1, 2, 1, 1, 2
    w_uk = np.ones((H, d_nope, d_c))
    w_uv = np.array([[[1.0, 0.0], [0.0, 2.0]]])
    c = np.array([[1.0, -1.0]])
    got = orc.mla_unabsorbed_bruteforce(c, np.zeros((1, d_r)), np.ones((H, d_nope)),
                                        np.zeros((H, d_r)), w_uk, w_uv, 1.0)
    assert np.allclose(got, [[1.0, -2.0]], rtol=0, atol=1e-15), got
    c = np.array([[0.0, 0.0], [math.log(3.0), 0.0]])
    got = orc.mla_unabsorbed_bruteforce(c, np.zeros((2, d_r)), np.ones((H, d_nope)),
                                        np.zeros((H, d_r)), w_uk, w_uv, 1.0)
    assert np.allclose(got, [[0.75 * math.log(3.0), 0.0]], rtol=1e-14, atol=1e-15), got


# ---------------------------------------------------------------- P9
def pin_p9_value_projection(orc):
    """The value up-projection on its own: W_UV[h] = I returns the latent
    output unchanged; a one-hot W_UV[h] (row v reads latent column c) moves
    out_latent[b, h, c] to out_v[b, h, v] for that head only, so a transposed
    or head-shifted weight fails; and the projections of the shard subsets of
    a G = 2 call, with and without the rotation, add up to the projection of
    the full call ([FR] Background: o_proj rowwise then all-reduce; reading A1)."""
    rng = np.random.default_rng(91)
    B, H, d_c, d_v = 2, 3, 8, 5
    y = rng.standard_normal((B, H, d_c))
    eye = np.broadcast_to(np.eye(d_c), (H, d_c, d_c))
    assert np.array_equal(orc.value_up_projection(y, eye), y)
    w = np.zeros((H, d_v, d_c))
    picks = {0: (1, 6), 1: (4, 0), 2: (0, 3)}  # head -> (v, c)
    for h, (v, c) in picks.items():
        w[h, v, c] = 2.0
    got = orc.value_up_projection(y, w)
    want = np.zeros((B, H, d_v))
    for h, (v, c) in picks.items():
        want[:, h, v] = 2.0 * y[:, h, c]
    assert np.array_equal(got, want), ("P9 one-hot", got, want)
    pool, seq_lens, q_lat, q_rope = _random_problem(92, B=2, H=3, d_c=16, d_r=4, lens=(6, 11))
    w_uv = rng.standard_normal((3, 7, 16))
    for transform in ("identity", "wht"):
        if transform == "wht":
            flat = pool.reshape(-1, pool.shape[-1])
            used = ~np.isnan(flat[:, 0])
            store = np.full_like(flat, np.nan)
            store = orc.latent_cache_append(store[None], flat[used], np.flatnonzero(used), 16, "wht", "f64")[0]
            src = store.reshape(pool.shape)
        else:
            src = pool
        full, _ = orc.tpla_decode_sharded(src, None, seq_lens, q_lat, q_rope, 0.3, 2, transform=transform)
        parts = [orc.tpla_decode_sharded(src, None, seq_lens, q_lat, q_rope, 0.3, 2, s, 1, transform=transform)[0]
                 for s in range(2)]
        summed = orc.value_up_projection(parts[0], w_uv) + orc.value_up_projection(parts[1], w_uv)
        assert _rel(summed, orc.value_up_projection(full, w_uv)) <= 1e-13, ("P9 shard sum", transform)


# ---------------------------------------------------------------- P10
def pin_p10_context_split_merge(orc):
    """Decoding each part of a split context and merging the parts by
    log-sum-exp gives the decode of the whole context ([FR] Directions: exact
    context parallelism, sequence split + log-sum-exp merge).  The whole-context
    decode is computed independently by the oracle's own decode, so a wrong
    weight, a missing un-rotation or a shard mix-up fails.  Covers G = 1, G = 2
    with a shard subset, the Hadamard transform, a part with no tokens and a
    sequence with none at all."""
    rng = np.random.default_rng(101)
    B, H, d_c, d_r = 3, 2, 16, 4
    lens = (13, 5, 0)
    lat = [rng.standard_normal((t, d_c)) * 2.0 for t in lens]
    rope = [rng.standard_normal((t, d_r)) for t in lens]
    q_lat = rng.standard_normal((B, H, d_c))
    q_rope = rng.standard_normal((B, H, d_r))
    cuts = [(0, 4), (4, 4), (4, 13)]  # token ranges of the parts; the second is empty for every sequence
    for transform, G, s0, n in (("identity", 1, 0, 1), ("identity", 2, 1, 1), ("wht", 2, 0, 2), ("wht", 4, 1, 2)):
        def pool_of(ranges):
            parts_lat = [lat[b][min(a, lens[b]):min(e, lens[b])] for b, (a, e) in enumerate(ranges)]
            parts_rope = [rope[b][min(a, lens[b]):min(e, lens[b])] for b, (a, e) in enumerate(ranges)]
            pool, seq_lens = _pool(parts_lat, parts_rope, max_len=13)
            if transform == "wht":
                flat = pool.reshape(-1, pool.shape[-1])
                used = ~np.isnan(flat[:, 0])
                if np.any(used):
                    store = orc.latent_cache_append(np.full_like(flat, np.nan)[None], flat[used],
                                                    np.flatnonzero(used), d_c, "wht", "f64")[0]
                    pool = store.reshape(pool.shape)
            return pool, seq_lens
        full_pool, full_lens = pool_of([(0, 13)] * B)
        want, want_lse = orc.tpla_decode_sharded(full_pool, None, full_lens, q_lat, q_rope, 0.4, G, s0, n,
                                                 transform=transform)
        outs, lses = [], []
        for a, e in cuts:
            pool, seq_lens = pool_of([(a, e)] * B)
            o, l = orc.tpla_decode_sharded(pool, None, seq_lens, q_lat, q_rope, 0.4, G, s0, n, transform=transform)
            outs.append(o)
            lses.append(l)
        got, got_lse = orc.merge_context_parts(np.stack(outs), np.stack(lses), G, s0, n, transform=transform)
        assert np.max(np.abs(got - want)) <= 1e-12, ("P10 out", transform, G, np.max(np.abs(got - want)))
        assert np.array_equal(np.isneginf(got_lse), np.isneginf(want_lse)), ("P10 lse -inf", transform, G)
        fin = ~np.isneginf(want_lse)
        assert np.max(np.abs(got_lse[fin] - want_lse[fin])) <= 1e-12, ("P10 lse", transform, G)


# ---------------------------------------------------------------- P2
def pin_p2_hadamard_invariance_g1(orc):
    """At G = 1 an orthogonal rotation of both query and latent leaves the
    output unchanged ([ABS]: orthogonal transform before slicing; [REV]
    referee report: Proposition 1 on orthogonal transforms).  Exact with the
    storage rounding switched off; at bf16 storage only the rounding differs."""
    rng = np.random.default_rng(21)
    B, H, d_c, d_r = 2, 5, 64, 16
    lens = (33, 5)
    lat = [rng.standard_normal((t, d_c)) for t in lens]
    rope = [rng.standard_normal((t, d_r)) for t in lens]
    pool, seq_lens = _pool(lat, rope)
    q_lat = rng.standard_normal((B, H, d_c))
    q_rope = rng.standard_normal((B, H, d_r))
    rows = np.concatenate([np.concatenate([lat[b], rope[b]], axis=1) for b in range(B)])
    slots = np.concatenate([b * pool.shape[1] + np.arange(lens[b]) for b in range(B)])
    base, base_lse = orc.mla_decode_absorbed(pool, None, seq_lens, q_lat, q_rope, 0.2)
    empty = np.full_like(pool, np.nan)
    rot = orc.latent_cache_append(empty, rows, slots, d_c, "wht", "f64")
    out, lse = orc.mla_decode_absorbed(rot, None, seq_lens, q_lat, q_rope, 0.2, transform="wht")
    assert _rel(out, base) <= 1e-12, ("P2 exact", _rel(out, base))
    assert np.allclose(lse, base_lse, rtol=1e-12, atol=1e-12)
    rot16 = orc.latent_cache_append(empty, rows, slots, d_c, "wht", "bf16")
    out16, _ = orc.mla_decode_absorbed(rot16, None, seq_lens, q_lat, q_rope, 0.2, transform="wht")
    err = _rel(out16, base)
    assert 1e-6 < err <= 1e-2, ("P2 bf16", err)


# ---------------------------------------------------------------- P3
def pin_p3_shard_decomposition(orc):
    """The G-shard output is the sum of G independent attentions, shard s
    over [latent slice s | rope] with the matching query slice ([ABS]:
    attention runs per shard, then an all-reduce adds the results; reading
    A1).  Each shard is re-run as a single-shard problem on sliced data."""
    G = 4
    pool, seq_lens, q_lat, q_rope = _random_problem(31, d_c=32, d_r=8)
    d_c = q_lat.shape[2]
    w = d_c // G
    out, lse = orc.tpla_decode_sharded(pool, None, seq_lens, q_lat, q_rope, 0.3, G)
    total = np.zeros_like(out)
    for s in range(G):
        cols = list(range(s * w, (s + 1) * w)) + list(range(d_c, pool.shape[2]))
        sub = pool[:, :, cols]
        o_s, l_s = orc.mla_decode_absorbed(sub, None, seq_lens, q_lat[:, :, s * w:(s + 1) * w], q_rope, 0.3)
        total[:, :, s * w:(s + 1) * w] += o_s
        assert np.allclose(lse[:, s, :], l_s, rtol=1e-14, atol=1e-14), ("P3 lse", s)
    assert _rel(out, total) <= 1e-14, ("P3", _rel(out, total))


def pin_p3b_subset_additivity(orc):
    """One device's share (a shard subset) is additive: the all-reduce of the
    per-shard outputs equals the all-shard output (reading A13), with and
    without the rotation (the rotation back is linear)."""
    G = 4
    pool, seq_lens, q_lat, q_rope = _random_problem(32, d_c=32, d_r=8)
    for transform in ("identity", "wht"):
        full, lse = orc.tpla_decode_sharded(pool, None, seq_lens, q_lat, q_rope, 0.3, G, transform=transform)
        acc = np.zeros_like(full)
        for s in range(G):
            o, l = orc.tpla_decode_sharded(pool, None, seq_lens, q_lat, q_rope, 0.3, G, s, 1, transform=transform)
            acc += o
            assert np.allclose(l[:, 0], lse[:, s], rtol=1e-14, atol=1e-14)
            if transform == "identity":
                mask = np.ones(q_lat.shape[2], dtype=bool)
                mask[s * 8:(s + 1) * 8] = False
                assert np.all(o[:, :, mask] == 0.0)
        assert _rel(acc, full) <= 1e-13, ("P3b", transform, _rel(acc, full))


# ---------------------------------------------------------------- P18 (prefill)
def pin_p18_prefill_equals_unabsorbed_causal(orc):
    """Prefill keeps exact MLA over each new token's causal prefix ([REV] referee
    report, summary: prefill/decode separation): after the value up-projection,
    every new token's row equals un-absorbed MLA (K and V expanded through W_UK
    and W_UV by explicit loops) over the cached tokens up to its own position.
    Sequence 0 continues a cached context (3 new of 7), sequence 1 is a fresh
    prompt (5 new of 5)."""
    rng = np.random.default_rng(18)
    H, d_c, d_r, d_nope, d_v = 2, 8, 4, 3, 5
    lens, new = (7, 5), (3, 5)
    scale = 0.41
    lat = [rng.standard_normal((t, d_c)) for t in lens]
    rope = [rng.standard_normal((t, d_r)) for t in lens]
    pool, seq_lens = _pool(lat, rope)
    query_start = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    nq = int(query_start[-1])
    q_nope = rng.standard_normal((nq, H, d_nope))
    q_rope = rng.standard_normal((nq, H, d_r))
    w_uk = rng.standard_normal((H, d_nope, d_c))
    w_uv = rng.standard_normal((H, d_v, d_c))
    q_lat = np.stack([np.stack([w_uk[h].T @ q_nope[r, h] for h in range(H)]) for r in range(nq)])
    out, lse = orc.mla_prefill_absorbed(pool, None, seq_lens, query_start, q_lat, q_rope, scale)
    assert out.shape == (nq, H, d_c) and lse.shape == (nq, H)
    projected = orc.value_up_projection(out, w_uv)
    for b in range(2):
        for j in range(new[b]):
            r = int(query_start[b]) + j
            vis = lens[b] - new[b] + j + 1
            ref = orc.mla_unabsorbed_bruteforce(lat[b][:vis], rope[b][:vis], q_nope[r], q_rope[r], w_uk, w_uv, scale)
            assert _rel(projected[r], ref) <= 1e-12, ("P18", b, j, _rel(projected[r], ref))


def _sdpa_causal(pool, seq_lens, query_start, q_lat, q_rope, scale, hmat):
    """Absorbed prefill through torch's scaled_dot_product_attention (fp64) with
    an explicit boolean mask: new token j of n sees keys t <= T - n + j."""
    nq, H, d_c = q_lat.shape
    out = np.zeros((nq, H, d_c))
    for b in range(len(seq_lens)):
        r0, r1 = int(query_start[b]), int(query_start[b + 1])
        T, n = int(seq_lens[b]), r1 - r0
        if n == 0:
            continue
        c, r = pool[b, :T, :d_c], pool[b, :T, d_c:]
        qt = q_lat[r0:r1] @ hmat if hmat is not None else q_lat[r0:r1]
        q = torch.from_numpy(np.ascontiguousarray(np.concatenate([qt, q_rope[r0:r1]], axis=2).transpose(1, 0, 2)))
        k = torch.from_numpy(np.ascontiguousarray(np.concatenate([c, r], axis=1))).expand(H, T, -1)
        v = torch.from_numpy(np.ascontiguousarray(c)).expand(H, T, -1)
        mask = torch.from_numpy(np.arange(T)[None, :] <= (T - n + np.arange(n))[:, None])
        o = torch.nn.functional.scaled_dot_product_attention(q.unsqueeze(0), k.unsqueeze(0), v.unsqueeze(0),
                                                             attn_mask=mask, scale=scale)
        y = o[0].numpy().transpose(1, 0, 2)
        out[r0:r1] = y @ hmat if hmat is not None else y
    return out


def pin_p18b_prefill_sdpa_causal(orc):
    """Prefill = torch SDPA (fp64) with the offset causal mask, on a paged pool,
    plain and with the Hadamard-rotated cache (scipy's Hadamard matrix); lse of
    one row against scipy's logsumexp of its visible logits."""
    rng = np.random.default_rng(181)
    H, d_c, d_r = 3, 16, 8
    lens, new = (11, 6, 9), (4, 0, 9)
    page, B = 4, len(lens)
    per = (max(lens) + page - 1) // page
    lat = [rng.standard_normal((t, d_c)) for t in lens]
    rope = [rng.standard_normal((t, d_r)) for t in lens]
    pool, seq_lens = _pool(lat, rope, max_len=per * page)
    query_start = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    nq = int(query_start[-1])
    q_lat = rng.standard_normal((nq, H, d_c))
    q_rope = rng.standard_normal((nq, H, d_r))
    # the same rows in a paged pool of 4-token pages, pages shuffled
    perm = rng.permutation(B * per)
    paged = np.full((B * per * page, d_c + d_r), np.nan)
    bt = np.zeros((B, per), dtype=np.int32)
    for b in range(B):
        for i in range(per):
            bt[b, i] = perm[b * per + i]
            paged[bt[b, i] * page:(bt[b, i] + 1) * page] = pool[b, i * page:(i + 1) * page]
    out, lse = orc.mla_prefill_absorbed(paged.reshape(-1, page, d_c + d_r), bt, seq_lens, query_start, q_lat,
                                        q_rope, 0.3)
    ref = _sdpa_causal(pool, seq_lens, query_start, q_lat, q_rope, 0.3, None)
    assert _rel(out, ref) <= 1e-12, ("P18b", _rel(out, ref))
    r = 2  # sequence 0, new token 2: sees 11 - 4 + 2 + 1 = 10 tokens
    logits = 0.3 * (q_lat[r] @ pool[0, :10, :d_c].T + q_rope[r] @ pool[0, :10, d_c:].T)
    assert np.allclose(lse[r], scipy.special.logsumexp(logits, axis=1), rtol=1e-14, atol=1e-13)
    # rotated cache written by the oracle's own append with exact storage
    rows = np.concatenate([pool[b, :lens[b]] for b in range(B)])
    slots = np.concatenate([b * pool.shape[1] + np.arange(lens[b]) for b in range(B)])
    rot = orc.latent_cache_append(np.full_like(pool, np.nan), rows, slots, d_c, "wht", "f64")
    out_r, _ = orc.mla_prefill_absorbed(rot, None, seq_lens, query_start, q_lat, q_rope, 0.3, transform="wht")
    hmat = scipy.linalg.hadamard(d_c).astype(np.float64) / math.sqrt(d_c)
    rot_ref = pool.copy()
    rot_ref[:, :, :d_c] = pool[:, :, :d_c] @ hmat
    ref_r = _sdpa_causal(rot_ref, seq_lens, query_start, q_lat, q_rope, 0.3, hmat)
    assert _rel(out_r, ref_r) <= 1e-12, ("P18b wht", _rel(out_r, ref_r))
    assert _rel(out_r, out) <= 1e-12, ("P18b rotation leaves exact MLA unchanged", _rel(out_r, out))


def pin_p18c_prefill_closed_forms(orc):
    """The first token of a fresh prompt sees only itself: its output is its own
    latent row and its lse its own logit; a sequence without new tokens adds no
    row; a row with no visible token (more new tokens than cached) is 0 / -inf."""
    rng = np.random.default_rng(182)
    H, d_c, d_r = 2, 8, 4
    lens, new = (5, 3, 2), (5, 0, 3)
    lat = [rng.standard_normal((t, d_c)) for t in lens]
    rope = [rng.standard_normal((t, d_r)) for t in lens]
    pool, seq_lens = _pool(lat, rope)
    query_start = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    q_lat = rng.standard_normal((8, H, d_c))
    q_rope = rng.standard_normal((8, H, d_r))
    out, lse = orc.mla_prefill_absorbed(pool, None, seq_lens, query_start, q_lat, q_rope, 0.5)
    assert np.array_equal(out[0], np.broadcast_to(lat[0][0], (H, d_c))), out[0]
    own = 0.5 * (q_lat[0] @ lat[0][0] + q_rope[0] @ rope[0][0])
    assert np.allclose(lse[0], own, rtol=1e-15, atol=1e-15)
    # sequence 2: 3 new tokens but 2 cached: row 5 sees nothing, row 6 sees token 0
    assert np.all(out[5] == 0.0) and np.all(np.isneginf(lse[5]))
    assert np.array_equal(out[6], np.broadcast_to(lat[2][0], (H, d_c)))
    assert np.isfinite(lse[7]).all() and not np.array_equal(out[7], out[6])


# ---------------------------------------------------------------- P4
def _sdpa_gla(pool, seq_lens, q_lat, q_rope, scale, G, hmat):
    """TPLA as grouped latent attention with G*H virtual heads through torch's
    scaled_dot_product_attention in float64 ([REV] forward implications: TPLA
    is grouped latent attention over G*H virtual heads, one per (shard, head))."""
    B, H, d_c = q_lat.shape
    w = d_c // G
    out = np.zeros((B, H, d_c))
    for b in range(B):
        T = int(seq_lens[b])
        if T == 0:
            continue
        c = pool[b, :T, :d_c]
        r = pool[b, :T, d_c:]
        qt = q_lat[b] @ hmat if hmat is not None else q_lat[b]
        q = np.stack([np.concatenate([qt[:, s * w:(s + 1) * w], q_rope[b]], axis=1) for s in range(G)])  # [G,H,w+dr]
        k = np.stack([np.concatenate([c[:, s * w:(s + 1) * w], r], axis=1) for s in range(G)])  # [G,T,w+dr]
        v = np.stack([c[:, s * w:(s + 1) * w] for s in range(G)])  # [G,T,w]
        qq = torch.from_numpy(q).reshape(1, G * H, 1, -1)
        kk = torch.from_numpy(np.repeat(k[:, None], H, axis=1)).reshape(1, G * H, T, -1)
        vv = torch.from_numpy(np.repeat(v[:, None], H, axis=1)).reshape(1, G * H, T, -1)
        o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=scale)
        o = o.reshape(G, H, w).numpy()
        y = np.concatenate([o[s] for s in range(G)], axis=1)
        out[b] = y @ hmat if hmat is not None else y
    return out


def pin_p4_gla_identity(orc):
    """TPLA = GLA with G*H virtual heads, checked against torch SDPA (fp64),
    for G = 1, 2, 4 and with the Hadamard rotation (scipy's Hadamard matrix)."""
    for G in (1, 2, 4):
        pool, seq_lens, q_lat, q_rope = _random_problem(40 + G, d_c=32, d_r=8, lens=(12, 3, 20))
        out, _ = orc.tpla_decode_sharded(pool, None, seq_lens, q_lat, q_rope, 0.25, G)
        ref = _sdpa_gla(pool, seq_lens, q_lat, q_rope, 0.25, G, None)
        assert _rel(out, ref) <= 1e-12, ("P4", G, _rel(out, ref))
        # rotated cache, built by the oracle's append with exact storage
        rows = np.concatenate([pool[b, :seq_lens[b]] for b in range(len(seq_lens))])
        slots = np.concatenate([b * pool.shape[1] + np.arange(seq_lens[b]) for b in range(len(seq_lens))])
        rot = orc.latent_cache_append(np.full_like(pool, np.nan), rows, slots, 32, "wht", "f64")
        out_r, _ = orc.tpla_decode_sharded(rot, None, seq_lens, q_lat, q_rope, 0.25, G, transform="wht")
        hmat = scipy.linalg.hadamard(32).astype(np.float64) / math.sqrt(32)
        rot_ref = pool.copy()
        rot_ref[:, :, :32] = pool[:, :, :32] @ hmat
        ref_r = _sdpa_gla(rot_ref, seq_lens, q_lat, q_rope, 0.25, G, hmat)
        assert _rel(out_r, ref_r) <= 1e-12, ("P4 wht", G, _rel(out_r, ref_r))


# ---------------------------------------------------------------- P5
def pin_p5_hadamard(orc):
    """Sylvester Hadamard: equals scipy.linalg.hadamard(n)/sqrt(n), is
    symmetric and its own inverse; a radix-2 butterfly without bit reversal
    gives the same transform (reading A5)."""
    for n in (1, 2, 4, 8, 64, 512):
        h = orc.hadamard(n)
        ref = scipy.linalg.hadamard(n).astype(np.float64) / math.sqrt(n)
        assert np.array_equal(h.shape, (n, n))
        assert np.max(np.abs(h - ref)) <= 1e-15, n
        assert np.max(np.abs(h - h.T)) == 0.0
        assert np.max(np.abs(h @ h - np.eye(n))) <= 1e-13
    x = np.random.default_rng(5).standard_normal(512)
    y = x.copy()
    span = 1
    while span < 512:
        for start in range(0, 512, 2 * span):
            a = y[start:start + span].copy()
            b = y[start + span:start + 2 * span].copy()
            y[start:start + span] = a + b
            y[start + span:start + 2 * span] = a - b
        span *= 2
    y /= math.sqrt(512)
    assert np.max(np.abs(orc.hadamard(512) @ x - y)) <= 1e-13


# ---------------------------------------------------------------- P6
def pin_p6_closed_forms(orc):
    """Closed forms of softmax attention: one token returns its latent row and
    its own logit as lse; all-zero queries return the mean row with
    lse = ln T; a key that leads by more than 50 in logit returns its row."""
    G = 2
    rng = np.random.default_rng(61)
    d_c, d_r, H = 16, 4, 3
    lat = [rng.standard_normal((1, d_c))]
    rope = [rng.standard_normal((1, d_r))]
    pool, lens = _pool(lat, rope)
    q_lat = rng.standard_normal((1, H, d_c))
    q_rope = rng.standard_normal((1, H, d_r))
    out, lse = orc.tpla_decode_sharded(pool, None, lens, q_lat, q_rope, 0.7, G)
    assert np.array_equal(out[0], np.repeat(lat[0], H, axis=0))
    w = d_c // G
    for s in range(G):
        for h in range(H):
            ell = 0.7 * (sum(q_lat[0, h, j] * lat[0][0, j] for j in range(s * w, (s + 1) * w))
                         + sum(q_rope[0, h, j] * rope[0][0, j] for j in range(d_r)))
            assert abs(lse[0, s, h] - ell) <= 1e-14 * max(1.0, abs(ell))
    # zero queries
    lat = [rng.standard_normal((13, d_c))]
    rope = [rng.standard_normal((13, d_r))]
    pool, lens = _pool(lat, rope)
    out, lse = orc.tpla_decode_sharded(pool, None, lens, np.zeros((1, H, d_c)), np.zeros((1, H, d_r)), 0.7, G)
    mean = lat[0].sum(axis=0) / 13.0
    assert np.max(np.abs(out[0] - mean[None])) <= 1e-15
    assert np.max(np.abs(lse - math.log(13.0))) <= 1e-15
    # one dominant key per shard (lead > 50 after scaling)
    lat0 = rng.standard_normal((9, d_c)) * 0.01
    lat0[4, :] = 0.0
    lat0[4, 0] = 100.0   # shard 0 favours token 4
    lat0[6, w] = 100.0   # shard 1 favours token 6
    pool, lens = _pool([lat0], [np.zeros((9, d_r))])
    q = np.zeros((1, 1, d_c))
    q[0, 0, 0] = 1.0
    q[0, 0, w] = 1.0
    out, _ = orc.tpla_decode_sharded(pool, None, lens, q, np.zeros((1, 1, d_r)), 1.0, G)
    assert np.max(np.abs(out[0, 0, :w] - lat0[4, :w])) <= 1e-18 * 100 + 1e-20
    assert np.max(np.abs(out[0, 0, w:] - lat0[6, w:])) <= 1e-18 * 100 + 1e-20


def pin_p6b_empty_sequence(orc):
    """An empty sequence yields zeros and lse = -inf (reading A10); NaN rows
    outside a sequence's length never reach the result."""
    pool, seq_lens, q_lat, q_rope = _random_problem(62, lens=(0, 5, 0))
    out, lse = orc.tpla_decode_sharded(pool, None, seq_lens, q_lat, q_rope, 0.5, 2)
    assert np.all(out[0] == 0) and np.all(out[2] == 0)
    assert np.all(np.isneginf(lse[0])) and np.all(np.isneginf(lse[2]))
    assert np.all(np.isfinite(out[1])) and np.all(np.isfinite(lse[1]))


# ---------------------------------------------------------------- P7
def pin_p7_not_exact_for_g2(orc):
    """Independent per-shard softmax is not exact MLA ([FR] Directions: the
    feature axis cannot be split exactly because softmax couples the whole
    latent; [REV] skeptic critique, Sec. 4.3.1 Hadamard counterexample).
    Returns the relative difference for the record."""
    pool, seq_lens, q_lat, q_rope = _random_problem(71, d_c=64, d_r=16, lens=(50, 40, 30))
    g1, _ = orc.tpla_decode_sharded(pool, None, seq_lens, q_lat, q_rope, 0.2, 1)
    g2, _ = orc.tpla_decode_sharded(pool, None, seq_lens, q_lat, q_rope, 0.2, 2)
    diff = _rel(g2, g1)
    assert diff > 1e-2, diff
    return diff


# ---------------------------------------------------------------- P8
def pin_p8_softmax_lse_scipy(orc):
    """Per (b, h, shard) the output and lse equal scipy's softmax and
    logsumexp applied to logits formed by explicit loops."""
    G = 2
    pool, seq_lens, q_lat, q_rope = _random_problem(81, B=2, H=3, d_c=16, d_r=4, lens=(11, 6))
    out, lse = orc.tpla_decode_sharded(pool, None, seq_lens, q_lat, q_rope, 0.45, G)
    w = 8
    for b in range(2):
        T = int(seq_lens[b])
        for h in range(3):
            for s in range(G):
                logits = np.array([0.45 * (sum(q_lat[b, h, j] * pool[b, t, j] for j in range(s * w, (s + 1) * w))
                                           + sum(q_rope[b, h, j] * pool[b, t, 16 + j] for j in range(4)))
                                   for t in range(T)])
                p = scipy.special.softmax(logits)
                ref = sum(p[t] * pool[b, t, s * w:(s + 1) * w] for t in range(T))
                assert np.max(np.abs(out[b, h, s * w:(s + 1) * w] - ref)) <= 1e-14
                assert abs(lse[b, s, h] - scipy.special.logsumexp(logits)) <= 1e-13


# ---------------------------------------------------------------- paging and append
def pin_paged_gather(orc):
    """A paged cache with a random block table gives bitwise the same result
    as the contiguous cache holding the same rows."""
    rng = np.random.default_rng(91)
    B, H, d_c, d_r, P = 3, 2, 16, 4, 4
    lens = [9, 4, 0]
    pool, seq_lens = _pool([rng.standard_normal((t, d_c)) for t in lens], [rng.standard_normal((t, d_r)) for t in lens])
    q_lat = rng.standard_normal((B, H, d_c))
    q_rope = rng.standard_normal((B, H, d_r))
    ref, ref_lse = orc.tpla_decode_sharded(pool, None, seq_lens, q_lat, q_rope, 0.3, 2)
    npages = sum((t + P - 1) // P for t in lens) + 2
    perm = rng.permutation(npages)
    paged = np.full((npages, P, d_c + d_r), np.nan)
    table = np.full((B, 3), -1, dtype=np.int32)
    k = 0
    for b, t in enumerate(lens):
        for j in range((t + P - 1) // P):
            table[b, j] = perm[k]
            n = min(P, t - j * P)
            paged[perm[k], :n] = pool[b, j * P:j * P + n]
            k += 1
    out, lse = orc.tpla_decode_sharded(paged, table, seq_lens, q_lat, q_rope, 0.3, 2)
    assert np.array_equal(out, ref) and np.array_equal(lse, ref_lse)


def pin_append(orc):
    """Append writes row i at flat slot i; with the rotation the stored latent
    is the bf16 rounding of scipy-Hadamard times the row (torch's bf16
    conversion of the float32 product, up to one unit in the last place where
    the float32 product sits next to a rounding tie), the rope part is
    copied unchanged."""
    rng = np.random.default_rng(95)
    d_c, d_r = 64, 8
    rows = torch.from_numpy(rng.standard_normal((20, d_c + d_r))).to(torch.bfloat16).to(torch.float64).numpy()
    slots = rng.permutation(24)[:20]
    pool = np.full((6, 4, d_c + d_r), np.nan)
    ident = orc.latent_cache_append(pool, rows, slots, d_c, "identity", "bf16")
    flat = ident.reshape(24, -1)
    assert np.array_equal(flat[slots], rows)
    unused = np.setdiff1d(np.arange(24), slots)
    assert np.all(np.isnan(flat[unused]))
    rot = orc.latent_cache_append(pool, rows, slots, d_c, "wht", "bf16").reshape(24, -1)
    hmat = scipy.linalg.hadamard(d_c).astype(np.float64) / math.sqrt(d_c)
    prod = rows[:, :d_c] @ hmat
    ref = torch.from_numpy(prod.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    got = rot[slots, :d_c]
    ulp = np.ldexp(1.0, np.frexp(ref)[1] - 8)
    assert np.all(np.abs(got - ref) <= ulp)
    assert np.mean(got == ref) > 0.99
    assert np.array_equal(rot[slots, d_c:], rows[:, d_c:])


def pin_p14_rms_norm_in_append(orc):
    """RMSNorm with unit gain in the append ([REV] referee report: Proposition 1,
    RMSNorm under orthogonal transforms; key_machinery: Condition 1, shard RMS
    norms proportional to the global norm):
    * Proposition 1: rotating then normalising the whole latent stores exactly
      H applied to the normalised row (computed here with scipy's Hadamard);
    * each slice of a shard-local norm has mean square m / (m + eps), m the mean
      square of that slice of the rotated row (closed form);
    * when every slice has the same norm (Condition 1 holding exactly), the
      shard-local norm equals the whole-latent norm;
    * with eps = 0 the norm does not depend on the row's scale;
    * the rope part is stored unchanged, and bf16 storage rounds the normalised
      value."""
    rng = np.random.default_rng(141)
    d_c, d_r, n = 64, 8, 6
    rows = rng.standard_normal((n, d_c + d_r)) * np.linspace(0.5, 3.0, d_c + d_r)
    pool = np.full((2, 4, d_c + d_r), np.nan)
    slots = np.arange(n)
    hmat = scipy.linalg.hadamard(d_c).astype(np.float64) / math.sqrt(d_c)

    glob = orc.latent_cache_append(pool, rows, slots, d_c, "wht", "f64", norm_slices=1).reshape(8, -1)[slots]
    x = rows[:, :d_c]
    want = (x / np.sqrt(np.mean(x * x, axis=1, keepdims=True))) @ hmat.T
    assert np.max(np.abs(glob[:, :d_c] - want)) <= 1e-13, "P14 Proposition 1"
    assert np.array_equal(glob[:, d_c:], rows[:, d_c:]), "P14 rope"

    eps = 1e-2
    for transform in ("identity", "wht"):
        loc = orc.latent_cache_append(pool, rows, slots, d_c, transform, "f64", norm_slices=4,
                                      eps=eps).reshape(8, -1)[slots]
        base = x @ hmat.T if transform == "wht" else x
        for s in range(4):
            sl = slice(16 * s, 16 * (s + 1))
            m = np.mean(base[:, sl] ** 2, axis=1)
            got = np.mean(loc[:, sl] ** 2, axis=1)
            assert np.max(np.abs(got - m / (m + eps))) <= 1e-13, ("P14 slice mean square", transform, s)

    u = rng.standard_normal(16)
    eq = np.concatenate([u, -u[::-1], np.roll(u, 3), u * np.tile([1.0, -1.0], 8)])  # four slices, one norm
    eq_rows = np.concatenate([np.stack([eq, 2.5 * eq]), rng.standard_normal((2, d_r))], axis=1)
    a = orc.latent_cache_append(pool, eq_rows, [0, 1], d_c, "identity", "f64", norm_slices=4).reshape(8, -1)[:2]
    b = orc.latent_cache_append(pool, eq_rows, [0, 1], d_c, "identity", "f64", norm_slices=1).reshape(8, -1)[:2]
    assert np.max(np.abs(a - b)) <= 1e-14, "P14 Condition 1 exact"
    assert np.max(np.abs(a[0, :d_c] - a[1, :d_c])) <= 1e-14, "P14 scale invariance"

    bf = orc.latent_cache_append(pool, rows, slots, d_c, "wht", "bf16", norm_slices=2, eps=1e-6).reshape(8, -1)[slots]
    exact = orc.latent_cache_append(pool, rows, slots, d_c, "wht", "f64", norm_slices=2, eps=1e-6).reshape(8, -1)[slots]
    ref = torch.from_numpy(exact[:, :d_c].astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    ulp = np.ldexp(1.0, np.frexp(ref)[1] - 8)
    assert np.all(np.abs(bf[:, :d_c] - ref) <= ulp) and np.mean(bf[:, :d_c] == ref) > 0.99, "P14 rounding"


# ---------------------------------------------------------------- bf16 and golden fixtures
def pin_bf16_rne(orc):
    """Round-to-nearest-even to bfloat16 agrees with torch's conversion on
    float32 inputs, and with the hand-derived cases in golden/bf16_rne.txt."""
    x = np.random.default_rng(7).standard_normal(200000).astype(np.float32) * np.float32(3.0)
    x = np.concatenate([x, x * np.float32(1e30), x * np.float32(1e-30)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(orc.bf16_rne(x.astype(np.float64)), ref)
    with open(os.path.join(GOLDEN, "bf16_rne.txt")) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            src, want = line.split()
            got = float(orc.bf16_rne(np.array([float.fromhex(src)]))[0])
            assert got == float.fromhex(want), (src, want, got)


def pin_golden_hand_cases(orc):
    """Hand-derived decode results in golden/tpla_hand_cases.json."""
    with open(os.path.join(GOLDEN, "tpla_hand_cases.json")) as fh:
        cases = json.load(fh)["cases"]
    for case in cases:
        lat = np.array(case["latent"], dtype=np.float64)
        rope = np.array(case["rope"], dtype=np.float64)
        pool, lens = _pool([lat], [rope])
        q_lat = np.array(case["q_latent"], dtype=np.float64)[None]
        q_rope = np.array(case["q_rope"], dtype=np.float64)[None]
        transform = case.get("transform", "identity")
        if transform == "wht":
            d_c = lat.shape[1]
            slots = np.arange(lat.shape[0])
            pool = orc.latent_cache_append(np.full_like(pool, np.nan), np.concatenate([lat, rope], 1),
                                           slots, d_c, "wht", "f64")
        out, lse = orc.tpla_decode_sharded(pool, None, lens, q_lat, q_rope, case["scale"], case["shards"],
                                           transform=transform)
        want = np.array([[eval(e, {"e": math.e, "ln": math.log, "exp": math.exp, "sqrt": math.sqrt})
                          for e in row] for row in case["expected_out"]])
        assert np.max(np.abs(out[0] - want)) <= 1e-14, (case["name"], out[0], want)
        if "expected_lse" in case:
            want_lse = np.array([[eval(e, {"e": math.e, "ln": math.log, "exp": math.exp})
                                  for e in row] for row in case["expected_lse"]])
            assert np.max(np.abs(lse[0] - want_lse)) <= 1e-14, (case["name"], lse[0], want_lse)


ALL_PINS = [
    pin_p1_absorbed_equals_unabsorbed,
    pin_p1b_bruteforce_closed_form,
    pin_p2_hadamard_invariance_g1,
    pin_p3_shard_decomposition,
    pin_p3b_subset_additivity,
    pin_p4_gla_identity,
    pin_p5_hadamard,
    pin_p6_closed_forms,
    pin_p6b_empty_sequence,
    pin_p7_not_exact_for_g2,
    pin_p8_softmax_lse_scipy,
    pin_p9_value_projection,
    pin_p10_context_split_merge,
    pin_p18_prefill_equals_unabsorbed_causal,
    pin_p18b_prefill_sdpa_causal,
    pin_p18c_prefill_closed_forms,
    pin_paged_gather,
    pin_append,
    pin_p14_rms_norm_in_append,
    pin_bf16_rne,
    pin_golden_hand_cases,
]
