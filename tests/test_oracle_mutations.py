"""Plant mistakes in a copy of the oracle (on the CPU) and check the pins catch each one.

A pin set that passes a broken oracle would not pin anything; every planted
mistake below must make at least one pin fail.
"""

import os
import types

import pytest

from oracle_pins import ALL_PINS

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "tpla_oracle.py")

MUTATIONS = {
    "drop_rope_logit": ("@ c_lat[:, cols].T + rope_logits)", "@ c_lat[:, cols].T)"),
    "drop_scale": ("logits = scale * (", "logits = 1.0 * ("),
    "scale_only_latent": ("logits = scale * (q_tilde[:, cols] @ c_lat[:, cols].T + rope_logits)",
                          "logits = scale * (q_tilde[:, cols] @ c_lat[:, cols].T) + rope_logits"),
    "wrong_slice": ("cols = slice(s * w, (s + 1) * w)", "cols = slice(0, w)"),
    "hadamard_not_symmetric": ("base = np.array([[1.0, 1.0], [1.0, -1.0]])", "base = np.array([[1.0, 1.0], [-1.0, 1.0]])"),
    "hadamard_bad_norm": ("return h / np.sqrt(n)", "return h / n"),
    "no_output_unrotation": ("out[b] = y @ hmat if hmat is not None else y", "out[b] = y"),
    "no_query_rotation": ("q_tilde = q_lat[b] @ hmat if hmat is not None else q_lat[b]", "q_tilde = q_lat[b]"),
    "lse_without_max": ("lse[b, i] = (m + np.log(z))[:, 0]", "lse[b, i] = np.log(z)[:, 0]"),
    "no_normalisation": ("y[:, cols] = (p @ c_lat[:, cols]) / z", "y[:, cols] = (p @ c_lat[:, cols])"),
    "max_wrong_axis": ("m = logits.max(axis=1, keepdims=True)", "m = logits.max(axis=0, keepdims=True)"),
    "sum_wrong_axis": ("z = p.sum(axis=1, keepdims=True)", "z = p.sum(axis=0, keepdims=True)"),
    "gather_wrong_offset": ("rows[t] = pool[page, t % page_size]", "rows[t] = pool[page, (t + 1) % page_size]"),
    "gather_wrong_page": ("int(block_table[b][t // page_size])", "int(block_table[b][t % page_size])"),
    "bf16_truncates": ("y = np.rint(x[finite] / quantum) * quantum", "y = np.trunc(x[finite] / quantum) * quantum"),
    "bf16_wrong_precision": ("q_exp = np.maximum(e - 8, -133)", "q_exp = np.maximum(e - 9, -133)"),
    "append_drops_rope": ("flat[slots, d_latent:] = rows[:, d_latent:]", "flat[slots, d_latent:] = 0.0"),
    "append_no_rounding": ("flat[slots, :d_latent] = _store(lat, dtype) if", "flat[slots, :d_latent] = lat if"),
    "shard_output_summed_not_placed": ("y[:, cols] = (p @ c_lat[:, cols]) / z", "y[:, :w] += (p @ c_lat[:, cols]) / z"),
    "rope_from_latent": ("k_rope = rows[:, d_c:]", "k_rope = rows[:, :d_c][:, :rows.shape[1] - d_c]"),
    "projection_transposed_weight": ("out_latent[:, h, :] @ w_uv[h].T", "out_latent[:, h, :] @ w_uv[h][:, ::-1].T"),
    "projection_wrong_head": ("out_latent[:, h, :] @ w_uv[h].T", "out_latent[:, h, :] @ w_uv[(h + 1) % heads].T"),
    "merge_weight_without_lse": ("y[cols] += np.exp(l[p] - lse[b, i, h]) * ys[p][cols]", "y[cols] += ys[p][cols] / parts"),
    "merge_no_unrotation": ("ys = [out_parts[p, b, h] @ hmat if hmat is not None else out_parts[p, b, h] for p in range(parts)]",
                            "ys = [out_parts[p, b, h] for p in range(parts)]"),
    "merge_lse_without_max": ("lse[b, i, h] = m + np.log(z)", "lse[b, i, h] = np.log(z)"),
    "norm_sum_not_mean": ("np.mean(part * part, axis=-1, keepdims=True) + eps", "np.sum(part * part, axis=-1, keepdims=True) + eps"),
    "norm_ignores_slices": ("lat = rms_normalize(lat, norm_slices, eps)", "lat = rms_normalize(lat, 1, eps)"),
    "norm_before_rotation": ("lat = rows[:, :d_latent] @ hadamard(d_latent) if transform == \"wht\" else rows[:, :d_latent]",
                             "lat = rows[:, :d_latent]\n    lat = rms_normalize(lat, norm_slices, eps) if norm_slices else lat\n"
                             "    lat = lat @ hadamard(d_latent) if transform == \"wht\" else lat"),
    "norm_eps_outside_root": ("part / np.sqrt(np.mean(part * part, axis=-1, keepdims=True) + eps)",
                              "part / (np.sqrt(np.mean(part * part, axis=-1, keepdims=True)) + eps)"),
    "prefill_off_by_one": ("visible = length - n_new + j + 1", "visible = length - n_new + j"),
    "prefill_no_causal_mask": ("visible = length - n_new + j + 1", "visible = length"),
    "prefill_wrong_query_row": ("r = r0 + j\n", "r = j\n"),
    "prefill_no_unrotation": ("out[r] = o @ hmat if hmat is not None else o", "out[r] = o"),
    "empty_lse_zero": ("lse = np.full((batch, shard_count, heads), -np.inf, dtype=np.float64)",
                       "lse = np.full((batch, shard_count, heads), 0.0, dtype=np.float64)"),
}


def _mutant(name):
    with open(SRC_PATH) as fh:
        src = fh.read()
    old, new = MUTATIONS[name]
    assert src.count(old) >= 1, f"mutation {name} no longer matches the oracle source"
    src = src.replace(old, new)
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src, f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name):
    mod = _mutant(name)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except Exception as exc:  # an assertion or a crash both count as caught
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, f"no pin catches the planted mistake {name!r}"
