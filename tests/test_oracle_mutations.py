"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
the pins in test_oracle_pins.py catch every one of them, while an equivalent
rewrite still passes. The real oracle is never modified."""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

# name -> (original text, mutated text, must the pins fail?)
MUTATIONS = {
    "mean_over_D_minus_1": ("axis=-1, keepdims=True) / head_dim",
                            "axis=-1, keepdims=True) / (head_dim - 1)", True),
    "eps_outside_sqrt": ("r = 1.0 / np.sqrt(mean_sq + eps)", "r = 1.0 / (np.sqrt(mean_sq) + eps)", True),
    "one_plus_w": ("return x * r * w", "return x * r * (1 + w)", True),
    "neox_sign_first_half": ("out[..., :half] = a * cos - b * sin", "out[..., :half] = a * cos + b * sin", True),
    "neox_sign_second_half": ("out[..., half:R] = b * cos + a * sin", "out[..., half:R] = b * cos - a * sin", True),
    "interleaved_pair_swapped": ("a, b = n[..., 0:R:2], n[..., 1:R:2]", "b, a = n[..., 0:R:2], n[..., 1:R:2]", True),
    "interleaved_sign": ("out[..., 0:R:2] = a * cos - b * sin", "out[..., 0:R:2] = a * cos + b * sin", True),
    "cos_sin_halves_swapped": ("return row[:, :half], row[:, half:rope_dim]",
                               "return row[:, half:rope_dim], row[:, :half]", True),
    "eps_dropped": ("eps64 = float(np.float32(eps))", "eps64 = 0.0", True),
    "bf16_double_rounding": ("u = _f64_to_f32_round_to_odd(x).view", "u = x.astype(np.float32).view", True),
    "bf16_truncation": ("(u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1)))", "(u)", True),
    "bf16_ties_away": ("(u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1)))",
                       "(u + np.uint64(0x8000))", True),
    "neox_half_from_head_dim": ("    half = R // 2\n    cos = np.asarray(cos",
                                "    half = n.shape[-1] // 2 if is_neox else R // 2\n    cos = np.asarray(cos", True),
    "k_weight_on_q": ("out_q = rope(rms_norm(q, wq, eps64)", "out_q = rope(rms_norm(q, wk, eps64)", True),
    "tail_zeroed": ("    out = n.copy()\n", "    out = np.zeros_like(n)\n", True),
    "position_off_by_one": ("row = cache[p].astype",
                            "row = cache[np.minimum(p + 1, cache.shape[0] - 1)].astype", True),
    "pairing_flag_inverted": ("    if is_neox:\n        a, b = n[..., :half]",
                              "    if not is_neox:\n        a, b = n[..., :half]", True),
    "fp16_double_rounding": ("return x.astype(np.float16).view(np.uint16)",
                             "return x.astype(np.float32).astype(np.float16).view(np.uint16)", True),
    "unfused_k_uses_q_weight": ("nk = rms_norm_io(k_bits, wk_bits", "nk = rms_norm_io(k_bits, wq_bits", True),
    "rope_step_pairing_inverted": ("cos[:, None, :], sin[:, None, :], R, is_neox)\n    return round_to_io_bits(out, dtype)",
                                   "cos[:, None, :], sin[:, None, :], R, not is_neox)\n    return round_to_io_bits(out, dtype)", True),
    "layer_norm_unbiased_variance": ("var = np.sum(c * c, axis=-1, keepdims=True) / head_dim",
                                     "var = np.sum(c * c, axis=-1, keepdims=True) / (head_dim - 1)", True),
    "layer_norm_bias_dropped": ("        out = out + np.asarray(b, dtype=np.float64)", "        out = out", True),
    "layer_norm_not_centered": ("    c = x - mean\n", "    c = x - 0 * mean\n", True),
    "layernorm_io_weights_swapped": ("dec(wq_bits), dec(wk_bits), dec(bq_bits), dec(bk_bits)",
                                     "dec(wk_bits), dec(wq_bits), dec(bq_bits), dec(bk_bits)", True),
    "layernorm_io_biases_swapped": ("dec(wq_bits), dec(wk_bits), dec(bq_bits), dec(bk_bits)",
                                    "dec(wq_bits), dec(wk_bits), dec(bk_bits), dec(bq_bits)", True),
    "layernorm_io_k_weight_on_q": ("dec(wq_bits), dec(wk_bits), dec(bq_bits), dec(bk_bits)",
                                   "dec(wk_bits), dec(wk_bits), dec(bq_bits), dec(bk_bits)", True),
    "layernorm_k_bias_from_q": ("nk = layer_norm(k, wk, bk, eps64)", "nk = layer_norm(k, wk, bq, eps64)", True),
    "layernorm_q_weight_from_k": ("nq = layer_norm(q, wq, bq, eps64)", "nq = layer_norm(q, wk, bq, eps64)", True),
    "layernorm_io_pairing_inverted": ("positions, is_neox=is_neox, eps=eps, rope_dim=rope_dim)\n    return round_to_io_bits(oq",
                                      "positions, is_neox=not is_neox, eps=eps, rope_dim=rope_dim)\n    return round_to_io_bits(oq", True),
    "layernorm_io_eps_dropped": ("positions, is_neox=is_neox, eps=eps, rope_dim=rope_dim)\n    return round_to_io_bits(oq",
                                 "positions, is_neox=is_neox, eps=0.0, rope_dim=rope_dim)\n    return round_to_io_bits(oq", True),
    "equivalent_rewrite": ("np.sum(x * x, axis=-1", "np.sum(np.abs(x) * np.abs(x), axis=-1", False),
}


def _run(name, src, tmp_root):
    a, b, _ = MUTATIONS[name]
    d = os.path.join(tmp_root, name)
    shutil.copytree(os.path.join(ROOT, "tests"), os.path.join(d, "tests"),
                    ignore=shutil.ignore_patterns("__pycache__", "test_oracle_mutations.py"))
    os.makedirs(os.path.join(d, "oracle"))
    open(os.path.join(d, "oracle", "__init__.py"), "w").close()
    with open(os.path.join(d, "oracle", "qknr_oracle.py"), "w") as f:
        f.write(src.replace(a, b, 1))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "tests/test_oracle_pins.py"], cwd=d, capture_output=True, text=True,
                       timeout=600)
    return r.returncode


@pytest.mark.slow
def test_pins_catch_planted_mistakes():
    src = open(os.path.join(ROOT, "oracle", "qknr_oracle.py")).read()
    for name, (a, _, _) in MUTATIONS.items():
        assert src.count(a) >= 1, f"mutation site for {name} no longer in the oracle"
    tmp = tempfile.mkdtemp(prefix="qknr_mut_")
    try:
        with cf.ThreadPoolExecutor(4) as ex:
            rcs = dict(zip(MUTATIONS, ex.map(lambda n: _run(n, src, tmp), MUTATIONS)))
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    missed = [n for n, (_, _, must) in MUTATIONS.items() if must and rcs[n] == 0]
    false_alarm = [n for n, (_, _, must) in MUTATIONS.items() if not must and rcs[n] != 0]
    assert not missed, f"pins missed planted mistakes: {missed}"
    assert not false_alarm, f"pins rejected an equivalent rewrite: {false_alarm}"
