"""Planted-mistake check of the oracle (CPU).

Each mutant below rewrites one expression of one oracle function into a plausible mistake -- a
dropped term, a flipped sign, a wrong constant, index, tie rule or rounding -- and at least one of
the pins listed beside it must fail while the mutant is in place.  That the pins pass on the
unmutated oracle is checked first, so a pin that errors for an unrelated reason cannot count as a
catch.

Mechanics: the function's source is recompiled with the one substitution (which must occur
exactly once) in its own module's namespace, and every module attribute of the oracle and of the
pin modules that refers to the original function is rebound to the mutant for the duration of
the case, then restored.
"""
import importlib
import inspect
import sys
import textwrap

import pytest

from conftest import load_golden

# (id, module, function, original text, mutated text, pins); a pin is (test module, test
# function, keyword arguments)
MUTANTS = [
    # number formats (formats.py)
    ("e4m3_bias", "oracle.formats", "e4m3_decode", "(e - 7).astype", "(e - 8).astype",
     [("test_oracle_formats", "test_e4m3_decode_matches_torch_all_codes", {})]),
    ("e4m3_subnormal_step", "oracle.formats", "e4m3_decode", "m * 2.0 ** -9", "m * 2.0 ** -10",
     [("test_oracle_formats", "test_e4m3_decode_matches_torch_all_codes", {})]),
    ("e4m3_tie_odd", "oracle.formats", "e4m3_encode", "(hi % 2 == 0)", "(hi % 2 == 1)",
     [("test_oracle_formats", "test_e4m3_encode_matches_torch_in_range", {})]),
    ("e4m3_sign_dropped", "oracle.formats", "e4m3_encode", "np.where(neg, code | 0x80, code)",
     "np.where(neg, code, code)", [("test_oracle_formats", "test_e4m3_encode_matches_torch_in_range", {})]),
    ("bf16_one_bit_short", "oracle.formats", "bf16_round", "np.maximum(e - 8, -133)", "np.maximum(e - 9, -133)",
     [("test_oracle_formats", "test_bf16_round_matches_torch", {})]),
    ("e2m1_bias", "oracle.formats", "e2m1_decode", "(e - 1).astype", "e.astype",
     [("test_oracle_mx4", "test_e2m1_value_table", {})]),
    ("e2m1_tie_odd", "oracle.formats", "e2m1_encode", "(hi % 2 == 0)", "(hi % 2 == 1)",
     [("test_oracle_mx4", "test_e2m1_encode_brute_force", {})]),
    # ExpCast (expcast.py) and its closed forms (analysis.py)
    ("expcast_beta_sign", "oracle.expcast", "expcast_code", "u + C_F32", "u + np.float32(120.35)",
     [("test_oracle_expcast", "test_worked_example", {}),
      ("test_oracle_expcast", "test_same_byte_fraction_over_a_doubling", {})]),
    ("expcast_clip_126", "oracle.expcast", "expcast_code", "np.clip(r, 0.0, 120.0)", "np.clip(r, 0.0, 126.0)",
     [("test_oracle_expcast", "test_specials", {}), ("test_oracle_expcast", "test_constants", {})]),
    ("expcast_floor", "oracle.expcast", "expcast_code", "r = np.rint(t)", "r = np.floor(t)",
     [("test_oracle_expcast", "test_worked_example", {})]),
    ("exp_then_cast_scale", "oracle.expcast", "exp_then_cast_code", "np.exp2(u + 8.0)", "np.exp2(u + 7.0)",
     [("test_oracle_expcast", "test_worked_example", {}),
      ("test_oracle_expcast", "test_same_byte_fraction_over_a_doubling", {})]),
    ("mitchell_dropped_one", "oracle.analysis", "mitchell_e", "(np.exp2(f) - 1.0)", "np.exp2(f)",
     [("test_oracle_expcast", "test_mitchell_error_and_minimax_shift", {})]),
    ("ratio_beta_sign", "oracle.analysis", "ratio_r", "8.0 * f + beta", "8.0 * f - beta",
     [("test_oracle_expcast", "test_ratio_bounds", {}),
      ("test_oracle_expcast", "test_ratio_formula_matches_code_decode", {})]),
    ("tv_bound_no_sqrt", "oracle.analysis", "tv_bound", "(np.sqrt(b) - np.sqrt(a)) / (np.sqrt(b) + np.sqrt(a))",
     "(b - a) / (b + a)", [("test_oracle_expcast", "test_tv_bound", {})]),
    ("energy_share_no_bv", "oracle.analysis", "block_energy_split", "share = Bv * float(mu @ mu)",
     "share = float(mu @ mu)", [("test_oracle_expcast", "test_energy_identity_eq5", {})]),
    ("eq2_value_term_p", "oracle.analysis", "output_error_split", "Pq @ (V - Vq)", "P @ (V - Vq)",
     [("test_oracle_attention", "test_output_error_split_eq2", {})]),
    ("diam_halved", "oracle.analysis", "diam2", "np.sqrt(max(d2.max(), 0.0))", "np.sqrt(max(d2.max(), 0.0)) / 2",
     [("test_oracle_expcast", "test_diam2_closed_form", {})]),
    # attention (attention.py)
    ("exact_no_scale", "oracle.attention", "attention_exact", "S = (Q[i0:i0 + 256] @ K.T) * scale",
     "S = (Q[i0:i0 + 256] @ K.T)", [("test_oracle_attention", "test_exact_attention_matches_torch_sdpa", {})]),
    ("alpha_sign", "oracle.attention", "attention_tiled", "np.exp2((m - m_new) / 8.0)", "np.exp2((m_new - m) / 8.0)",
     [("test_oracle_attention", "test_tiled_recurrence_exact_mode_equals_exact_attention", {"demean": False}),
      ("test_oracle_attention", "test_tiled_probabilities_are_the_pinned_codes", {"p_mode": "expcast"})]),
    ("mean_term_dropped", "oracle.attention", "attention_tiled", " + r[:, None] * mu_t[j][None, :]", "",
     [("test_oracle_attention", "test_tiled_recurrence_exact_mode_equals_exact_attention", {"demean": True})]),
    ("expcast_b_without_beta", "oracle.attention", "attention_tiled", "b = fl32(C_F32 - fl32(m_new))",
     "b = fl32(np.float32(120.0) - fl32(m_new))",
     [("test_oracle_attention", "test_tiled_probabilities_are_the_pinned_codes", {"p_mode": "expcast"})]),
    ("epilogue_without_sv", "oracle.attention", "attention_tiled",
     "O = (A * np.asarray(sV, dtype=np.float64)[None, :]) / l[:, None]", "O = A / l[:, None]",
     [("test_oracle_attention", "test_tiled_recurrence_exact_mode_equals_exact_attention", {"demean": True})]),
    ("expcast_half_slope", "oracle.attention", "attention_tiled", "t = fl32(a64[:, None] * s + b[:, None])",
     "t = fl32(0.5 * a64[:, None] * s + b[:, None])",
     [("test_oracle_attention", "test_tiled_expcast_rows_obey_prop31", {}),
      ("test_oracle_attention", "test_tiled_probabilities_are_the_pinned_codes", {"p_mode": "expcast"})]),
    ("exp_cast_slope", "oracle.attention", "attention_tiled", "y.astype(np.float64) / 8.0 + 8.0",
     "y.astype(np.float64) / 4.0 + 8.0",
     [("test_oracle_attention", "test_tiled_probabilities_are_the_pinned_codes", {"p_mode": "exp_cast"}),
      ("test_oracle_attention", "test_tiled_exp_cast_rows_obey_e4m3_tv_bound", {})]),
    ("running_max_per_tile", "oracle.attention", "attention_tiled",
     "m_new = np.maximum(m, xhat)\n            b = ", "m_new = xhat\n            b = ",
     [("test_oracle_attention", "test_tiled_probabilities_are_the_pinned_codes", {"p_mode": "expcast"})]),
    ("rowsum_drops_a_key", "oracle.attention", "attention_tiled", "r = P.sum(axis=1)", "r = P[:, 1:].sum(axis=1)",
     [("test_oracle_attention", "test_tiled_recurrence_exact_mode_equals_exact_attention", {"demean": False})]),
    ("slope_applied_twice", "oracle.attention", "attention_tiled", "qa = fl32(sQr)",
     "qa = fl32(np.float32(L) * fl32(sQr))",
     [("test_oracle_attention", "test_prescaled_query_operand_equals_raw_query_path", {}),
      ("test_oracle_attention", "test_tiled_expcast_rows_obey_prop31_prescaled_query", {})]),
    # V-Smooth (vsmooth.py)
    ("kmeans_ties_high", "oracle.vsmooth", "kmeans_assign", "np.argmin(sq_distances(V, C), axis=1)",
     "(np.asarray(C).shape[0] - 1 - np.argmin(sq_distances(V, C)[:, ::-1], axis=1))",
     [("test_oracle_vsmooth", "test_kmeans_ties_and_empty_clusters", {})]),
    ("kmeans_empty_to_zero", "oracle.vsmooth", "kmeans_update", "C[nz] = sums[nz] / counts[nz, None]",
     "C = sums / np.maximum(counts, 1)[:, None]", [("test_oracle_vsmooth", "test_kmeans_ties_and_empty_clusters", {})]),
    ("kmeans_objective_l1", "oracle.vsmooth", "kmeans_objective", "float((diff * diff).sum())",
     "float(np.abs(diff).sum())", [("test_oracle_vsmooth", "test_kmeans_fixed_point_properties", {})]),
    ("kmeans_no_update", "oracle.vsmooth", "kmeans_lloyd", "C = kmeans_update(V, labels, C)", "C = C",
     [("test_oracle_vsmooth", "test_kmeans_fixed_point_properties", {})]),
    ("init_rows_unshifted", "oracle.vsmooth", "kmeans_init_strided", "((2 * np.arange(k) + 1) * N) // (2 * k)",
     "(np.arange(k) * N) // k", [("test_oracle_vsmooth", "test_strided_init_rows", {})]),
    ("sort_unstable", "oracle.vsmooth", "stable_argsort", 'kind="stable"', 'kind="quicksort"',
     [("test_oracle_vsmooth", "test_stable_sort_against_bucket_sort", {})]),
    ("offsets_shifted", "oracle.vsmooth", "cluster_offsets", "np.cumsum(counts)]", "np.cumsum(counts) - 1]",
     [("test_oracle_vsmooth", "test_stable_sort_against_bucket_sort", {})]),
    ("pow2_scale_boundary", "oracle.vsmooth", "pow2_scale", "amax <= np.ldexp(E4M3_MAX, E - 1)",
     "amax < np.ldexp(E4M3_MAX, E - 1)", [("test_oracle_vsmooth", "test_pow2_block_scale_definition", {})]),
    ("key_mean_n_minus_1", "oracle.vsmooth", "key_channel_mean", "K.sum(0) / K.shape[0]",
     "K.sum(0) / (K.shape[0] - 1)", [("test_oracle_vsmooth", "test_key_channel_mean_closed_form", {})]),
    ("k_not_centred", "oracle.vsmooth", "quantize_k", "Ks = (Kp - kbar[None, :]).astype(np.float32)",
     "Ks = Kp.astype(np.float32)", [("test_oracle_vsmooth", "test_permuted_quantisers_blocks", {})]),
    ("k_rotation_scale_sqrt", "oracle.vsmooth", "quantize_k", "(s / np.float32(Ks.shape[1]))",
     "(s / np.float32(np.sqrt(Ks.shape[1])))",
     [("test_oracle_rotation", "test_rotated_quantisers_reproduce_the_centred_scores", {"hadamard": True})]),
    ("q_without_slope", "oracle.vsmooth", "quantize_q", "X = (fl32(Q) * L).astype(np.float32)",
     "X = fl32(Q).astype(np.float32)", [("test_oracle_vsmooth", "test_q_quantiser_folds_log2e_scale", {})]),
    ("block_mean_bv_minus_1", "oracle.vsmooth", "block_means", ".sum(1) / BV", ".sum(1) / (BV - 1)",
     [("test_oracle_vsmooth", "test_quantize_v_demeaning", {})]),
    ("sv_over_raw_v", "oracle.vsmooth", "quantize_v", "sV = _scale_from_amax(np.abs(R).max(axis=0))",
     "sV = _scale_from_amax(np.abs(Vp).max(axis=0))", [("test_oracle_vsmooth", "test_quantize_v_demeaning", {})]),
    ("mu_not_divided_by_sv", "oracle.vsmooth", "quantize_v", "mu_t = bf16_round(mu / sV[None, :])",
     "mu_t = bf16_round(mu)", [("test_oracle_vsmooth", "test_quantize_v_demeaning", {})]),
    ("zero_amax_scale", "oracle.vsmooth", "_scale_from_amax",
     "return np.where(amax == 0, np.float32(1.0), s).astype(np.float32)", "return s.astype(np.float32)",
     [("test_oracle_vsmooth", "test_quantize_v_zero_residual_and_constant_block", {})]),
    # QK rotation (rotation.py)
    ("hadamard_block_order", "oracle.rotation", "hadamard", "np.block([[H, H], [H, -H]])",
     "np.block([[H, H], [-H, H]])", [("test_oracle_rotation", "test_hadamard_matches_library", {"n": 4})]),
    ("rotate_orthonormal", "oracle.rotation", "rotate", "X.astype(np.float64) @ H)",
     "X.astype(np.float64) @ H / np.sqrt(X.shape[-1]))", [("test_oracle_rotation", "test_rotate_special_vectors", {})]),
    # 4-bit path (mx4.py)
    ("mx_exponent_floor", "oracle.mx4", "mx_exponent", "np.maximum(E, -100)", "np.maximum(E, -90)",
     [("test_oracle_mx4", "test_mx_exponent_examples", {"amax": 1e-40, "E": -100})]),
    ("key_group_bit3", "oracle.mx4", "key_group", "return 2 * (k // 64) + ((k >> 2) & 1)",
     "return 2 * (k // 64) + ((k >> 3) & 1)",
     [("test_oracle_mx4", "test_key_groups_are_the_pv_operand_slot_groups", {})]),
    ("p4_row_max", "oracle.mx4", "quantize_p4", "mx_exponent(P[:, cols].max(axis=1), fmt)", "mx_exponent(P.max(axis=1), fmt)",
     [("test_oracle_mx4", "test_quantize_p4_brute_force", {})]),
    ("mx4_alpha_sign", "oracle.mx4", "attention_tiled_mx4", "alpha = np.exp2(m - m_new)", "alpha = np.exp2(m_new - m)",
     [("test_oracle_mx4", "test_tiled_exact_mode_is_exact_attention", {})]),
    ("mx4_p_unquantised", "oracle.mx4", "attention_tiled_mx4",
     "P = quantize_p4(fl32(np.exp2(fl32(s - m_new[:, None]).astype(np.float64))), fmt)",
     "P = fl32(np.exp2(fl32(s - m_new[:, None]).astype(np.float64))).astype(np.float64)",
     [("test_oracle_mx4", "test_mx4_recurrence_closed_form", {})]),
    ("mx4_mean_term_dropped", "oracle.mx4", "attention_tiled_mx4", " + r[:, None] * mu_b[j][None, :]", "",
     [("test_oracle_mx4", "test_tiled_exact_mode_is_exact_attention", {})]),
    ("v4_signed_max", "oracle.mx4", "quantize_v4", "mx_exponent(np.abs(R[:, rows, :]).max(axis=1), fmt)",
     "mx_exponent(R[:, rows, :].max(axis=1), fmt)", [("test_oracle_mx4", "test_v4_quantiser_groups_and_bound", {})]),
    ("q4_without_slope", "oracle.mx4", "quantize_q4", "X = (fl32(Q) * log2e_scale4(softmax_scale, Q.shape[1])).astype(np.float32)",
     "X = fl32(Q).astype(np.float32)", [("test_oracle_mx4", "test_q4_k4_quantisers_fold_slope_and_centre", {})]),
    ("k4_not_centred", "oracle.mx4", "quantize_k4", "Ks = (Kp - kbar[None, :]).astype(np.float32)",
     "Ks = Kp.astype(np.float32)", [("test_oracle_mx4", "test_q4_k4_quantisers_fold_slope_and_centre", {})]),
    ("k4_rotation_exponent", "oracle.mx4", "quantize_k4", "return codes, E - 7", "return codes, E",
     [("test_oracle_mx4", "test_k4_rotated_keys_are_the_centred_keys_times_h_over_d", {})]),
    ("e2m3_mantissa_step", "oracle.formats", "e2m3_decode", "np.ldexp(1.0 + m / 8.0", "np.ldexp(1.0 + m / 4.0",
     [("test_oracle_mx6", "test_e2m3_value_table", {})]),
    ("e2m3_tie_odd", "oracle.formats", "e2m3_encode", "(hi % 2 == 0)", "(hi % 2 == 1)",
     [("test_oracle_mx6", "test_e2m3_encode_brute_force", {})]),
    # diagnostics
    ("cube_inner_first", "oracle.diagnostics", "static_cube_order", "np.lexsort((inner, cid))",
     "np.lexsort((cid, inner))", [("test_oracle_diagnostics", "test_static_cube_order_is_a_permutation_of_whole_cubes", {})]),
    ("share_of_residual", "oracle.diagnostics", "block_mean_share", "block_energy_split(Vp[j * BV:(j + 1) * BV])[4]",
     "block_energy_split(Vp[j * BV:(j + 1) * BV])[3]", [("test_oracle_diagnostics", "test_block_mean_share_extremes", {})]),
    ("dequant_without_mean", "oracle.diagnostics", "dequantized_v", "(codes + mu_rows)", "codes",
     [("test_oracle_diagnostics", "test_value_error_of_grid_values_is_zero_and_bounded_otherwise", {})]),
    ("value_error_unpermuted", "oracle.diagnostics", "value_rel_mse", "Vp = fl32(V[perm])", "Vp = fl32(V)",
     [("test_oracle_diagnostics", "test_value_error_falls_with_value_grouping", {}),
      ("test_oracle_diagnostics", "test_value_error_of_grid_values_is_zero_and_bounded_otherwise", {})]),
    ("eq2_value_term_sign", "oracle.diagnostics", "output_error_terms", "np.linalg.norm(PqV - Oq)",
     "np.linalg.norm(PqV + Oq)", [("test_oracle_diagnostics", "test_eq2_terms_add_up_and_value_term_vanishes_on_grid_values", {})]),
    ("tv_natural_exp", "oracle.diagnostics", "row_tv", "p = np.exp2(u)", "p = np.exp(u)",
     [("test_oracle_diagnostics", "test_row_tv_obeys_prop31_and_the_e4m3_bound", {})]),
]

_PIN_OK = {}


def _run_pin(pin):
    mod_name, fn_name, kwargs = pin
    fn = getattr(importlib.import_module(mod_name), fn_name)
    kw = dict(kwargs)
    if "golden" in inspect.signature(fn).parameters:
        kw["golden"] = load_golden
    fn(**kw)


def _pin_passes_unmutated(pin):
    key = (pin[0], pin[1], tuple(sorted(pin[2].items())))
    if key not in _PIN_OK:
        _run_pin(pin)          # raises (and fails the case) if the pin is broken on its own
        _PIN_OK[key] = True
    return True


def _rebind(orig, new):
    """Point every reference to `orig` in the oracle and pin modules at `new`; returns the undo list."""
    undo = []
    for m in list(sys.modules.values()):
        name = getattr(m, "__name__", "") or ""
        if not (name == "oracle" or name.startswith("oracle.") or name.startswith("test_oracle")):
            continue
        for attr, val in list(vars(m).items()):
            if val is orig:
                setattr(m, attr, new)
                undo.append((m, attr))
    return undo


def _make_mutant(mod_name, fn_name, old, new):
    mod = importlib.import_module(mod_name)
    orig = getattr(mod, fn_name)
    src = textwrap.dedent(inspect.getsource(orig))
    assert src.count(old) == 1, f"{mod_name}.{fn_name}: the mutated text must occur exactly once"
    ns = {}
    exec(compile(src.replace(old, new), f"<mutant of {mod_name}.{fn_name}>", "exec"), mod.__dict__, ns)
    return orig, ns[fn_name]


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("mid,mod_name,fn_name,old,new,pins", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_fails_a_pin(mid, mod_name, fn_name, old, new, pins):
    for pin in pins:
        for m in set(p[0] for p in pins):
            importlib.import_module(m)
        assert _pin_passes_unmutated(pin)
    orig, mutant = _make_mutant(mod_name, fn_name, old, new)
    undo = _rebind(orig, mutant)
    assert undo, "the mutant was bound nowhere"
    caught = []
    try:
        for pin in pins:
            try:
                _run_pin(pin)
            except Exception as e:   # an assertion of the pin, or the mutant breaking its caller
                caught.append((pin[1], type(e).__name__))
    finally:
        for m, attr in undo:
            setattr(m, attr, orig)
    assert caught, f"mutant {mid} passed every listed pin"


def test_every_oracle_module_is_mutated():
    mods = {m[1] for m in MUTANTS}
    assert mods == {"oracle.formats", "oracle.expcast", "oracle.analysis", "oracle.attention",
                    "oracle.vsmooth", "oracle.rotation", "oracle.mx4", "oracle.diagnostics"}
