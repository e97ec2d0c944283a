"""Plant plausible mistakes in the oracle (on the CPU, in a temporary copy of one
function) and check that at least one pin fails for each. This shows the pins
are sensitive to the errors they are meant to catch."""
import contextlib
import inspect
import textwrap

import pytest

import oracle.block
import oracle.formats
import oracle.mlp
import oracle.nvfp4
import test_oracle_formats as TF
import test_oracle_mlp as TM
import test_oracle_pack as TP
import test_oracle_block as TB
import test_oracle_w4a4 as TW


@contextlib.contextmanager
def mutated(module, name, old, new):
    src = textwrap.dedent(inspect.getsource(getattr(module, name)))
    assert old in src, f"mutation anchor not found in {name}: {old!r}"
    ns = dict(vars(module))
    exec(compile(src.replace(old, new, 1), f"<mutant {name}>", "exec"), ns)
    orig = getattr(module, name)
    setattr(module, name, ns[name])
    try:
        yield
    finally:
        setattr(module, name, orig)


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


MUTANTS = [
    # (module, function, anchor, replacement, pins that must catch it)
    (oracle.nvfp4, "_quantize_blocks", "code[:, 0::2] | (code[:, 1::2] << 4)", "code[:, 1::2] | (code[:, 0::2] << 4)",
     [TP.test_pack_golden_hand_derived, TP.test_nibble_order_against_brute_weight]),
    (oracle.nvfp4, "_quantize_blocks", "(bamax / F32(6.0)) / gscale", "bamax / gscale",
     [lambda: TP.test_pack_invariants(0), TP.test_pack_golden_hand_derived]),
    (oracle.nvfp4, "pack", "F32(amax / F32(2688.0))", "F32(amax / F32(448.0))",
     [lambda: TP.test_pack_invariants(0), TP.test_pack_golden_hand_derived]),
    (oracle.formats, "e4m3_encode", "np.rint((2.0 * mant - 1.0) * 8.0)", "np.floor((2.0 * mant - 1.0) * 8.0 + 0.5)",
     [TP.test_pack_golden_hand_derived, TF.test_e4m3_encode_matches_torch_cast]),
    (oracle.formats, "e2m1_encode", "up_even = ((i + 1) % 2) == 0", "up_even = True",
     [TF.test_e2m1_encode_vs_nearest_search]),
    (oracle.formats, "e2m1_encode", "np.signbit(q)", "(q < 0)",
     [TF.test_e2m1_encode_vs_nearest_search, TP.test_pack_negative_zero_inside_nonzero_block]),
    (oracle.formats, "minifloat_decode", "frac * 2.0 ** (1 - bias)", "frac * 2.0 ** (-bias)",
     [TF.test_generic_minifloat_matches_torch_e4m3fn_all_bytes, TF.test_e2m1_value_table]),
    (oracle.nvfp4, "dequant_unscaled", "np.repeat(_E4M3_VALUE[np.asarray(scales, np.uint8)], GROUP, axis=-1)",
     "np.tile(_E4M3_VALUE[np.asarray(scales, np.uint8)], GROUP)",
     [TP.test_nibble_order_against_brute_weight]),
    (oracle.mlp, "linear", "s2 * (x @ wu.T)", "s2 * (x @ wu[::-1].T)",
     [lambda: TM.test_linear_vs_brute(2, 3, 32), TM.test_linear_integer_exact]),
    (oracle.mlp, "silu", "z / (1.0 + np.exp(-z))", "z / (1.0 + np.exp(z))",
     [TM.test_linear_gated_vs_brute, TM.test_silu_closed_form_values]),
    (oracle.mlp, "moe", "h = silu(s2g * (xe @ wg.T)) * (s2u * (xe @ wu.T))", "h = silu(s2u * (xe @ wu.T)) * (s2g * (xe @ wg.T))",
     [TM.test_moe_vs_brute]),
    (oracle.mlp, "moe", "y += w[:, j:j + 1] * slots[:, j]", "y += w[:, :1] * slots[:, j]",
     [TM.test_moe_vs_brute]),
    (oracle.mlp, "route", "perm_parts.append(slots)", "perm_parts.append(slots[::-1])",
     [lambda: TM.test_route_vs_stable_argsort_and_brute(20, 3, 5, 10, 0, 30)]),
    # W4A4: the activation's own amax in place of the calibrated scale; a dropped
    # input scale; H quantized against the gate/up scale
    (oracle.nvfp4, "quantize_act", "_quantize_blocks(bf16_to_f32(x_bits), input_scale)",
     "_quantize_blocks(bf16_to_f32(x_bits), F32(np.max(np.abs(bf16_to_f32(x_bits))) / F32(2688.0)))",
     [lambda: TW.test_quantize_act_round_trip_on_grid(1.0), TW.test_quantize_act_saturation_hand_derived]),
    (oracle.mlp, "act_fake_quant", "dequant_unscaled(codes, scales) * F64(np.float32(input_scale))",
     "dequant_unscaled(codes, scales)", [TW.test_moe_w4a4_k1_reduces_to_pinned_dense_pieces]),
    (oracle.mlp, "moe_w4a4", "hq = act_fake_quant(h_bits, in_scale_d)", "hq = act_fake_quant(h_bits, in_scale_gu)",
     [TW.test_moe_w4a4_k1_reduces_to_pinned_dense_pieces]),
    # router and shared expert: ties to the higher index; softmax over all experts;
    # gate and up swapped
    (oracle.block, "topk_softmax", "key=lambda e: (-logits[t, e], e)", "key=lambda e: (-logits[t, e], -e)",
     [TB.test_topk_ties_go_to_the_lower_index]),
    (oracle.block, "topk_softmax", "z = np.exp(sel - sel.max(axis=1, keepdims=True))\n    return ids.astype(np.int32), z / z.sum(axis=1, keepdims=True)",
     "z = np.exp(sel - sel.max(axis=1, keepdims=True))\n    return ids.astype(np.int32), z / np.exp(logits - sel.max(axis=1, keepdims=True)).sum(axis=1, keepdims=True)",
     [lambda: TB.test_topk_matches_stable_argsort(7, 16, 4)]),
    (oracle.block, "shared_mlp", "h = silu(x @ _bf(wg_bits).T) * (x @ _bf(wu_bits).T)", "h = silu(x @ _bf(wu_bits).T) * (x @ _bf(wg_bits).T)",
     [TB.test_shared_mlp_reduces_to_dense_nvfp4_mlp]),
    (oracle.block, "moe_bf16", "slots[tt, jj] = h @ _bf(wd_bits[e]).T", "slots[tt, jj] = h @ _bf(wd_bits[e])[:, ::-1].T",
     [TB.test_moe_bf16_reduces_to_nvfp4_moe_on_exact_weights]),
]


@pytest.mark.parametrize("i", range(len(MUTANTS)))
def test_planted_mistake_is_caught(i):
    module, name, old, new, pins = MUTANTS[i]
    with mutated(module, name, old, new):
        caught = [_fails(p) for p in pins]
    assert any(caught), f"no pin caught the mutant of {name}: {new!r}"
