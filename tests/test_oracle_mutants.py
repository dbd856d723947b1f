"""Plant plausible mistakes in the oracle (on the CPU) and check that some pin
catches each one.  A mutant is the oracle function's own source with one
textual change, compiled into the oracle module's namespace for the duration
of the test."""
import inspect
import textwrap

import pytest

import oracle
import oracle.attention as oatt
import oracle.quant as oq
import pins


def _mutate(monkeypatch, module, name, old, new):
    src = textwrap.dedent(inspect.getsource(getattr(module, name)))
    assert src.count(old) >= 1, f"mutation anchor not found in {name}: {old!r}"
    ns = dict(module.__dict__)
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), ns)
    fn = ns[name]
    fn.__globals__.update({k: v for k, v in module.__dict__.items() if k not in fn.__globals__})
    monkeypatch.setattr(module, name, fn)
    if hasattr(oracle, name):
        monkeypatch.setattr(oracle, name, fn)
    # functions in the same module must see the mutant too
    for other in (oq, oatt):
        if hasattr(other, name):
            monkeypatch.setattr(other, name, fn)


def _some_pin_fails(checks):
    for chk in checks:
        try:
            chk()
        except (AssertionError, ValueError, IndexError):
            return True
    return False


QUANT_PINS = [pins.check_quant_closed_forms, pins.check_quant_bruteforce, pins.check_pack_literals,
              pins.check_layout_literals, pins.check_column_permutation_invariance,
              pins.check_quantize_pack_slots, pins.check_grouped_quantize_pack]
DECODE_PINS = [pins.check_decode_vs_sdpa, pins.check_inverse_rotation_direction,
               pins.check_rotated_space_identity, pins.check_decode_special_cases,
               pins.check_decode_invariances, pins.check_partition_merge, pins.check_bf16_paged_vs_sdpa,
               pins.check_decode_vs_sdpa_grouped]

MUTANTS = [
    # (module, function, anchor, replacement, pins)
    (oq, "rotate_round_f32", ".astype(np.float64))", ".astype(np.float64).T)", QUANT_PINS),
    (oq, "quantize_group", "/ np.float32(3.0)", "/ np.float32(4.0)", QUANT_PINS),
    (oq, "quantize_group", "np.rint(t)", "np.floor(t)", QUANT_PINS),
    (oq, "quantize_group", "yc = np.minimum(np.maximum(y, -tau), tau)", "yc = y", QUANT_PINS),
    (oq, "quantize_group", "zero16 = mn.astype(np.float16)", "zero16 = (mn * 0).astype(np.float16)", QUANT_PINS),
    (oq, "quantize_rows_grouped", ".reshape(n * ng, group)", ".reshape(group, n * ng).T", QUANT_PINS),
    (oq, "quantize_pack_ref", "sz_pool[page, g, j * PAGE + off, 0]", "sz_pool[page, g, off * ng + j, 0]",
     QUANT_PINS),
    (oq, "pack_codes_row", "(c[..., 1::4] << 2)", "(c[..., 1::4] << 4)", QUANT_PINS),
    (oq, "k_byte_offsets", "(i // w) * (PAGE * w) + o * w + (i % w)", "o * (d // 4) + i", QUANT_PINS),
    (oq, "v_byte_offsets", "i * PAGE + o", "o * (d // 4) + i", QUANT_PINS),
    (oatt, "dequant_history", "return z + code_levels", "return 0 * z + code_levels", DECODE_PINS),
    (oatt, "dequant_history", "t % PAGE, g, d)", "(t + 1) % PAGE, g, d)", DECODE_PINS),
    (oatt, "dequant_history", "np.repeat(z, d // ng, axis=1), np.repeat(s, d // ng, axis=1)",
     "np.tile(z, (1, d // ng)), np.tile(s, (1, d // ng))", DECODE_PINS),
    (oatt, "decode_attn_ref", "xk @ Rk.T", "xk @ Rk", DECODE_PINS),
    (oatt, "decode_attn_ref", "xv @ Rv.T", "xv @ Rv", DECODE_PINS),
    (oatt, "decode_attn_ref", "range(g * G, (g + 1) * G)", "range(g, Hq, n_kv)", DECODE_PINS),
    (oatt, "decode_attn_ref", 'bf16_to_f64(cfg["sink_k"][b, g, : sl[b]]), ', "", DECODE_PINS),
    (oatt, "attn_plain", "* np.float64(sm_scale)", "", DECODE_PINS),
    (oatt, "merge_partials", "w = np.where(np.isfinite(ms), np.exp(ms - Msafe), 0.0)",
     "w = np.where(np.isfinite(ms), 1.0, 0.0)", DECODE_PINS),
]


@pytest.mark.parametrize("module,name,old,new,checks", MUTANTS,
                         ids=[f"{m[1]}:{i}" for i, m in enumerate(MUTANTS)])
def test_mutant_is_caught(monkeypatch, module, name, old, new, checks):
    _mutate(monkeypatch, module, name, old, new)
    assert _some_pin_fails(checks), f"no pin catches the mutant {name}: {old!r} -> {new!r}"


def test_unmutated_oracle_passes_all_pins():
    for chk in QUANT_PINS + DECODE_PINS:
        chk()
