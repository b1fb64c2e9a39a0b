"""Each plausible mistake planted in a copy of the oracle's C source must
make at least one oracle pin fail. The mutants are built on the CPU into a
temporary directory; the real oracle is never modified."""
import os
import subprocess
import sys
import tempfile

import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import oracle  # noqa: E402
from oracle_pins import ALL_CHECKS  # noqa: E402

# (name, text in oracle.c, replacement)
MUTANTS = [
    ("shard_floor", "shard += 1;                     /* ceiling */", ";"),
    ("pad_not_zeroed", "memset(out + off * elem_size, 0,", "(void)(out + off * elem_size), (void)(0,"),
    ("flatten_drops_last", "for (int32_t t = 0; t < ntensors; t++) {\n        if (numels[t] < 0)",
     "for (int32_t t = 0; t < ntensors - 1; t++) {\n        if (numels[t] < 0)"),
    ("bf16_truncate", "hi += 1;                                     /* carries into exponent */", ";"),
    ("bf16_ties_away", "(lo == 0x8000u && (hi & 1u))", "(lo == 0x8000u)"),
    ("bf16_nan_not_quiet", "return (uint16_t)(hi | 0x0040u);", "return (uint16_t)(hi);"),
    ("reduce_skips_rank0", "float s = grad_at(reps[0], is_bf16, idx);", "float s = 0.0f;"),
    ("reduce_no_average", "return s / nf;", "return s;"),
    ("m_unfused", "float mm = fmaf(g, c1, *m * b1);", "float mm = g * c1 + *m * b1;"),
    ("v_unfused", "float vv = fmaf(c2 * g, g, *v * b2);", "float vv = c2 * g * g + *v * b2;"),
    ("m_decays_with_b2", "float mm = fmaf(g, c1, *m * b1);", "float mm = fmaf(g, c1, *m * b2);"),
    ("m_weight_c2", "float mm = fmaf(g, c1, *m * b1);", "float mm = fmaf(g, c2, *m * b1);"),
    ("v_not_squared", "float vv = fmaf(c2 * g, g, *v * b2);", "float vv = fmaf(c2, g, *v * b2);"),
    ("no_bias_correction_m", "float mh = mm / bc1;", "float mh = mm;"),
    ("no_bias_correction_v", "float vh = vv / bc2;", "float vh = vv;"),
    ("bias_corrections_swapped", "float mh = mm / bc1;\n    float vh = vv / bc2;",
     "float mh = mm / bc2;\n    float vh = vv / bc1;"),
    ("eps_inside_root", "float den = sqrtf(vh) + eps;", "float den = sqrtf(vh + eps);"),
    ("update_sign", "*master = *master - u;", "*master = *master + u;"),
    ("no_lr", "float u = (lr * mh) / den;", "float u = mh / den;"),
    ("bc_uses_t_minus_1", "sc[6] = (float)(1.0 - pow(b1, (double)t));",
     "sc[6] = (float)(1.0 - pow(b1, (double)(t - 1)));"),
    ("bc_in_single", "sc[7] = (float)(1.0 - pow(b2, (double)t));",
     "sc[7] = 1.0f - powf((float)b2, (float)t);"),
    ("one_minus_b1_in_single", "sc[1] = (float)(1.0 - b1);", "sc[1] = 1.0f - (float)b1;"),
    ("out_offset_ignored", "((uint16_t *)out)[out_off + i] = oracle_bf16_round(master[i]);\n        else\n            ((float *)out)[out_off + i] = master[i];\n    }\n    return ORACLE_OK;\n}\n\n/* Master",
     "((uint16_t *)out)[i] = oracle_bf16_round(master[i]);\n        else\n            ((float *)out)[i] = master[i];\n    }\n    return ORACLE_OK;\n}\n\n/* Master"),
    ("master_load_ignores_lo", "master[i] = grad_at(flat, is_bf16, lo + i);", "master[i] = grad_at(flat, is_bf16, i);"),
    ("zero2_wrong_term", "case 2: return 2.0 * psi + 14.0 * psi / n;", "case 2: return 2.0 * psi + 12.0 * psi / n;"),
    ("zero1_wrong_term", "case 1: return 4.0 * psi + 12.0 * psi / n;", "case 1: return 4.0 * psi + 14.0 * psi / n;"),
    ("dim0_floor", "    if (c * world < d0)\n        c += 1;", "    if (c * world < d0)\n        c += 0;"),
    ("dim0_no_clamp", "    if (first > d0) first = d0;\n", ""),
    ("state_two_tensors", "return 3 * shard * (int64_t)sizeof(float);", "return 2 * shard * (int64_t)sizeof(float);"),
    ("unflatten_misses_offset", "memcpy(dsts[t], in + off * elem_size,", "memcpy(dsts[t], in,"),
]


@pytest.fixture(scope="module")
def src():
    with open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")) as f:
        return f.read()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(src, name, old, new, tmp_path):
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mutated = src.replace(old, new)
    c = tmp_path / "mutant.c"
    c.write_text(mutated)
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", *oracle.CFLAGS, "-w", str(c), "-o", str(so), "-lm"])
    saved = oracle._lib
    oracle._lib = oracle.load(str(so))
    caught = None
    try:
        for check in ALL_CHECKS:
            try:
                check()
            except (AssertionError, ValueError, FloatingPointError) as e:  # noqa: PERF203
                caught = (check.__name__, repr(e)[:200])
                break
    finally:
        oracle._lib = saved
    assert caught is not None, f"mutant {name} passed every pin"
