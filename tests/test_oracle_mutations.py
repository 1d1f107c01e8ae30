"""Planted mistakes in copies of the oracle (CPU only) must each fail a pin.

Each mutant is a one-line change of ``oracle/oracle.c`` -- a flipped sign, a
dropped term, a wrong index, a transposed operand, a wrong angle or decode --
compiled to a temporary library.  The pin suite in ``test_oracle_pins.py`` is
run against it and at least one pin has to fail.  This shows the pins fix the
oracle's arithmetic, not just agree with it.
"""
import inspect

import pytest

import oracle
from tests import test_oracle_kv_remap as kv_pins
from tests import test_oracle_pins as pins

# (name, exact source text, replacement, which occurrence)
MUTANTS = [
    ("rotation_direction", "double s = (double)direction * sn[i];",
     "double s = -(double)direction * sn[i];", 0),
    ("rotation_first_sign", "y[nope + i] = a * cs[i] - b * s;",
     "y[nope + i] = a * cs[i] + b * s;", 0),
    ("rotation_dropped_term", "y[nope + h2 + i] = b * cs[i] + a * s;",
     "y[nope + h2 + i] = b * cs[i];", 0),
    ("frequency_exponent", "double inv_freq = pow(theta, -2.0 * (double)i / (double)pe);",
     "double inv_freq = pow(theta, -2.0 * (double)i / (double)(pe + 2));", 0),
    ("angle_position_off_by_one", "double phi = (double)position * inv_freq;",
     "double phi = (double)(position + 1) * inv_freq;", 0),
    ("fwd_transposed_w", "acc += w[g * nh + h] * x[h * d + c];",
     "acc += w[h * nh + g] * x[h * d + c];", 0),
    ("dx_untransposed_w", "acc += w[g * nh + h] * dy[g * d + c];",
     "acc += w[h * nh + g] * dy[g * d + c];", 0),
    ("dx_wrong_rotation", "rotate_head(dx + h * d, out + h * d, p->nope, p->pe, cs, sn, +1);",
     "rotate_head(dx + h * d, out + h * d, p->nope, p->pe, cs, sn, -1);", 0),
    ("dw_wrong_rotation", "rotate_head(o + h * d, x + h * d, p->nope, p->pe, cs, sn, -1);",
     "rotate_head(o + h * d, x + h * d, p->nope, p->pe, cs, sn, +1);", 1),
    ("dw_transposed_output", "acc[g * nh + h] += t;", "acc[h * nh + g] += t;", 0),
    ("dw_wrong_head", "t += dy[g * d + c] * x[h * d + c];", "t += dy[g * d + c] * x[g * d + c];", 0),
    ("dw_abs_dropped", "t += fabs(dy[g * d + c] * x[h * d + c]);", "t += dy[g * d + c] * x[h * d + c];", 0),
    ("dw_abs_one_factor", "t += fabs(dy[g * d + c] * x[h * d + c]);", "t += fabs(dy[g * d + c]) * x[h * d + c];", 0),
    ("dw_dropped_slab", "for (int32_t k = 0; k < nthreads; ++k) t += slabs[(int64_t)k * nh * nh + i];",
     "for (int32_t k = 0; k + 1 < nthreads; ++k) t += slabs[(int64_t)k * nh * nh + i];", 0),
    ("rows_skip_first_of_chunk", "tasks[t].lo = n * t / nthreads;",
     "tasks[t].lo = n * t / nthreads + (t > 0);", 0),
    ("bf16_decode_truncated", "uint32_t u = ((uint32_t)b) << 16;",
     "uint32_t u = ((uint32_t)(b & 0xFFF0u)) << 16;", 0),
    ("fwd_at_sign", "if (c < nope + h2) return a * cs[i] + b * sn[i];",
     "if (c < nope + h2) return a * cs[i] - b * sn[i];", 0),
    ("fwd_at_transposed_w", "acc += bf16_bits_to_double(W[g * nh + h]) *",
     "acc += bf16_bits_to_double(W[h * nh + g]) *", 0),
    ("dx_at_sign", "if (c < nope + h2) out[k] = ga * cs[i] - gb * sn[i];",
     "if (c < nope + h2) out[k] = ga * cs[i] + gb * sn[i];", 0),
    ("dx_at_untransposed_w", "double wg = bf16_bits_to_double(W[g * nh + h]);",
     "double wg = bf16_bits_to_double(W[h * nh + g]);", 0),
    ("dw_at_wrong_head", "inv_rope_elem_bf16(p->O, s, h, c, nh, p->nope, p->pe, cs, sn);",
     "inv_rope_elem_bf16(p->O, s, g, c, nh, p->nope, p->pe, cs, sn);", 0),
    ("kv_remap_batch_off_by_one", "out[r * topk + k] = v >= 0 ? (int32_t)(v + b * seqlen_kv) : pad_value;",
     "out[r * topk + k] = v >= 0 ? (int32_t)(v + (b + 1) * seqlen_kv) : pad_value;", 0),
    ("kv_remap_zero_is_padding", "out[r * topk + k] = v >= 0 ? (int32_t)(v + b * seqlen_kv) : pad_value;",
     "out[r * topk + k] = v > 0 ? (int32_t)(v + b * seqlen_kv) : pad_value;", 0),
    ("kv_remap_batch_of_column", "int64_t b = r / sq;", "int64_t b = r % sq;", 0),
]


def _replace_nth(text, old, new, n):
    start = -1
    for _ in range(n + 1):
        start = text.index(old, start + 1)
    return text[:start] + new + text[start + len(old):]


def _pin_cases():
    """(name, callable) for every pin, parametrized cases expanded."""
    out = []
    members = inspect.getmembers(pins, inspect.isfunction) + inspect.getmembers(kv_pins, inspect.isfunction)
    for name, fn in members:
        # the stored-output regression guard is the oracle's own output, not a pin
        if not name.startswith("test_") or name.startswith("test_golden"):
            continue
        marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        if not marks:
            out.append((name, fn, {}))
            continue
        argnames, values = marks[0].args
        argnames = [a.strip() for a in argnames.split(",")]
        for v in values:
            v = v if isinstance(v, (tuple, list)) else (v,)
            out.append((f"{name}{tuple(v)}", fn, dict(zip(argnames, v))))
    return out


def test_mutants_are_listed_once_in_the_source():
    src = oracle.source_text()
    for name, old, _new, n in MUTANTS:
        assert src.count(old) > n, name


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_each_planted_mistake_fails_a_pin(mutant, tmp_path):
    name, old, new, n = mutant
    lib = oracle.build_variant(_replace_nth(oracle.source_text(), old, new, n),
                               str(tmp_path / f"liboracle_{name}.so"))
    failed = []
    oracle.use_library(lib)
    try:
        for case_name, fn, kwargs in _pin_cases():
            try:
                fn(**kwargs)
            except Exception:  # AssertionError or a rejected call
                failed.append(case_name)
    finally:
        oracle.use_library(None)
    assert failed, f"mutant {name} passed every pin"
