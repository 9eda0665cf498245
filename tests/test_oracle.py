"""The CPU oracle against its pins (no GPU), and the pins against mutated oracles.

The pins live in oracle_pins.py; each is run here on the real oracle.  The
mutation test then plants one plausible mistake at a time in a private copy of
oracle.c (a dropped term, a wrong sign, index or bias, a reversed order, a
transposed operand), builds it, and requires that at least one pin fails on
it -- evidence that the pins constrain every part of the definition.
"""
import os
import subprocess
import sys
import tempfile

import pytest

import oracle_pins
from oracle import oracle as oracle_mod


@pytest.fixture(scope="module")
def orc():
    if not os.path.exists(oracle_mod.LIB):
        oracle_mod.build()
    return oracle_mod.load()


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)


# (name, text in oracle.c, replacement): each must occur exactly once.
MUTANTS = [
    ("score_order_reversed", "if (a->score > b->score)", "if (a->score < b->score)"),
    ("tie_break_reversed",
     "if (a->row < b->row)\n        return -1;\n    if (a->row > b->row)\n        return 1;",
     "if (a->row < b->row)\n        return 1;\n    if (a->row > b->row)\n        return -1;"),
    ("relu_dropped", "(x > 0.0 ? x : 0.0)", "x"),
    ("relu_wrong_side", "(x > 0.0 ? x : 0.0)", "(x < 0.0 ? x : 0.0)"),
    ("weight_dropped", "s += (double)wt[h] *", "s += 1.0 *"),
    ("first_head_dropped", "for (h = 0; h < H; ++h) {\n                double x",
     "for (h = 1; h < H; ++h) {\n                double x"),
    ("k_row_reversed", "x += qt[h * D + d] * kj[d];", "x += qt[h * D + d] * kj[D - 1 - d];"),
    ("q_transposed", "jb->q[(t * H + h) * D + d]", "jb->q[(t * D + d) * H + h]"),
    ("q_sign", "qt[h * D + d] = v;", "qt[h * D + d] = -v;"),
    ("causal_off_by_one", "n = (pos + 1) / ratio;", "n = pos / ratio;"),
    ("causal_inclusive_partial", "n = (pos + 1) / ratio;", "n = (pos + ratio) / ratio;"),
    ("output_descending", "return (a > b) - (a < b);", "return (a < b) - (a > b);"),
    ("pad_zero", "o[c] = c < m ? (int32_t)chosen[c] : -1;", "o[c] = c < m ? (int32_t)chosen[c] : 0;"),
    ("keeps_one_less", "m = n < jb->topk ? n : jb->topk;", "m = n < jb->topk ? n : jb->topk - 1;"),
    ("f16_bias", "expo - 25); /*", "expo - 24); /*"),
    ("f16_subnormal", "ldexp((double)frac, -24);", "ldexp((double)frac, -25);"),
    ("bf16_bias", "expo - 134); /*", "expo - 133); /*"),
    ("bf16_frac_bits", "int frac = bits & 0x7F;", "int frac = bits & 0x3F;"),
    # query projection and rounding into the storage type
    ("round_truncates", "double r = nearbyint(a / q);", "double r = floor(a / q);"),
    ("round_half_away", "double r = nearbyint(a / q);", "double r = floor(a / q + 0.5);"),
    ("proj_w_transposed", "jb->wq[o * jb->din + i]", "jb->wq[i * jb->O + o]"),
    ("proj_skips_last_input", "for (i = 0; i < jb->din; ++i) {\n                const double a",
     "for (i = 0; i + 1 < jb->din; ++i) {\n                const double a"),
    # sparse attention
    ("attn_scale_dropped", "s[r] = jb->scale * x;", "s[r] = x;"),
    ("attn_window_one_short", "lo = p - jb->window + 1;", "lo = p - jb->window + 2;"),
    ("attn_window_excludes_self", "hi = p < jb->L - 1 ? p : jb->L - 1;",
     "hi = p - 1 < jb->L - 1 ? p - 1 : jb->L - 1;"),
    ("attn_padding_ends_list", "if (j < 0)\n                continue;", "if (j < 0)\n                break;"),
    ("attn_no_max_shift", "s[r] = exp(s[r] - m);", "s[r] = exp(s[r]);"),
    ("attn_unnormalised", "const double a = s[r] / z;", "const double a = s[r];"),
    ("attn_local_values_reversed", "vrow[nr] = jb->vl + r * DV;", "vrow[nr] = jb->vl + (hi - (r - lo)) * DV;"),
    ("attn_every_head_is_head0", "jb->q[(t * HA + h) * DK + d]", "jb->q[(t * HA) * DK + d]"),
    ("attn_all_one_row_more", "for (r = 0; r < nv; ++r) {", "for (r = 0; r <= nv && r < jb->N; ++r) {"),
    ("attn_all_visible_off_by_one", "oracle_visible_rows(p, jb->ratio, jb->N)",
     "oracle_visible_rows(p - 1, jb->ratio, jb->N)"),
    ("attn_pooled_keys_reversed", "krow[nr] = jb->kp + (int64_t)j * DK;",
     "krow[nr] = jb->kp + (int64_t)(jb->N - 1 - j) * DK;"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    src = open(oracle_mod.SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    with tempfile.TemporaryDirectory() as tmp:
        c = os.path.join(tmp, "mutant.c")
        so = os.path.join(tmp, "libmutant.so")
        with open(c, "w") as f:
            f.write(src.replace(old, new))
        oracle_mod.build(out=so, src=c)
        # a separate process, so that a mutant which misbehaves badly cannot take
        # the test runner down with it
        r = subprocess.run([sys.executable, oracle_pins.__file__, so], capture_output=True,
                           text=True, timeout=300)
        assert r.returncode == 1, f"mutant {name} passed every pin:\n{r.stdout}{r.stderr}"
        assert "FAIL" in r.stdout
