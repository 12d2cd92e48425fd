"""The oracle's pins catch planted mistakes (CPU only).

Each case copies the oracle's C source, plants one plausible mistake by
text substitution (a swapped nibble order, an off-by-one bias, a wrong tie
rule, a flipped sign, a transposed index, an unstable sort ...), compiles
the copy into a temporary library, points the oracle wrapper at it and runs
the pin tests.  At least one pin must fail for every mutant.
"""
import ctypes
import inspect
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as pins_mod

SRC = os.path.join(os.path.dirname(oracle.__file__), "moe_oracle.c")

MUTANTS = {
    "nibble_order": ("(kk % 2 == 0) ? (byte & 0x0Fu) : (byte >> 4)",
                     "(kk % 2 == 1) ? (byte & 0x0Fu) : (byte >> 4)"),
    "e8m0_bias": ("ldexp(1.0, (int)byte - 127)", "ldexp(1.0, (int)byte - 126)"),
    "e2m1_table": ("{0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0}",
                   "{0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 5.0}"),
    "tie_to_odd": ("(dd == bd && (i & 1) == 0)", "(dd == bd && (i & 1) == 1)"),
    "scale_emax": ("block_scale_exp(amax, 2);", "block_scale_exp(amax, 1);"),
    "scale_floor": ("int se = (ex - 1) - emax_elem;", "int se = ex - emax_elem;"),
    "e4m3_subnormal": ("ldexp((double)m / 8.0, -6)", "ldexp((double)m / 8.0, -7)"),
    "router_transposed": ("const uint16_t* we = w_bf16 + (int64_t)e * d;",
                          "const uint16_t* we = w_bf16 + (int64_t)e;"),
    "router_abs_of_sum": ("a += fabs(p);", "a += p;"),
    "dflash_accept_reversed": ("if (!(up < pt)) break;", "if (up < pt) break;"),
    "dflash_residual_sign": ("const float dlt = pt_row[i] - pd_row[i];", "const float dlt = pd_row[i] - pt_row[i];"),
    "dflash_prefix_ge": ("if (run > thr) return i;", "if (run >= thr) return i;"),
    "dflash_no_residual": ("tok = draw_index(res, V, r[b]);", "tok = draw_index(pt_row, V, r[b]);"),
    "dflash_no_fallback": ("if (tok < 0) tok = draw_index(pt_row, V, r[b]);", ""),
    "dflash_r_unclamped": ("r24 = f >= 16777215.0 ? 16777215u : (uint64_t)f;", "r24 = (uint64_t)f;"),
    "route_tie_high": ("(best < 0 || l[e] > l[best])", "(best < 0 || l[e] >= l[best])"),
    "softmax_sign": ("sum += exp((double)l[ids[j]] - l0);",
                     "sum += exp(l0 - (double)l[ids[j]]);"),
    "permute_reverse": ("for (int32_t p = 0; p < P; ++p) {\n        int32_t pos",
                        "for (int32_t p = P - 1; p >= 0; --p) {\n        int32_t pos"),
    "silu_sign": ("gn / (1.0 + exp(-gn)) * un", "gn / (1.0 + exp(gn)) * un"),
    "gate_up_swap": ("hh[n] = gn / (1.0 + exp(-gn)) * un;", "hh[n] = un / (1.0 + exp(-un)) * gn;"),
    "down_transposed": ("om += w_elem(dp, ds, f, m, n) * hh[n];",
                        "om += w_elem(dp, ds, f, n % d, m % f) * hh[n];"),
    "combine_first_weight": ("yt[m] += wt[j] * o[m];", "yt[m] += wt[0] * o[m];"),
    "mxfp8_h_skipped": ("if (act_mode == ORC_ACT_MXFP8) mxfp8_round_trip(hh, f, qc, qs);", ""),
    "x_not_widened_exactly": ("uint32_t u = (uint32_t)bits << 16;",
                              "uint32_t u = ((uint32_t)bits << 16) | 0x8000u;"),
}

# the pin tests to run against each mutant (all of them, minus the ones
# that only re-check thread counts or argument validation, and the sweep of
# the quantiser over whole workloads, which repeats the quantiser comparison
# on more data for half a minute)
PIN_TESTS = [(n, f) for n, f in inspect.getmembers(pins_mod, inspect.isfunction)
             if n.startswith("test_") and n not in ("test_forward_rejects_bad_shapes",
                                                     "test_forward_threads_do_not_change_result",
                                                     "test_quantizers_agree_on_every_weight_of_the_workload")]


def _run_all_pins():
    failed = []
    for name, fn in PIN_TESTS:
        params = getattr(fn, "pytestmark", [])
        arglists = [{}]
        for mark in params:
            if mark.name == "parametrize":
                argname, values = mark.args[0], mark.args[1]
                arglists = [{argname: v} for v in values]
        for kw in arglists:
            try:
                fn(**kw)
            except (AssertionError, ValueError):
                failed.append(name)
                break
    return failed


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_catch_planted_mistake(mutant, tmp_path, monkeypatch):
    old, new = MUTANTS[mutant]
    src = open(SRC).read()
    assert old in src, f"mutation anchor for {mutant} not found"
    mpath = tmp_path / "moe_oracle.c"
    mpath.write_text(src.replace(old, new))
    (tmp_path / "moe_oracle.h").write_text(
        open(os.path.join(os.path.dirname(SRC), "moe_oracle.h")).read())
    so = tmp_path / "liboracle_mutant.so"
    subprocess.check_call(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                           "-o", str(so), str(mpath), "-lm"])
    monkeypatch.setattr(oracle, "_lib", oracle.bind(ctypes.CDLL(str(so))))
    failed = _run_all_pins()
    assert failed, f"no pin caught mutant {mutant!r}"
