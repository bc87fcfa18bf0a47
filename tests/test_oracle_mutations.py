"""The oracle's pins catch plausible mistakes in it (a mutation check; CPU only).

Each case plants one mistake in a copy of one oracle module: a dropped term, a wrong
operand, a rounding or saturation rule changed, a boundary off by one. The copy is the
module's source with that fragment (or two) replaced, executed as a sibling module of
the oracle package. Every reference to the original functions, in the oracle package, its submodules
and the pin test modules, is rebound to the copy's. The pins meant for that part of the
oracle then run, and at least one of them must fail. Nothing here involves the GPU path.
"""
import importlib
import inspect
import sys
import types

import pytest

import oracle  # noqa: F401  (the package whose modules are copied)
import test_oracle_attention as TA
import test_oracle_e4m3 as TE
import test_oracle_scaling as TS


def _mutant(modname, edits):
    """The module and a copy of it with each (old, new) fragment replaced (each old once)."""
    mod = importlib.import_module(modname)
    src = inspect.getsource(mod)
    for old, new in edits:
        assert src.count(old) == 1, (modname, old)
        src = src.replace(old, new)
    m = types.ModuleType(modname + "_mutant")
    m.__package__ = "oracle"
    m.__file__ = mod.__file__
    exec(compile(src, m.__name__, "exec"), m.__dict__)
    return mod, m


def _rebind(monkeypatch, mod, mutant):
    """Point every reference to mod's functions and classes at mutant's."""
    originals = {name: obj for name, obj in vars(mod).items()
                 if callable(obj) and getattr(obj, "__module__", None) == mod.__name__}
    holders = [m for name, m in list(sys.modules.items())
               if m is not None and (name == "oracle" or name.startswith("oracle.")
                                     or name.startswith("test_oracle"))]
    n = 0
    for name, obj in originals.items():
        for holder in holders:
            for attr, val in list(vars(holder).items()):
                if val is obj:
                    monkeypatch.setattr(holder, attr, getattr(mutant, name))
                    n += 1
    assert n > 0


def _catches(pins):
    """Names of the pins that fail with an assertion (any other error propagates)."""
    caught = []
    for pin in pins:
        try:
            pin()
        except AssertionError:
            caught.append(getattr(pin, "__name__", "pin"))
    return caught


E4M3 = "oracle.e4m3"
SCALING = "oracle.scaling"
ATT = "oracle.attention"

CASES = [
    ("E4M3 ties rounded away from zero", E4M3,
     [("np.rint(np.ldexp(af, -spacing_exp))", "np.floor(np.ldexp(af, -spacing_exp) + 0.5)")],
     [TE.test_special_values, lambda: TE.test_exhaustive_bf16_vs_brute_force(1.0)]),
    ("E4M3 without saturation", E4M3,
     [("is_sat = (~is_nan) & (a >= E4M3_MAX)", "is_sat = (~is_nan) & np.isinf(a)")],
     [TE.test_special_values, TE.test_monotone_and_max]),
    ("E4M3 exponent off by one", E4M3,
     [("c[~sub] = ((ven + 7) << 3) | mant.astype(np.int64)",
       "c[~sub] = ((ven + 6) << 3) | mant.astype(np.int64)")],
     [TE.test_published_table_values, TE.test_roundtrip_all_finite_codes]),
    ("inverse scale as 1/scale", SCALING,
     [("inv = float(round_f32(E4M3_MAX / a))", "inv = float(round_f32(1.0 / scale))")],
     [TS.test_scale_pair_exhaustive_vs_fractions]),
    ("ring window without the current forward", SCALING,
     [("        slot = self.count % RING_SLOTS\n",
       "        slot = self.count % RING_SLOTS\n"
       "        prior = [float(np.max(self.slots[t])) for t in range(3)]\n"),
      ("        return [float(np.max(self.slots[t])) for t in range(3)]",
       "        return prior")],
     [TS.test_ring_window_closed_form, TS.test_ring_random_trajectory_matches_window_max]),
    ("static amax not rounded to binary32", SCALING,
     [("return [float(v) for v in round_f32(cal * m)]", "return [float(v) for v in cal * m]")],
     [TS.test_scale_file_worked_example]),
    ("amax of signed values", SCALING,
     [("return float(np.max(np.abs(x)))", "return float(np.max(x))")],
     [lambda: TS.test_amax_vs_integer_bits(0)]),
    ("row maximum over the first 64 keys only", ATT,
     [("M = np.ceil(np.max(t, axis=1, keepdims=True))",
       "M = np.ceil(np.max(t[:, :64], axis=1, keepdims=True))")],
     [TA.test_weights_sum_to_one_and_key_permutation, TA.test_row_maximum_over_all_keys_not_a_prefix]),
    ("reference exponent rounded down", ATT,
     [("M = np.ceil(np.max(t, axis=1, keepdims=True))",
       "M = np.floor(np.max(t, axis=1, keepdims=True))")],
     [TA.test_worked_two_key_example, TA.test_weights_sum_to_one_and_key_permutation]),
    ("exact row maximum as the reference", ATT,
     [("M = np.ceil(np.max(t, axis=1, keepdims=True))", "M = np.max(t, axis=1, keepdims=True)")],
     [TA.test_worked_two_key_example, TA.test_one_pass_with_power_of_two_rescale_gives_the_rule]),
    ("natural exponential in place of base 2", ATT,
     [("p_tilde = np.exp2(t - M)", "p_tilde = np.exp(t - M)")],
     [TA.test_worked_two_key_example]),
    ("softmax scale dropped", ATT,
     [("        s = raw * c\n", "        s = raw * float(scale_q) * float(scale_k)\n")],
     [TA.test_worked_two_key_example]),
    ("P scaled by 224 instead of 448", ATT,
     [("p8 = e4m3_encode(p_tilde * E4M3_MAX)", "p8 = e4m3_encode(p_tilde * 224.0)")],
     [TA.test_worked_two_key_example, TA.test_weights_sum_to_one_and_key_permutation]),
    ("normalised by the unquantised weights", ATT,
     [("        L = np.sum(p, axis=1)", "        L = np.sum(p_tilde * E4M3_MAX, axis=1)")],
     [TA.test_worked_two_key_example, TA.test_weights_sum_to_one_and_key_permutation]),
    ("K in place of V", ATT,
     [("out[r0:r1] = (p @ v) * float(scale_v) / L[:, None]",
       "out[r0:r1] = (p @ k) * float(scale_v) / L[:, None]")],
     [TA.test_zero_query_gives_mean, TA.test_single_key_and_constant_v]),
    ("a sequence sees the next sequence's first key", ATT,
     [("fp8_attention_head(q8[rows, h], k8[lo:hi, h], v8[lo:hi, h],",
       "fp8_attention_head(q8[rows, h], k8[lo:hi + 1, h], v8[lo:hi + 1, h],")],
     [TA.test_block_diagonal_isolation_brute_force]),
    ("reference softmax normalised over the keys' axis", ATT,
     [("out[r0:r1] = (p @ v) / np.sum(p, axis=1, keepdims=True)",
       "out[r0:r1] = (p @ v) / np.sum(p, axis=0, keepdims=True)[:, :1]")],
     [TA.test_reference_attention_vs_library_and_brute_force]),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_pins_catch_the_planted_mistake(monkeypatch, case):
    label, modname, edits, pins = case
    mod, mutant = _mutant(modname, edits)
    _rebind(monkeypatch, mod, mutant)
    assert _catches(pins), f"no pin caught: {label}"


def test_unmutated_oracle_passes_the_same_pins():
    # the harness itself: with no mistake planted, every pin used above passes
    pins = sorted({p for c in CASES for p in c[3]}, key=lambda p: getattr(p, "__name__", ""))
    assert not _catches(pins)
