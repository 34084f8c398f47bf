"""Plant plausible mistakes into a copy of the oracle (CPU only); the pins must catch each.

Each mutation is a textual edit of the oracle's source, executed as a fresh
module; the real oracle is never modified.
"""
import importlib.util
import inspect
import types

import pytest

import oracle_pins as pins
from oracle import attention as att

SOURCE = inspect.getsource(att)

MUTATIONS = {
    # mask alignment off by one in either direction
    "mask_sees_next_key": ("<= rows[:, None]", "<= rows[:, None] + 1"),
    "mask_hides_diagonal": ("<= rows[:, None]", "< rows[:, None]"),
    # interleaved instead of contiguous GQA groups
    "gqa_interleaved": ("return h // (hq // hkv)", "return h % hkv"),
    # base-2 log-sum-exp
    "lse_log2": ("(m + np.log(l))", "(m + np.log2(l))"),
    # softmax normaliser dropped
    "no_normaliser": ("return e / l, ", "return e, "),
    # backward: dropped Delta term, wrong operand orientation, missing scale, sign
    "ds_without_delta": ("ds = p * (dp - delta[:, None])\n        out", "ds = p * dp\n        out"),
    "dk_untransposed": ("scale * (ds.T @ q[r0:r1])", "scale * (ds @ q[r0:r1])"),
    "dv_untransposed": ("+= p.T @ dpo", "+= p @ dpo"),
    "dq_missing_scale": ('out["dq"][r0:r1] = scale * (ds @ kk)', 'out["dq"][r0:r1] = ds @ kk'),
    "dp_sign": ("dp = dpo @ vv.T", "dp = -(dpo @ vv.T)"),
    "scale_after_softmax": ("s = scale * (q_rows @ k.T)", "s = q_rows @ k.T"),
}


def mutated_module(name):
    old, new = MUTATIONS[name]
    assert SOURCE.count(old) >= 1, f"mutation {name} does not apply"
    src = SOURCE.replace(old, new)
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src, mod.__name__, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_some_pin_catches_mutation(name):
    mod = mutated_module(name)
    results = {}
    for pin in pins.ALL_PINS:
        try:
            with __import__("numpy").errstate(all="ignore"):
                results[pin.__name__] = bool(pin(mod))
        except Exception:  # a crash also counts as caught
            results[pin.__name__] = False
    assert not all(results.values()), f"no pin caught {name}: {results}"


def test_unmutated_copy_passes():
    src_mod = types.ModuleType("oracle_copy")
    exec(compile(SOURCE, "oracle_copy", "exec"), src_mod.__dict__)
    assert all(pin(src_mod) for pin in pins.ALL_PINS)
