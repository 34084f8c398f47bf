"""CPU checks of the block oracle (context-parallel building block): its pins, and
planted mistakes that the pins must catch."""
import inspect
import types

import numpy as np
import pytest

import oracle_block_pins as pins
from oracle import blocks


@pytest.mark.parametrize("pin", pins.ALL_BLOCK_PINS, ids=lambda p: p.__name__)
def test_block_pin(pin):
    assert pin(blocks)


SOURCE = inspect.getsource(blocks)

MUTATIONS = {
    # causal limit off by one, or positions taken from the wrong block
    "mask_hides_equal_position": ("[None, :] <= (q_pos0", "[None, :] < (q_pos0"),
    "key_positions_from_query": ("return (k_pos0 + np.arange(n_k))", "return (q_pos0 + np.arange(n_k))"),
    # merge: unnormalised weights, base-2 log-sum-exp
    "merge_unnormalised": ("coef = np.where(fin[None], w / np.where(fin, tot, 1.0)[None], 0.0)",
                           "coef = np.where(fin[None], w, 0.0)"),
    "merge_log2": ("m0 + np.log(np.where(fin, tot, 1.0))", "m0 + np.log2(np.where(fin, tot, 1.0))"),
    # backward: Delta dropped, partial instead of merged normalisation, dV untransposed
    "bwd_without_delta": ("ds = p * (dp - delta[:, None])", "ds = p * dp"),
    "bwd_dv_untransposed": ("dv[b, g] += p.T @ do[b, h]", "dv[b, g] += (p @ do[b, h][: p.shape[1]])"),
    "bwd_dk_missing_scale": ("dk[b, g] += scale * ds.T @ q[b, h]", "dk[b, g] += ds.T @ q[b, h]"),
}


def mutated(name):
    old, new = MUTATIONS[name]
    assert SOURCE.count(old) >= 1, f"mutation {name} does not apply"
    mod = types.ModuleType(f"blocks_mutant_{name}")
    exec(compile(SOURCE.replace(old, new), mod.__name__, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_some_block_pin_catches_mutation(name):
    mod = mutated(name)
    results = {}
    for pin in pins.ALL_BLOCK_PINS:
        try:
            with np.errstate(all="ignore"):
                results[pin.__name__] = bool(pin(mod))
        except Exception:  # a crash also counts as caught
            results[pin.__name__] = False
    assert not all(results.values()), f"no pin caught {name}: {results}"
