"""CPU test: plant plausible mistakes in copies of the numpy/torch oracle functions (the
attention comparator and the backward pass) and check that their pins in
tests/test_oracle_pins.py catch every one of them. The mutants are built from the
functions' own source text and swapped in for the duration of one test."""
import inspect
import warnings

import pytest

import oracle
import oracle.oracle as oracle_module
import test_oracle_pins as pins


def _mutant(fn, old, new):
    src = inspect.getsource(fn)
    assert src.count(old) == 1, f"mutation site not unique in {fn.__name__}: {old}"
    ns = dict(vars(oracle_module))
    exec(compile(src.replace(old, new), f"<mutant of {fn.__name__}>", "exec"), ns)
    return ns[fn.__name__]


def _failures(tests):
    failed = 0
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")  # overflow in a mutant is a failure, reported by its assert
        for t in tests:
            try:
                t()
            except (AssertionError, ValueError, IndexError, RuntimeError, FloatingPointError):
                failed += 1
    return failed


ATTN = {
    "no_scale": ("s = scale * (K[b, j, :n] @ q[b, h])", "s = (K[b, j, :n] @ q[b, h])"),
    "cached_head_by_modulo": ("j = h // G", "j = h % H_kv"),
    "no_normalisation": ("o[b, h] = (w @ V[b, j, :n]) / w.sum()", "o[b, h] = (w @ V[b, j, :n])"),
    "values_from_keys": ("o[b, h] = (w @ V[b, j, :n]) / w.sum()", "o[b, h] = (w @ K[b, j, :n]) / w.sum()"),
    "lengths_ignored": ("n = T_max if seq_lens is None else min(max(int(seq_lens[b]), 0), T_max)",
                        "n = T_max"),
    "no_max_shift": ("w = np.exp(s - s.max())", "w = np.exp(s)"),
}
ATTN_PINS = (pins.test_attn_decode_worked_example, pins.test_attn_decode_grouped_heads_and_lengths,
             pins.test_attn_decode_closed_forms, pins.test_attn_decode_matches_library_softmax_and_is_order_free)


@pytest.mark.parametrize("name", sorted(ATTN))
def test_attn_pins_catch_mutant(monkeypatch, name):
    monkeypatch.setattr(oracle, "attn_decode_reference", _mutant(oracle_module.attn_decode_reference, *ATTN[name]))
    assert _failures(ATTN_PINS) > 0, name


BWD = {
    "no_decay": ("St = torch.exp(la[:, t])[..., None] * S", "St = S"),
    "no_scale": ("outs.append(scale * torch.einsum", "outs.append(1.0 * torch.einsum"),
    "dhT_ignored": ("loss = loss + (S * t64(dhT)).sum()", "loss = loss"),
    "beta_dropped": ("e = bb[:, t][..., None] * (vv[:, t]", "e = 1.0 * (vv[:, t]"),
    "readout_before_write": ("outs.append(scale * torch.einsum(\"bhkv,bhk->bhv\", S, qq[:, t]))",
                             "outs.append(scale * torch.einsum(\"bhkv,bhk->bhv\", St, qq[:, t]))"),
}
BWD_PINS = (pins.test_backward_matches_finite_differences, pins.test_backward_closed_forms)


@pytest.mark.parametrize("name", sorted(BWD))
def test_backward_pins_catch_mutant(monkeypatch, name):
    monkeypatch.setattr(oracle, "kda_backward_reference", _mutant(oracle_module.kda_backward_reference, *BWD[name]))
    assert _failures(BWD_PINS) > 0, name


def test_unmutated_copies_pass_the_pins(monkeypatch):
    # the harness itself: a copy with an empty mutation must pass every pin
    monkeypatch.setattr(oracle, "attn_decode_reference",
                        _mutant(oracle_module.attn_decode_reference, "j = h // G", "j = h // G"))
    monkeypatch.setattr(oracle, "kda_backward_reference",
                        _mutant(oracle_module.kda_backward_reference, "St = torch.exp", "St = torch.exp"))
    assert _failures(ATTN_PINS + BWD_PINS) == 0
