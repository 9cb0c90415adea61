"""Planted mistakes in the oracle are caught by its pins (CPU only).

Each case copies the oracle's source, plants one plausible mistake (a sign,
a transposed operand, a dropped term, a wrong index or rounding rule), loads
the copy as a module of its own, and runs every pin of
tests/test_oracle_pins.py against it: at least one pin must fail.  The
unchanged source must pass every pin under the same harness.  The mistakes
live only in these in-memory copies; the oracle on disk is never changed.
"""
import inspect
import itertools
import os
import types

import pytest

import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "gptq_oracle.py")

# (label, text in the oracle, planted replacement); each text occurs once
MUTATIONS = [
    ("compensation sign", "W1[:, k + 1:] -= np.outer(err, U[c, c + 1:i2])",
     "W1[:, k + 1:] += np.outer(err, U[c, c + 1:i2])"),
    ("compensation with U transposed", "W1[:, k + 1:] -= np.outer(err, U[c, c + 1:i2])",
     "W1[:, k + 1:] -= np.outer(err, U[c + 1:i2, c])"),
    ("lazy update dropped", "W[:, i2:] -= Err @ U[i1:i2, i2:]", "W[:, i2:] -= 0.0 * (Err @ U[i1:i2, i2:])"),
    ("lazy update with the wrong rows of U", "W[:, i2:] -= Err @ U[i1:i2, i2:]",
     "W[:, i2:] -= Err @ U[i1 + 1:i2 + 1, i2:]"),
    ("error not scaled by U_cc", "err = (w - q) / ucc", "err = (w - q)"),
    ("act-order ascending", 'np.argsort(-np.diag(H), kind="stable")', 'np.argsort(np.diag(H), kind="stable")'),
    ("act-order ties to the higher index", 'np.argsort(-np.diag(H), kind="stable")',
     'len(H) - 1 - np.argsort(-np.diag(H)[::-1], kind="stable")[::-1]'),
    ("lambda from the largest diagonal entry", "lam = damp * np.mean(np.diag(H))",
     "lam = damp * np.max(np.diag(H))"),
    ("lambda not scaled by the diagonal", "return H + lam * np.eye(d)", "return H + damp * np.eye(d)"),
    ("range not widened to include 0", "xmin = np.minimum(wg.min(axis=1), 0.0)", "xmin = wg.min(axis=1)"),
    ("zero point not rounded", "zero = np.rint(-xmin / scale)", "zero = -xmin / scale"),
    ("rounding half away from zero", "code = np.clip(np.rint(w / scale) + zero, 0.0, float(maxq))",
     "code = np.clip(np.floor(w / scale + 0.5) + zero, 0.0, float(maxq))"),
    ("2^b intervals instead of 2^b - 1", "    maxq = 2 ** bits - 1\n    xmin", "    maxq = 2 ** bits\n    xmin"),
    ("symmetric zero one off", "zero = np.full_like(scale, float(2 ** (bits - 1)))",
     "zero = np.full_like(scale, float(2 ** (bits - 1) - 1))"),
    ("crossing group without the block's pending compensation",
     "past = W[:, i2:max(end, i2)] - Err[:, :k] @ U[i1:c, i2:max(end, i2)]", "past = W[:, i2:max(end, i2)]"),
    ("group parameters at every column", "if c % g == 0:", "if True:"),
    ("Hessian without the factor 2", "H += 2.0 * (x.T @ x)", "H += x.T @ x"),
    ("g_idx in sweep order", "g_idx[perm] = np.arange(d_in) // g", "g_idx[:] = np.arange(d_in) // g"),
    ("codes left in sweep order", "codes[:, perm] = codes_s", "codes[:, :] = codes_s"),
    ("pack: big-endian within a word", "out[:, wi] |= (c[:, k] << np.uint64(sh)) & np.uint64(0xFFFFFFFF)",
     "out[:, wi] |= (c[:, k] << np.uint64(32 - bits - sh if sh + bits <= 32 else sh)) & np.uint64(0xFFFFFFFF)"),
    ("loss from the damped Hessian", "loss=layer_loss(W0, w_hat, H)",
     "loss=layer_loss(W0, w_hat, damp_hessian(H, damp))"),
    ("static groups looked up by sweep position", "static = (st_scales, st_zeros, perm // g)",
     "static = (st_scales, st_zeros, np.arange(d_in) // g)"),
    ("static group parameters from the permuted weights", "static_group_params(W0, bits, group_size, sym)",
     "static_group_params(Wp, bits, group_size, sym)"),
    ("static g_idx in sweep order", "        g_idx[:] = np.arange(d_in) // g\n    else:",
     "        g_idx[perm] = np.arange(d_in) // g\n    else:"),
    ("static group parameters retaken during the sweep", "elif c % g == 0:", "if c % g == 0:"),
]


def _load_variant(src: str, name: str):
    mod = types.ModuleType(name)
    mod.__file__ = SRC
    exec(compile(src, SRC, "exec"), mod.__dict__)
    return mod


def _pin_calls():
    """Every test function of the pin module with each of its parameter sets."""
    for fname, fn in sorted(vars(pins).items()):
        if not fname.startswith("test_") or not callable(fn):
            continue
        marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        grids = []
        for m in marks:
            names = [n.strip() for n in m.args[0].split(",")] if isinstance(m.args[0], str) else list(m.args[0])
            vals = [v if len(names) > 1 else (v,) for v in m.args[1]]
            grids.append([dict(zip(names, v)) for v in vals])
        if not grids:
            yield fname, fn, {}
            continue
        for combo in itertools.product(*grids):
            kw = {}
            for d in combo:
                kw.update(d)
            yield fname, fn, kw


def _run_pins(mod):
    """Names of the pins that fail with the module bound as the oracle."""
    failed = []
    saved = pins.O
    pins.O = mod
    try:
        for fname, fn, kw in _pin_calls():
            params = inspect.signature(fn).parameters
            if any(p not in kw for p in params):
                continue   # fixtures other than parameters are not used by the pins
            try:
                fn(**kw)
            except (Exception, pytest.fail.Exception):   # a failed check, or an error the mistake raised
                failed.append(fname)
    finally:
        pins.O = saved
    return failed


def _source():
    with open(SRC) as f:
        return f.read()


def test_unchanged_oracle_passes_every_pin():
    assert _run_pins(_load_variant(_source(), "oracle_copy")) == []


@pytest.mark.parametrize("label,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(label, old, new):
    src = _source()
    assert src.count(old) == 1, f"mutation site of '{label}' not unique"
    failed = _run_pins(_load_variant(src.replace(old, new), "oracle_mutant"))
    assert failed, f"no pin caught: {label}"
