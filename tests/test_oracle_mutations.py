"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of an oracle source file (a dropped
factor, a flipped sign, an off-by-one bound, a wrong index or operand), loads
the copy as a separate module, points private copies of the pin test modules
at it, and runs their tests until one fails.  A mistake that no pin catches
fails this test.  The oracle itself is never modified; everything runs on the
CPU.
"""

import importlib.util
import inspect
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")

# (name, oracle file, text to replace, replacement, pin modules to run in order)
MUTATIONS = [
    ("causal mask excludes the diagonal", "attention.py",
     "vis = dist >= 0", "vis = dist > 0", ["fwd"]),
    ("window keeps one key too many", "attention.py",
     "(dist < window)", "(dist <= window)", ["window"]),
    ("global tokens one too many", "attention.py",
     "(kpos < n_global)", "(kpos <= n_global)", ["global"]),
    ("grouped-query heads mapped modulo", "attention.py",
     "kg = k[bi, :, h // group, :]          # [Lk, d]",
     "kg = k[bi, :, h % hkv, :]          # [Lk, d]", ["fwd"]),
    ("forward drops the scale", "attention.py",
     "s = scale * (q[bi, rows, h, :] @ kg.T)", "s = (q[bi, rows, h, :] @ kg.T)", ["fwd"]),
    ("LSE in base 2", "attention.py",
     "row_lse = ml + np.log(np.exp(sl - ml[:, None]).sum(axis=1))",
     "row_lse = ml + np.log2(np.exp(sl - ml[:, None]).sum(axis=1))", ["fwd"]),
    ("P multiplies K instead of V", "attention.py",
     "o[bi, rows[live], h, :] = p @ vg", "o[bi, rows[live], h, :] = p @ kg", ["fwd"]),
    ("merge weights not normalised by the union's LSE", "attention.py",
     "w = np.where(live, np.exp(lse_r - lse_safe), 0.0)",
     "w = np.where(live, np.exp(lse_r - m_safe), 0.0)", ["merge"]),
    ("merge LSE drops the max", "attention.py",
     "lse = np.where(live, m_safe + np.log(total), -np.inf)",
     "lse = np.where(live, np.log(total), -np.inf)", ["merge"]),
    ("delta enters dS with the wrong sign", "attention.py",
     "ds = p * (dp - delta[bi, h, rows][:, None])",
     "ds = p * (dp + delta[bi, h, rows][:, None])", ["bwd"]),
    ("dK drops the scale", "attention.py",
     "dk[bi, :, g, :] += scale * (ds.T @ qi)", "dk[bi, :, g, :] += (ds.T @ qi)", ["bwd"]),
    ("dK overwritten instead of summed over a head group", "attention.py",
     "dk[bi, :, g, :] += scale * (ds.T @ qi)", "dk[bi, :, g, :] = scale * (ds.T @ qi)", ["bwd"]),
    ("dV built from dS instead of P", "attention.py",
     "dv[bi, :, g, :] += p.T @ doi", "dv[bi, :, g, :] += ds.T @ doi", ["bwd"]),
    ("dQ contracts dS with V instead of K", "attention.py",
     "dq[bi, rows, h, :] += scale * (ds @ kg)", "dq[bi, rows, h, :] += scale * (ds @ vg)",
     ["bwd"]),
    ("backward P ignores the LSE", "attention.py",
     "np.exp(np.where(vis, s, 0.0) - row_lse[:, None])", "np.exp(np.where(vis, s, 0.0))",
     ["bwd"]),
    ("delta averaged instead of summed over head_dim", "attention.py",
     "np.transpose((o * do).sum(axis=3), (0, 2, 1))",
     "np.transpose((o * do).mean(axis=3), (0, 2, 1))", ["bwd"]),
    ("helper serves the wrong owner", "schedule.py",
     "owner = w + p - t\n", "owner = w + p - t - 1\n", ["schedule"]),
    ("helpers repeat a pair at even P", "schedule.py",
     "elif p - t > t:", "elif p - t >= t:", ["schedule"]),
    ("window schedule reaches one chunk too far", "schedule.py",
     "(t - 1) * c + 1 < w_", "(t - 1) * c < w_", ["window"]),
    ("window schedule calls a band pair full", "schedule.py",
     "(t + 1) * c - 1 < w_", "(t + 1) * c - 2 < w_", ["window"]),
    ("tile map masks the tile that ends on the diagonal", "schedule.py",
     "masked = last_k > first_q or", "masked = last_k >= first_q or", ["schedule"]),
    ("tile map visits a tile one step outside the window", "schedule.py",
     "first_q - last_k < window", "first_q - last_k <= window", ["window"]),
    ("global schedule keeps the empty chunk-0 pair", "schedule.py",
     "items = [it for it in items if not (it[3] == 0 and g == c)]", "items = list(items)",
     ["global"]),
    ("row maximum taken as the minimum", "attention.py",
     "m = s.max(axis=1)", "m = s.min(axis=1)", ["fwd"]),
    ("rows without keys get LSE 0", "attention.py",
     "lse = np.full((b, hq, lq), -np.inf, dtype=np.float64)",
     "lse = np.full((b, hq, lq), 0.0, dtype=np.float64)", ["fwd"]),
    ("merge treats rows that every part leaves empty as live", "attention.py",
     "live = np.isfinite(m)\n    m_safe", "live = np.ones_like(m, dtype=bool)\n    m_safe",
     ["merge"]),
    ("one worker's global item missing", "schedule.py",
     "items += [(0, w, w, -1, GLOBAL, w) for w in range(p)]",
     "items += [(0, w, w, -1, GLOBAL, w) for w in range(1, p)]", ["global"]),
    ("window schedule skips the first worker of a step", "schedule.py",
     "for w in range(t, p):", "for w in range(t + 1, p):", ["window"]),
    ("balanced schedule one step short", "schedule.py",
     "steps = 1 + p // 2", "steps = p // 2", ["schedule"]),
    ("unbalanced schedule calls the diagonal pair full", "schedule.py",
     "items.append((t, w, w, w - t, DIAG if t == 0 else FULL, w))",
     "items.append((t, w, w, w - t, FULL, w))", ["schedule"]),
    ("non-causal tile map marks tiles masked", "schedule.py",
     "            if not causal:\n                out[qt, kt] = 1",
     "            if not causal:\n                out[qt, kt] = 2", ["schedule"]),
]


def _load(path, name):
    spec = importlib.util.spec_from_file_location(name, path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _mutant(fname, old, new, tag):
    src = open(os.path.join(ROOT, "oracle", fname)).read()
    assert src.count(old) == 1, f"mutation site not unique in {fname}: {old!r}"
    mod = type(sys)(f"oracle_mutant_{tag}")
    exec(compile(src.replace(old, new), f"<mutant {fname}>", "exec"), mod.__dict__)
    return mod


def _cases(fn):
    """Keyword arguments of every parametrised instance of a test function."""
    combos = [{}]
    for mark in getattr(fn, "pytestmark", []):
        if mark.name != "parametrize":
            continue
        names, values = mark.args[0], mark.args[1]
        names = [n.strip() for n in names.split(",")] if isinstance(names, str) else list(names)
        combos = [{**c, **dict(zip(names, v if len(names) > 1 else (v,)))}
                  for c in combos for v in (getattr(x, "values", x) for x in values)]
    return combos


def _first_failing_pin(pins):
    for mod in pins:
        tests = [f for n, f in inspect.getmembers(mod, inspect.isfunction) if n.startswith("test_")]
        tests.sort(key=lambda f: f.__code__.co_firstlineno)
        for fn in tests:
            for kw in _cases(fn):
                try:
                    with np.errstate(all="ignore"):  # a mutant may produce NaN or inf
                        fn(**kw)
                except Exception:  # an assertion, or any error the mistake causes
                    return f"{mod.__name__}::{fn.__name__}{kw or ''}"
    return None


@pytest.mark.parametrize("name,fname,old,new,modules", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_the_mistake(name, fname, old, new, modules):
    tag = str(abs(hash(name)))
    mutant = _mutant(fname, old, new, tag)
    sys.path.insert(0, TESTS)
    try:
        pins = []
        for m in modules:
            pin = _load(os.path.join(TESTS, f"test_oracle_{m}.py"), f"pin_{m}_{tag}")
            for attr in dir(mutant):  # point the pin's oracle names at the mutant
                if not attr.startswith("_") and hasattr(pin, attr) and callable(getattr(mutant, attr)):
                    setattr(pin, attr, getattr(mutant, attr))
            pins.append(pin)
        caught = _first_failing_pin(pins)
    finally:
        sys.path.remove(TESTS)
    assert caught is not None, f"no pin of {modules} catches: {name}"
    print(f"{name}: caught by {caught}")
