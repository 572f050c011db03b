"""Pins of the oracle's rounding points (CPU only).

Two oracle functions are the reference for bit-level or near-bit-level claims:

* ``oracle.newton_schulz(..., "bf16")``, the reference of the bf16 iteration
  (X0, the Gram matrix, B and the new iterate are each rounded to bf16 once);
* ``oracle.adamw_step``, the bit-exact contract of the AdamW kernel (a fixed
  binary32 order of operations).

Both are pinned here by hand-worked cases in short binary fractions
(tests/golden/ns_bf16_cases.json, tests/golden/adamw_order_cases.json), whose
derivations are written out in the fixtures. To show that the cases can tell a
plausible misreading from the rule, each misreading is planted in a copy of the
oracle's own source (one textual edit, compiled and run on the CPU) and must
fail at least one case.
"""
import inspect
import json
import os
import textwrap

import numpy as np
import pytest

import oracle as O
import oracle.adamw as OA
import oracle.muon as OM

f32 = np.float32


def _hex(v):
    return float.fromhex(v) if isinstance(v, str) else float(v)


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as fh:
        return json.load(fh)


# ------------------------------------------------------------------ Newton-Schulz

def _ns_case_holds(ns, c) -> bool:
    x0 = np.array([[_hex(v) for v in r] for r in c["x0"]], dtype=np.float64)
    steps = [tuple(_hex(v) for v in t) for t in c["steps"]]
    u = np.array([[_hex(v) for v in r] for r in c["u"]], dtype=np.float64)
    got = ns(x0, steps, "bf16", len(steps))
    return got.shape == u.shape and np.array_equal(got, u)


def test_ns_bf16_hand_cases(golden_dir):
    doc = _load(golden_dir, "ns_bf16_cases.json")
    for c in doc["cases"]:
        assert _ns_case_holds(O.newton_schulz, c), c["name"]


def _mutant(module, func, old, new):
    """``module.func`` with one textual edit, compiled in the module's namespace."""
    src = textwrap.dedent(inspect.getsource(getattr(module, func)))
    assert src.count(old) == 1, f"planted edit does not apply: {old!r}"
    ns = dict(vars(module))
    exec(compile(src.replace(old, new), f"<mutant of {module.__name__}.{func}>", "exec"), ns)
    return ns[func]


NS_MISTAKES = {
    "X0 not rounded": ("X = _round(x0, precision)", "X = np.asarray(x0, dtype=f64)"),
    "Gram matrix not rounded": ("G = rnd(X @ X.T if wide else X.T @ X)", "G = (X @ X.T if wide else X.T @ X)"),
    "b A and c A A rounded apart": ("B = rnd(k(b) * G + k(c) * (G @ G))",
                                    "B = rnd(rnd(k(b) * G) + rnd(k(c) * (G @ G)))"),
    "B X rounded before a X is added": ("X = rnd(k(a) * X + (B @ X if wide else X @ B))",
                                        "X = rnd(k(a) * X + rnd(B @ X if wide else X @ B))"),
    "iterate not rounded": ("X = rnd(k(a) * X + (B @ X if wide else X @ B))",
                            "X = (k(a) * X + (B @ X if wide else X @ B))"),
    # B X^T has the shape of X^T: the mistaken iterate of a tall matrix comes back transposed
    "tall matrix multiplied on the wrong side": ("(B @ X if wide else X @ B)", "(B @ X if wide else B @ X.T)"),
}


@pytest.mark.parametrize("mistake", sorted(NS_MISTAKES))
def test_ns_bf16_planted_mistake_is_caught(golden_dir, mistake):
    old, new = NS_MISTAKES[mistake]
    ns = _mutant(OM, "newton_schulz", old, new)
    doc = _load(golden_dir, "ns_bf16_cases.json")
    caught = []
    for c in doc["cases"]:
        try:
            ok = _ns_case_holds(ns, c)
        except ValueError:   # shapes that do not conform
            ok = False
        if not ok:
            caught.append(c["name"])
    assert caught, f"no hand case detects: {mistake}"


# ------------------------------------------------------------------ AdamW

def _adamw_case_holds(step_fn, c) -> bool:
    p, m, v = step_fn(f32([_hex(c["p"])]), f32([_hex(c["g"])]), f32([_hex(c["m"])]), f32([_hex(c["v"])]),
                      c["step"], lr=_hex(c["lr"]), beta1=_hex(c["beta1"]), beta2=_hex(c["beta2"]),
                      eps=_hex(c["eps"]), weight_decay=_hex(c["weight_decay"]))
    for got, key in ((p, "p2"), (m, "m2"), (v, "v2")):
        if c[key] is None:
            continue
        if f32(got[0]).view(np.uint32) != f32(_hex(c[key])).view(np.uint32):
            return False
    return True


def test_adamw_order_hand_cases(golden_dir):
    doc = _load(golden_dir, "adamw_order_cases.json")
    for c in doc["cases"]:
        assert _adamw_case_holds(O.adamw_step, c), c["name"]


ADAMW_MISTAKES = {
    "(ss m) / den": ('p = p - k["ss"] * (m / den)', 'p = p - (k["ss"] * m) / den'),
    "sqrt(v) times 1/s2": ('den = np.sqrt(v) / k["s2"] + k["eps"]',
                           'den = np.sqrt(v) * (f32(1) / k["s2"]) + k["eps"]'),
    "first moment as lerp": ('m = k["b1"] * m + k["c1"] * g', 'm = m + k["c1"] * (g - m)'),
    "(c2 g) g": ('v = k["b2"] * v + k["c2"] * (g * g)', 'v = k["b2"] * v + (k["c2"] * g) * g'),
    "eps before the division": ('den = np.sqrt(v) / k["s2"] + k["eps"]', 'den = (np.sqrt(v) + k["eps"]) / k["s2"]'),
    "eps under the root": ('den = np.sqrt(v) / k["s2"] + k["eps"]', 'den = np.sqrt(v + k["eps"]) / k["s2"]'),
    "decay after the update": ('p = p - k["ss"] * (m / den)',
                               'p = p - k["ss"] * (m / den)\n        if k["decay"]:\n            p = p * k["cd"]'),
}


@pytest.mark.parametrize("mistake", sorted(ADAMW_MISTAKES))
def test_adamw_planted_order_mistake_is_caught(golden_dir, mistake):
    old, new = ADAMW_MISTAKES[mistake]
    fn = _mutant(OA, "adamw_step", old, new)
    if mistake == "decay after the update":
        # also take the decay out of its place before the moments
        src = textwrap.dedent(inspect.getsource(OA.adamw_step))
        first = '        if k["decay"]:\n            p = p * k["cd"]\n'
        assert src.count(first) == 1
        src = src.replace(first, "", 1).replace(old, new)
        ns = dict(vars(OA))
        exec(compile(src, "<mutant of oracle.adamw.adamw_step>", "exec"), ns)
        fn = ns["adamw_step"]
    doc = _load(golden_dir, "adamw_order_cases.json")
    caught = [c["name"] for c in doc["cases"] if not _adamw_case_holds(fn, c)]
    assert caught, f"no hand case detects: {mistake}"
