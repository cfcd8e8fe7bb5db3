"""Pins of the oracle's EchoKV controller (oracle/controller.py) against what the page and the
mathematics fix, none of which re-types the controller's update:

- the budget the page prints for 128K context (tests/golden/page_numbers.json), and tau(L0) = tau0;
- the EMA against its closed forms: a constant reading c after a first reading x0 leaves
  c + (1 - alpha)^n (x0 - c) after n more firings, and a general sequence gives the weighted sum
  (1 - alpha)^n x0 + sum_k alpha (1 - alpha)^(n - k) x_k;
- the firing at which a layer is promoted under a constant reading, from the closed form solved
  for n (a logarithm), in both directions (promotion and demotion);
- worked scenarios of the page's "Bidirectional adjustment" passage;
- freezing stops all updates; the INT8 fallback when no width meets the budget.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import controller as oc

HERE = os.path.dirname(os.path.abspath(__file__))


def golden():
    with open(os.path.join(HERE, "golden", "page_numbers.json")) as f:
        return json.load(f)


def test_tau_printed_at_128k():
    g = golden()["echokv_tau_128k"]
    t = oc.tau(g["context"], g["tau0"], g["L0"])
    assert round(t, 3) == g["value"]
    assert abs(oc.tau(4096) - 0.022) < 1e-15          # the budget at L0 is tau0 itself
    assert oc.ALPHA == golden()["echokv_ema_alpha"]["value"]
    # doubling the context scales the budget by sqrt(2)
    assert abs(oc.tau(2 * 131072) / oc.tau(131072) - math.sqrt(2)) < 1e-12


def run(readings, layers=1, initial=8, context=4096):
    c = oc.Controller(layers, [initial] * layers)
    hist = []
    for r in readings:
        hist.append(c.observe(r, context))
    return c, hist


@pytest.mark.parametrize("x0,cval,n", [(0.5, 0.01, 1), (0.5, 0.01, 7), (0.0, 0.3, 25), (1e-4, 2.0, 60)])
def test_ema_constant_reading_closed_form(x0, cval, n):
    readings = [[[x0, x0, x0]]] + [[[cval, cval, cval]]] * n
    c, _ = run(readings)
    expect = cval + (1 - 0.1) ** n * (x0 - cval)
    for e in c.ema[0]:
        assert abs(e - expect) <= 1e-12 * max(1.0, abs(expect))


def test_ema_weighted_sum_form():
    rng = np.random.default_rng(3)
    for _ in range(20):
        n = int(rng.integers(1, 40))
        xs = rng.exponential(0.05, size=(n + 1, 3))
        c, _ = run([[list(x)] for x in xs])
        a = 0.1
        for j in range(3):
            expect = (1 - a) ** n * xs[0, j] + sum(a * (1 - a) ** (n - k) * xs[k, j] for k in range(1, n + 1))
            assert abs(c.ema[0][j] - expect) <= 1e-12


def first_switch(x0, cval, budget, a=0.1):
    """least n >= 1 with c + (1-a)^n (x0 - c) on the other side of the budget than x0"""
    # (1-a)^n (x0 - c) crosses (budget - c): n > log((budget - c)/(x0 - c)) / log(1 - a)
    n = math.log((budget - cval) / (x0 - cval)) / math.log(1 - a)
    return max(1, math.floor(n) + 1)


@pytest.mark.parametrize("x0,cval", [(0.005, 0.06), (0.001, 0.5), (0.2, 0.001), (0.03, 0.0)])
def test_switch_firing_closed_form(x0, cval):
    budget = oc.tau(4096)                          # 0.022
    # INT2 readings move from x0 to c; INT4 and INT8 stay far below the budget
    readings = [[[x0, 0.0, 0.0]]] + [[[cval, 0.0, 0.0]]] * 200
    _, hist = run(readings)
    start = 2 if x0 < budget else 4
    assert hist[0] == [start]
    switched = [i for i, h in enumerate(hist) if h != [start]]
    n = first_switch(x0, cval, budget)
    assert switched[0] == n, (switched[:3], n)
    assert all(h != [start] for h in hist[n:])       # monotone drift: no switch back


def test_promote_and_demote_scenarios():
    # an INT2 layer whose INT2 divergence rises above the budget moves up to INT4
    budget = oc.tau(4096)
    c = oc.Controller(1, [2])
    assert c.observe([[0.001, 0.0005, 0.0001]], 4096) == [2]
    for _ in range(60):
        bits = c.observe([[0.5, 0.001, 0.0001]], 4096)
    assert bits == [4]
    # ... and to INT8 when INT4 rises too
    for _ in range(60):
        bits = c.observe([[0.5, 0.5, 0.001]], 4096)
    assert bits == [8]
    # an INT8 layer whose INT4 divergence falls back below the budget is demoted to INT4
    for _ in range(80):
        bits = c.observe([[0.5, 0.001, 0.001]], 4096)
    assert bits == [4]
    assert c.ema[0][1] < budget < c.ema[0][0]


def test_fallback_and_non_monotone():
    c = oc.Controller(3, [16, 16, 16])
    bits = c.observe([[1.0, 1.0, 1.0],        # nothing under the budget -> INT8
                      [0.01, 1.0, 1.0],       # only INT2 under it -> INT2 (least width wins)
                      [1.0, 1.0, 0.01]], 4096)
    assert bits == [8, 2, 8]


def test_first_reading_initialises_and_budget_uses_context():
    c = oc.Controller(1, [4])
    assert c.bits == [4]                       # before the first firing: as created
    c.observe([[0.05, 0.01, 0.0]], 131072)     # 0.05 < 0.124: INT2 at 128K
    assert c.ema[0] == [0.05, 0.01, 0.0] and c.bits == [2]
    c2 = oc.Controller(1, [4])
    c2.observe([[0.05, 0.01, 0.0]], 4096)      # 0.05 > 0.022: INT4 at 4K
    assert c2.bits == [4]


def test_freeze():
    c = oc.Controller(2, [8, 8])
    c.observe([[0.001, 0.001, 0.0], [1.0, 0.001, 0.0]], 4096)
    snap = ([list(r) for r in c.ema], list(c.bits), c.firings)
    c.frozen = True
    for _ in range(10):
        assert c.observe([[1.0, 1.0, 1.0], [0.0, 0.0, 0.0]], 4096) == snap[1]
    assert ([list(r) for r in c.ema], list(c.bits), c.firings) == snap
