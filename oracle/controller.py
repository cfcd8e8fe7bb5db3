"""The EchoKV bit-width controller, written out from its definition in plain Python (fp64).

TEST INFRASTRUCTURE: only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` use this module. The product library has its own controller and shares no code
with it.

EchoKV, "Show the math -- what the canary actually computes":
  - every canary reading delta_{l,b} (one per layer and width b in {2, 4, 8}) enters an
    exponential moving average  EMA <- (1 - alpha) * EMA + alpha * delta,  alpha = 0.1;
  - the layer's width is the least b whose EMA is below the budget tau;
  - the choice is made again from scratch at every firing, so layers move both ways
    ("Bidirectional adjustment -- promote AND demote");
  - the budget follows the context length L: tau(L) = tau0 * sqrt(L / L0), tau0 = 0.022 at
    L0 = 4K ("The tau(L) scaling").
EchoKV, "Measurement protocol -- warmup, freeze, measure", Phase 2: once frozen, the controller
takes no further updates.

Where the page is silent (readings of this implementation):
  - the first reading of a (layer, width) pair is its EMA (there is no earlier value to decay);
  - when no width meets the budget the layer goes to INT8, the widest tier;
  - before its first firing a layer keeps the width it was created with.
"""
from __future__ import annotations

import math

WIDTHS = (2, 4, 8)
ALPHA = 0.1
TAU0 = 0.022
L0 = 4096.0


def tau(context_len: float, tau0: float = TAU0, l0: float = L0) -> float:
    """EchoKV, "The tau(L) scaling": tau(L) = tau0 * sqrt(L / L0)"""
    return tau0 * math.sqrt(context_len / l0)


def choose(ema_row, budget: float) -> int:
    """the least width whose smoothed divergence is under the budget; INT8 when none is"""
    for b, e in zip(WIDTHS, ema_row):
        if e < budget:
            return b
    return 8


class Controller:
    def __init__(self, num_layers: int, initial_bits, alpha: float = ALPHA, tau0: float = TAU0,
                 l0: float = L0):
        self.alpha, self.tau0, self.l0 = float(alpha), float(tau0), float(l0)
        self.ema = [[None, None, None] for _ in range(num_layers)]
        self.bits = [int(b) for b in initial_bits]
        self.frozen = False
        self.firings = 0

    def observe(self, kl, context_len: float):
        """one canary firing: kl[l][j] is the reading of layer l at width WIDTHS[j]"""
        if self.frozen:
            return list(self.bits)
        budget = tau(context_len, self.tau0, self.l0)
        keep = 1.0 - self.alpha
        for l, row in enumerate(self.ema):
            for j in range(3):
                x = float(kl[l][j])
                row[j] = x if row[j] is None else keep * row[j] + self.alpha * x
            self.bits[l] = choose(row, budget)
        self.firings += 1
        return list(self.bits)
