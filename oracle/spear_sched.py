"""Plain definition of the EC scheduler's selection step (test infrastructure only).

Method source: "SPEAR: A System for Post-Quantization Error-Adaptive Recovery
Enabling Efficient Low-Bit LLM Serving" (arXiv 2606.11244), Abstract: an
SLO-constrained, EC-aware scheduler decides where the error compensators run.
The abstract gives no rule; the reading taken here (and by the library) is a
0/1 choice per layer for one batch: keep the ECs of largest total weight whose
added time fits the slack left by the SLO.  Times are compared on a grid of G
steps (65536 for up to 256 layers, max(256, floor(65536 * 256 / n)) for n
layers beyond): the unit is u = max(slack / G, 1e-9), each layer's added time
is rounded up to whole units, and a set fits when its units sum to at most
min(G, floor(slack / u)) (rounding up never lets a chosen set exceed the
slack).  Among sets of the
largest weight (weights summed in layer order, as doubles) the one of fewest
units wins.  Layers with a negative added time (no EC) or weight 0 are never
chosen.

Nothing here is blocked or reordered: every subset of the candidate layers is
enumerated, so it is for small instances only.
"""

import itertools
import math

GRID_STEPS = 65536
FULL_GRID_LAYERS = 256


def grid_steps(n):
    """Grid steps for n layers."""
    return GRID_STEPS if n <= FULL_GRID_LAYERS else max(256, GRID_STEPS * FULL_GRID_LAYERS // n)


def grid(slack_us, n=1):
    """(unit, capacity in units) of the slack for n layers."""
    steps = grid_steps(n)
    unit = max(slack_us / steps, 1e-9)
    cap = min(steps, math.floor(slack_us / unit))
    return unit, cap


def units_of(extra_us, unit):
    """A layer's added time in whole grid units, rounded up."""
    return max(0, math.ceil(extra_us / unit - 1e-9))


def best_subset(extra_us, weights, slack_us):
    """(chosen index tuple, total weight, total units) of the best set."""
    if slack_us < 0:
        return (), 0.0, 0
    unit, cap = grid(slack_us, len(extra_us))
    cand = [i for i in range(len(extra_us)) if extra_us[i] >= 0 and float(weights[i]) > 0]
    best = ((), 0.0, 0)
    for k in range(1, len(cand) + 1):
        for sub in itertools.combinations(cand, k):
            u = sum(units_of(extra_us[i], unit) for i in sub)
            if u > cap:
                continue
            w = 0.0
            for i in sub:                      # layer order
                w += float(weights[i])
            if w > best[1] or (w == best[1] and u < best[2]):
                best = (sub, w, u)
    return best
