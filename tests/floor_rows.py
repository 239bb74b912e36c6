"""How many query-gradient rows the cancellation floor of the parity gate lifts, per workload (test
infrastructure: the oracle alone, on the workloads' seeded inputs).

The gate judges row r of dQ against max(|y_r|, 1e-3 max_head |y|, 1e-2 |S_i g_i (.) phi'(Q_i)|), the last term
being the floor on the eq. 13 term that the quotient rule's share cancels.  A row is "lifted" when that floor
is the largest of the three.  Run: python -m tests.floor_rows [workload ...] (default: mnist cifar long).
"""
from __future__ import annotations

import sys

import numpy as np

import oracle
from linear_rnn_layers_amd import inputs


def lifted_rows(q, k, v, do):
    """(rows, lifted rows, lifted rows past token 1, largest floor / row norm among lifted rows) over all heads of
    one input set (token 1's dQ is an exact zero, pin P4)."""
    q, k, v, do = (np.asarray(a, np.float64) for a in (q, k, v, do))
    _, den, _, _ = oracle.forward_causal(q, k, v)
    dq, _, _ = oracle.backward_causal(q, k, v, do)
    p = np.where(q > 0, q + 1, np.exp(q))
    kf = np.where(k > 0, k + 1, np.exp(k))
    g = do / den[..., None]
    B, H = q.shape[:2]
    n = lifted = later = 0
    worst = 0.0
    for b in range(B):
        for h in range(H):
            sq = oracle.numerator_backward(p[b, h], kf[b, h], v[b, h], g[b, h])[0]
            floor = 1e-2 * np.abs(sq * np.minimum(p[b, h], 1.0)).max(-1)
            yn = np.abs(dq[b, h]).max(-1)
            base = np.maximum(yn, 1e-3 * yn.max())
            hit = floor > base
            n += yn.size
            lifted += int(hit.sum())
            later += int(hit[1:].sum())
            if hit.any():
                worst = max(worst, float((floor[hit] / base[hit]).max()))
    return n, lifted, later, worst


def main(names):
    table = {"mnist": (inputs.MNIST, 1), "cifar": (inputs.CIFAR, 16), "long": (inputs.LONG, 1)}
    for name in names:
        w, layers = table[name]
        tot = lif = lat = 0
        worst = 0.0
        for layer in range(layers):
            q, k, v = w.qkv(layer)
            do = w.grad_out(layer)
            n, li, la, wr = lifted_rows(q, k, v, do)
            tot, lif, lat, worst = tot + n, lif + li, lat + la, max(worst, wr)
        print(f"{w.name}: {lif} of {tot} dQ rows lifted ({100.0 * lif / tot:.3f} %; {lat} past token 1), largest "
              f"floor / row norm {worst:.2f}", flush=True)


if __name__ == "__main__":
    main(sys.argv[1:] or ["mnist", "cifar", "long"])
