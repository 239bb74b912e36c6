"""Oracle-side helpers of the feature-map tests: rounding oracle features to the storage type, and the sizes of
the terms that the chain rule and the quotient rule sum (the floors of rows that are cancellations)."""
import numpy as np

import oracle
from linear_rnn_layers_amd import binding, inputs

BF16 = inputs.BF16
IDENT = binding.LA_FEATURE_IDENTITY
CANCEL_FLOOR = 1e-2


def store(x, dtype):
    """Round oracle values to the storage type, as the library stores a feature tensor between the map and the
    attention (the oracle-only chain keeps this rounding: it is part of the computation the dtype defines)."""
    x = np.asarray(x, np.float64).astype(np.float32)
    return inputs.round_to_bf16(x).astype(np.float64) if dtype == BF16 else x.astype(np.float64)


def rf_vjp_terms(x, w, dphi):
    """Per-row size of the terms the random-feature chain rule dX = sum_c dPhi_c phi_c (W_c - x) sums (a signed
    sum over the features), bounded by sum_c |dPhi_c| phi_c (|W_c| + |x|), float64: an error of e |dPhi_c| in
    each feature gradient reaches dX as at most e times this size."""
    x, dphi = np.asarray(x, np.float64), np.asarray(dphi, np.float64)
    a = np.abs(dphi) * oracle.feature_performer(x, w)
    t = np.einsum("bhnc,hcd->bhnd", a, np.abs(np.asarray(w, np.float64))) + np.abs(x) * a.sum(-1, keepdims=True)
    return t.max(-1)


def poly2_vjp_terms(x, dphi):
    """Per-row size of the terms of the polynomial chain rule: the same sums with every term taken by magnitude."""
    return np.abs(oracle.feature_poly2_vjp(np.abs(np.asarray(x, np.float64)), np.abs(np.asarray(dphi, np.float64))))\
        .max(-1)


def feat_key_cancel_terms(fq, fk, v, do):
    """|sum_{i>=j} phi(Q_i) (g_i . V_j)|, the numerator term of dPhi_K that the denominator's share r cancels
    (causal, g = dO / den), elementwise, from the oracle on the features."""
    fq, fk, v, do = (np.asarray(a, np.float64) for a in (fq, fk, v, do))
    _, den, _, _ = oracle.forward_causal(fq, fk, v, feature=IDENT)
    g = do / den[..., None]
    out = np.empty(fk.shape)
    for b in range(fq.shape[0]):
        for h in range(fq.shape[1]):
            out[b, h] = oracle.numerator_backward(fq[b, h], fk[b, h], v[b, h], g[b, h])[1]
    return np.abs(out)


def feat_cancel_scale(fq, fk, v, do, causal=True):
    """Per-row |S_i g_i|, the numerator term of dPhi_Q (g = dO / den), from the oracle on the features."""
    fq, fk, v, do = (np.asarray(a, np.float64) for a in (fq, fk, v, do))
    if causal:
        _, den, _, _ = oracle.forward_causal(fq, fk, v, feature=IDENT)
    else:
        den = np.einsum("bhnd,bhd->bhn", fq, fk.sum(2))
    g = do / den[..., None]
    u = np.empty(fq.shape)
    for b in range(fq.shape[0]):
        for h in range(fq.shape[1]):
            if causal:
                u[b, h] = oracle.numerator_backward(fq[b, h], fk[b, h], v[b, h], g[b, h])[0]
            else:
                u[b, h] = g[b, h] @ (fk[b, h].T @ v[b, h]).T
    return u
