"""Independent reference computations used to pin the oracle.

Nothing here calls the oracle or the HIP library.  phi comes from PyTorch's
library ``elu`` (alpha = 1) plus one, and the attention is the quadratic
masked definition of "Transformers are RNNs -- part 2/3" eq. 8 (non-causal:
eq. 3 of the reading notes) evaluated in float64 with numpy.
"""
from __future__ import annotations

import fractions
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def phi_lib(x: np.ndarray) -> np.ndarray:
    """elu(x) + 1 via torch.nn.functional.elu (a library routine), float64."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))
    return (torch.nn.functional.elu(t, alpha=1.0) + 1.0).numpy()


def brute_causal(q, k, v):
    """eq. 8 with sim(q, k) = phi(q) . phi(k): O_i = sum_{j<=i} s_ij V_j / sum_{j<=i} s_ij."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    B, H, N, _ = q.shape
    out = np.empty(v.shape)
    den = np.empty((B, H, N))
    mask = np.tril(np.ones((N, N)))
    for b in range(B):
        for h in range(H):
            sim = (phi_lib(q[b, h]) @ phi_lib(k[b, h]).T) * mask
            den[b, h] = sim.sum(axis=1)
            out[b, h] = (sim @ v[b, h]) / den[b, h][:, None]
    return out, den


def brute_noncausal(q, k, v):
    """Unmasked form (reading notes eq. 3 with the same sim)."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    out = np.empty(v.shape)
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            sim = phi_lib(q[b, h]) @ phi_lib(k[b, h]).T
            out[b, h] = (sim @ v[b, h]) / sim.sum(axis=1)[:, None]
    return out


def brute_noncausal_grad(q, k, v, do):
    """Gradients of sum(dO * O) of the unmasked form, by PyTorch autograd in float64 (library elu)."""
    ts = [torch.tensor(np.asarray(a, dtype=np.float64), requires_grad=True) for a in (q, k, v)]
    tq, tk, tv = ts
    pq = torch.nn.functional.elu(tq, alpha=1.0) + 1.0
    pk = torch.nn.functional.elu(tk, alpha=1.0) + 1.0
    sim = pq @ pk.transpose(-1, -2)
    out = (sim @ tv) / sim.sum(dim=-1, keepdim=True)
    (out * torch.from_numpy(np.asarray(do, dtype=np.float64))).sum().backward()
    return tuple(t.grad.numpy() for t in ts)


def brute_causal_state_grad(q, k, v, s0, z0, do, dsn, dzn):
    """Gradients of sum(dO * O) + sum(dSN * S_N) + sum(dZN * Z_N) with respect to Q, K, V, S0, Z0, by
    PyTorch autograd in float64 (library elu), where O is eq. 8's masked quotient with the initial state
    added to both sums and S_N = S0 + sum_j phi(K_j) V_j^T, Z_N = Z0 + sum_j phi(K_j)."""
    ts = [torch.tensor(np.asarray(a, dtype=np.float64), requires_grad=True) for a in (q, k, v, s0, z0)]
    tq, tk, tv, ts0, tz0 = ts
    pq = torch.nn.functional.elu(tq, alpha=1.0) + 1.0
    pk = torch.nn.functional.elu(tk, alpha=1.0) + 1.0
    n = tq.shape[-2]
    sim = (pq @ pk.transpose(-1, -2)) * torch.tril(torch.ones((n, n), dtype=torch.float64))
    num = sim @ tv + pq @ ts0
    den = sim.sum(dim=-1) + (pq * tz0.unsqueeze(-2)).sum(dim=-1)
    out = num / den.unsqueeze(-1)
    s_n = ts0 + pk.transpose(-1, -2) @ tv
    z_n = tz0 + pk.sum(dim=-2)
    f = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))  # noqa: E731
    ((out * f(do)).sum() + (s_n * f(dsn)).sum() + (z_n * f(dzn)).sum()).backward()
    return tuple(t.grad.numpy() for t in ts)


def brute_decay(q, k, v, log_a, s0=None, z0=None):
    """Decayed attention as an explicit weighted average: token j's weight at query i >= j is
    (phi(q_i).phi(k_j)) times the product of the decays a_{j+1} .. a_i, the initial state's weight the
    product a_1 .. a_i (products of the gates formed one by one).  Returns (O, den, S_N, Z_N)."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    a = np.exp(np.asarray(log_a, dtype=np.float64))
    B, H, N, D = q.shape
    M = v.shape[-1]
    out = np.empty((B, H, N, M))
    den = np.empty((B, H, N))
    sn = np.empty((B, H, D, M))
    zn = np.empty((B, H, D))
    for b in range(B):
        for h in range(H):
            pq, pk = phi_lib(q[b, h]), phi_lib(k[b, h])
            w = np.zeros((N, N + 1))  # column 0: the initial state, column j + 1: token j
            for i in range(N):
                prod = 1.0
                for j in range(i, -1, -1):
                    w[i, j + 1] = prod
                    prod *= a[b, h, j]
                w[i, 0] = prod
            s_init = np.zeros((D, M)) if s0 is None else np.asarray(s0, np.float64)[b, h]
            z_init = np.zeros(D) if z0 is None else np.asarray(z0, np.float64)[b, h]
            sim = (pq @ pk.T) * w[:, 1:]
            num = sim @ v[b, h] + w[:, :1] * (pq @ s_init)
            den[b, h] = sim.sum(axis=1) + w[:, 0] * (pq @ z_init)
            out[b, h] = num / den[b, h][:, None]
            wl = w[N - 1] if N else np.array([1.0])
            sn[b, h] = wl[0] * s_init + (pk * wl[1:, None]).T @ v[b, h]
            zn[b, h] = wl[0] * z_init + (pk * wl[1:, None]).sum(axis=0)
    return out, den, sn, zn


def brute_decay_grad(q, k, v, log_a, s0, z0, do, dsn, dzn):
    """Gradients of sum(dO*O) + sum(dSN*S_N) + sum(dZN*Z_N) of the decayed form with respect to Q, K, V,
    logA, S0, Z0 by PyTorch autograd in float64: weights exp(L_i - L_j) with L the running sum of logA."""
    ts = [torch.tensor(np.asarray(x, dtype=np.float64), requires_grad=True) for x in (q, k, v, log_a, s0, z0)]
    tq, tk, tv, tla, ts0, tz0 = ts
    pq = torch.nn.functional.elu(tq, alpha=1.0) + 1.0
    pk = torch.nn.functional.elu(tk, alpha=1.0) + 1.0
    n = tq.shape[-2]
    lam = torch.cumsum(tla, dim=-1)
    mask = torch.tril(torch.ones((n, n), dtype=torch.bool))
    diff = lam.unsqueeze(-1) - lam.unsqueeze(-2)
    w = torch.where(mask, torch.exp(torch.where(mask, diff, torch.zeros_like(diff))), torch.zeros_like(diff))
    sim = (pq @ pk.transpose(-1, -2)) * w
    w0 = torch.exp(lam)
    num = sim @ tv + w0.unsqueeze(-1) * (pq @ ts0)
    den = sim.sum(dim=-1) + w0 * (pq * tz0.unsqueeze(-2)).sum(dim=-1)
    out = num / den.unsqueeze(-1)
    wl = w[..., n - 1, :]
    s_n = w0[..., n - 1, None, None] * ts0 + (pk * wl.unsqueeze(-1)).transpose(-1, -2) @ tv
    z_n = w0[..., n - 1, None] * tz0 + (pk * wl.unsqueeze(-1)).sum(dim=-2)
    f = lambda x: torch.from_numpy(np.asarray(x, dtype=np.float64))  # noqa: E731
    ((out * f(do)).sum() + (s_n * f(dsn)).sum() + (z_n * f(dzn)).sum()).backward()
    return tuple(t.grad.numpy() for t in ts)


def brute_poly2_attention_grad(q, k, v, do, causal=True):
    """Attention with the degree-2 polynomial kernel sim(q, k) = 1 + q.k + (q.k)^2 written directly (no feature
    map), O and the gradients of sum(dO * O) with respect to q, k, v by PyTorch autograd in float64."""
    ts = [torch.tensor(np.asarray(a, dtype=np.float64), requires_grad=True) for a in (q, k, v)]
    tq, tk, tv = ts
    dot = tq @ tk.transpose(-1, -2)
    sim = 1.0 + dot + dot * dot
    if causal:
        n = tq.shape[-2]
        sim = sim * torch.tril(torch.ones((n, n), dtype=torch.float64))
    out = (sim @ tv) / sim.sum(dim=-1, keepdim=True)
    (out * torch.from_numpy(np.asarray(do, dtype=np.float64))).sum().backward()
    return (out.detach().numpy(),) + tuple(t.grad.numpy() for t in ts)


def brute_numerator(p, kf, vb):
    """Numerator of eq. 9 on feature-mapped inputs: Vbar_i = sum_{j<=i} (P_i . Kf_j) Vb_j."""
    n = p.shape[0]
    return (np.tril(np.ones((n, n))) * (p @ kf.T)) @ vb


def load_golden(name: str = "worked_example.txt"):
    """Parse the hand-derived worked examples: {key: list of Fractions}."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rhs = line.partition("=")
            out[key.strip()] = [fractions.Fraction(tok) for tok in rhs.split()]
    return out


def golden_array(g, key, shape):
    return np.array([float(x) for x in g[key]], dtype=np.float64).reshape(shape)


def rel_err(x, y):
    """max |x - y| / max |y| (tensor-wide), 0 when both are zero."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    scale = np.max(np.abs(y)) if y.size else 0.0
    diff = np.max(np.abs(x - y)) if y.size else 0.0
    return diff / scale if scale > 0 else diff
