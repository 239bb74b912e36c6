"""GPU parity of attention on wide feature vectors (C = 64 ns > 64 features, stored feature-sliced [B,H,ns,N,64])
and of the wide feature maps, against the float64 oracle on the plain layout [B,H,N,C].

The features are the oracle's own maps of seeded inputs (positive random features with C = 128, 256, 1024;
the degree-2 polynomial map of 32-wide heads, C = 1 + 32 + 32^2 zero-padded to 1088), rounded to the storage
type: the attention then runs on exactly the values the oracle sees.  Gate: rowerr <= 1e-4 (float32 storage)
/ 2e-2 (bf16); the feature gradient of the queries is floored at 1e-2 of its numerator term |S_i g_i|, the
cancellation of the quotient rule, as for the 64-feature heads.
"""
import numpy as np
import pytest
import torch

import oracle
from linear_rnn_layers_amd import binding, inputs
from tests.feature_util import CANCEL_FLOOR, IDENT, store
from tests.gpu_util import TOL, dev, dev32, host, rowerr

pytestmark = pytest.mark.gpu

F32, BF16 = inputs.F32, inputs.BF16


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "the GPU tests need a GPU"
    binding.load()
    yield


def sl(x):
    """[B,H,N,C] -> feature-sliced [B,H,C/64,N,64] (host arrays)."""
    B, H, N, C = x.shape
    return np.ascontiguousarray(np.asarray(x).reshape(B, H, N, C // 64, 64).transpose(0, 1, 3, 2, 4))


def unsl(x):
    B, H, ns, N, c = x.shape
    return np.ascontiguousarray(np.asarray(x).transpose(0, 1, 3, 2, 4).reshape(B, H, N, ns * c))


def feats(kind, B, H, N, C, seed, dtype):
    """Positive features of seeded inputs from the oracle's maps, rounded to the storage type (float32 values)."""
    if kind == "random":
        x = inputs.gaussian((B, H, N, 32), seed, 0.3, F32)
        w = inputs.gaussian((H, C, 32), seed + 1, 1.0, F32)
        f = oracle.feature_performer(x, w)
    else:
        x = inputs.gaussian((B, H, N, 32), seed, 0.25, F32)
        f = oracle.feature_poly2(x, C)
    return store(f, dtype).astype(np.float32)


CASES = [("random", 128, 32, 200), ("random", 256, 64, 333), ("poly2", 1088, 32, 300)]


def _inputs(kind, C, M, N, dtype, seed):
    B, H = 2, 2
    fq = feats(kind, B, H, N, C, seed, dtype)
    fk = feats(kind, B, H, N, C, seed + 10, dtype)
    v = inputs.gaussian((B, H, N, M), seed + 20, 1.0, dtype)
    do = inputs.gaussian((B, H, N, M), seed + 21, 1.0, dtype)
    # an initial state: the oracle's state after a 40-token prefix of the same kind
    pq = feats(kind, B, H, 40, C, seed + 30, dtype)
    pv = inputs.gaussian((B, H, 40, M), seed + 31, 1.0, dtype)
    _, _, s0, z0 = oracle.forward_causal(pq, pq, pv, feature=IDENT)
    return fq, fk, v, do, s0.astype(np.float32), z0.astype(np.float32)


@pytest.mark.parametrize("chunks", [0, 1])
@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("kind,C,M,N", CASES)
def test_wide_causal(kind, C, M, N, dtype, chunks):
    """Forward (O, den, final state) and backward (feature gradients, dV, initial-state gradient, with an
    upstream final-state gradient), from the forward's checkpoint and from a recomputed one; chunks = 1 forces
    64-token segments (many segments per slice, their aggregates scanned)."""
    opts = binding.options(segment_chunks=chunks) if chunks else None
    fq, fk, v, do, s0, z0 = _inputs(kind, C, M, N, dtype, 20000 + C + M)
    B, H = fq.shape[:2]
    dsn = inputs.gaussian((B, H, C, M), 20100, 0.01, F32)
    dzn = inputs.gaussian((B, H, C), 20101, 0.01, F32)
    Q, K, V, dO = dev(sl(fq), dtype), dev(sl(fk), dtype), dev(v, dtype), dev(do, dtype)
    S0, Z0, dSN, dZN = dev32(s0), dev32(z0), dev32(dsn), dev32(dzn)
    out = binding.forward_causal(Q, K, V, s0=S0, z0=Z0, return_state=True, feature=IDENT, opts=opts)
    g1 = binding.backward_causal(Q, K, V, out["o"], out["den"], dO, s0=S0, z0=Z0, ckpt=out["ckpt"], ds_n=dSN,
                                 dz_n=dZN, state_grad=True, feature=IDENT, opts=opts)
    g2 = binding.backward_causal(Q, K, V, out["o"], out["den"], dO, s0=S0, z0=Z0, ds_n=dSN, dz_n=dZN,
                                 state_grad=True, feature=IDENT, opts=opts)
    torch.cuda.synchronize()
    ro, rden, rs, rz = oracle.forward_causal(fq, fk, v, s0, z0, feature=IDENT)
    rq, rk, rv, rs0, rz0 = oracle.backward_causal(fq, fk, v, do, s0, z0, dsn, dzn, state_grad=True, feature=IDENT)
    tol = TOL[dtype]
    errs = {"O": rowerr(host(out["o"]), ro), "den": rowerr(host(out["den"]), rden, False),
            "S_N": rowerr(host(out["s"]), rs), "Z_N": rowerr(host(out["z"]), rz, False)}
    assert max(errs.values()) <= tol, errs
    # the numerator term S_i g_i of dPhi_Q (S_i: the state after token i, from the initial state on), for its
    # cancellation floor
    S = np.asarray(s0, np.float64).copy()
    unum = np.empty(fq.shape)
    g = np.asarray(do, np.float64) / rden[..., None]
    for n in range(N):
        S += np.einsum("bhc,bhm->bhcm", fk[:, :, n].astype(np.float64), v[:, :, n].astype(np.float64))
        unum[:, :, n] = np.einsum("bhcm,bhm->bhc", S, g[:, :, n])
    floor = CANCEL_FLOOR * np.abs(unum).max(-1)
    for name, g_ in (("ckpt", g1), ("recomputed", g2)):
        dq, dk, dv, ds0, dz0 = (host(t) for t in g_)
        # dZ0 = dZ_N + sum_i c_i phi(Q_i) is a signed sum, one C-vector per head (a row, as for the 64-feature
        # heads)
        errs = {"dPhiQ": rowerr(unsl(dq), rq, row_floor=floor), "dPhiK": rowerr(unsl(dk), rk),
                "dV": rowerr(dv, rv), "dS0": rowerr(ds0, rs0), "dZ0": rowerr(dz0[:, :, None, :], rz0[:, :, None, :])}
        assert max(errs.values()) <= tol, (name, errs)


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("kind,C,M,N", CASES)
def test_wide_backward_is_deterministic(kind, C, M, N, dtype):
    """The sums over slices run in a fixed order: two backward calls agree bit for bit."""
    fq, fk, v, do, _, _ = _inputs(kind, C, M, N, dtype, 20400 + C)
    Q, K, V, dO = dev(sl(fq), dtype), dev(sl(fk), dtype), dev(v, dtype), dev(do, dtype)
    out = binding.forward_causal(Q, K, V, feature=IDENT)
    a = binding.backward_causal(Q, K, V, out["o"], out["den"], dO, ckpt=out["ckpt"], feature=IDENT)
    b = binding.backward_causal(Q, K, V, out["o"], out["den"], dO, ckpt=out["ckpt"], feature=IDENT)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("kind,C,M,N", CASES)
def test_wide_noncausal_forward(kind, C, M, N, dtype):
    fq, fk, v, _, _, _ = _inputs(kind, C, M, N, dtype, 20200 + C)
    Q, K, V = dev(sl(fq), dtype), dev(sl(fk), dtype), dev(v, dtype)
    o, s, z = binding.forward_noncausal(Q, K, V, feature=IDENT, return_state=True)
    torch.cuda.synchronize()
    fq64, fk64, v64 = (np.asarray(a, np.float64) for a in (fq, fk, v))
    rs = np.einsum("bhnc,bhnm->bhcm", fk64, v64)
    rz = fk64.sum(2)
    errs = {"O": rowerr(host(o), oracle.forward_noncausal(fq, fk, v, feature=IDENT)), "S": rowerr(host(s), rs),
            "Z": rowerr(host(z), rz, False)}
    assert max(errs.values()) <= TOL[dtype], errs


@pytest.mark.parametrize("totals", [False, True])
@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("kind,C,M,N", CASES)
def test_wide_noncausal_backward(kind, C, M, N, dtype, totals):
    """dPhi_Q, dPhi_K, dV of the non-causal form on wide feature vectors, with the forward's totals S, Z or
    forming them again; dPhi_Q floored at 1e-2 of |S g_i| and dPhi_K at 1e-2 of |R V_j| (the terms the
    quotient rule's share cancels, as for the 64-feature heads)."""
    fq, fk, v, do, _, _ = _inputs(kind, C, M, N, dtype, 20700 + C)
    Q, K, V, dO = dev(sl(fq), dtype), dev(sl(fk), dtype), dev(v, dtype), dev(do, dtype)
    s = z = None
    if totals:
        _, s, z = binding.forward_noncausal(Q, K, V, feature=IDENT, return_state=True)
    dq, dk, dv = binding.backward_noncausal(Q, K, V, dO, feature=IDENT, s=s, z=z)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.backward_noncausal(fq, fk, v, do, feature=IDENT)
    fq64, fk64, v64, do64 = (np.asarray(a, np.float64) for a in (fq, fk, v, do))
    S = np.einsum("bhnc,bhnm->bhcm", fk64, v64)
    g = do64 / np.einsum("bhnc,bhc->bhn", fq64, fk64.sum(2))[..., None]
    R = np.einsum("bhnc,bhnm->bhcm", fq64, g)
    fl_q = CANCEL_FLOOR * np.abs(np.einsum("bhcm,bhnm->bhnc", S, g)).max(-1)
    fl_k = CANCEL_FLOOR * np.abs(np.einsum("bhcm,bhnm->bhnc", R, v64)).max(-1)
    errs = {"dPhiQ": rowerr(unsl(host(dq)), rq, row_floor=fl_q), "dPhiK": rowerr(unsl(host(dk)), rk, row_floor=fl_k),
            "dV": rowerr(host(dv), rv)}
    assert max(errs.values()) <= TOL[dtype], errs


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("kind,C,M", [("random", 256, 64), ("poly2", 1088, 32), ("random", 4096, 32)])
def test_wide_decode(kind, C, M, dtype):
    """A prefill of 100 tokens by the wide forward, then 24 decode steps: y of every step and the final state
    against the oracle's recurrence over the whole sequence."""
    B, H, P, T = 3, 2, 100, 24
    f = feats(kind, B, H, P + T, C, 20300 + C, dtype)
    fk = feats(kind, B, H, P + T, C, 20310 + C, dtype)
    v = inputs.gaussian((B, H, P + T, M), 20320, 1.0, dtype)
    out = binding.forward_causal(dev(sl(f[:, :, :P]), dtype), dev(sl(fk[:, :, :P]), dtype), dev(v[:, :, :P], dtype),
                                 return_state=True, checkpoint=False, feature=IDENT)
    S, Z = out["s"], out["z"]
    ys = []
    for t in range(P, P + T):
        ys.append(host(binding.decode_step(dev(f[:, :, t], dtype), dev(fk[:, :, t], dtype), dev(v[:, :, t], dtype),
                                           S, Z, feature=IDENT)))
    torch.cuda.synchronize()
    ro, _, rs, rz = oracle.forward_causal(f, fk, v, feature=IDENT)
    errs = {"y": rowerr(np.stack(ys, 2), ro[:, :, P:]), "S": rowerr(host(S), rs), "Z": rowerr(host(Z), rz, False)}
    assert max(errs.values()) <= TOL[dtype], errs


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("Din,C", [(32, 128), (32, 256), (64, 256), (32, 1024)])
def test_wide_random_features(Din, C, dtype):
    """The map (one workgroup per slice) and its vector-Jacobian product (a sum over every slice)."""
    B, H, N = 2, 3, 333
    x = inputs.gaussian((B, H, N, Din), 20500 + Din + C, 0.3, dtype)
    w = inputs.gaussian((H, C, Din), 20501, 1.0, F32)
    dphi = inputs.gaussian((B, H, N, C), 20502, 1.0, dtype)
    phi = binding.feature_random(dev(x, dtype), dev32(w))
    dx = binding.feature_random_vjp(dev(x, dtype), dev32(w), dev(sl(dphi), dtype))
    torch.cuda.synchronize()
    assert tuple(phi.shape) == (B, H, C // 64, N, 64)
    assert rowerr(unsl(host(phi)), oracle.feature_performer(x, w)) <= TOL[dtype]
    assert rowerr(host(dx), oracle.feature_performer_vjp(x, w, dphi)) <= TOL[dtype]


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("Din,C", [(9, 128), (32, 1088), (40, 1664), (63, 4096)])
def test_wide_poly2_features(Din, C, dtype):
    B, H, N = 2, 2, 150
    x = inputs.gaussian((B, H, N, Din), 20600 + Din, 0.5, dtype)
    dphi = inputs.gaussian((B, H, N, C), 20601, 1.0, dtype)
    phi = binding.feature_poly2(dev(x, dtype), C)
    dx = binding.feature_poly2_vjp(dev(x, dtype), dev(sl(dphi), dtype))
    torch.cuda.synchronize()
    assert rowerr(unsl(host(phi)), oracle.feature_poly2(x, C)) <= TOL[dtype]
    assert rowerr(host(dx), oracle.feature_poly2_vjp(x, dphi)) <= TOL[dtype]


@pytest.mark.parametrize("name", ["mnist-rf256", "cifar-poly2"])
def test_wide_feature_workloads(name):
    """The two wide feature-map workloads at full size as the training step runs them: the map of Q and K, the
    causal attention on the features (checkpointed forward, backward), the chain rule back through the map; each
    stage against the oracle at its own inputs (random features C = 256: all 16 x 8 heads of 784 tokens; degree-2
    polynomial Din = 32, C = 1088: the 8 heads of batch entry 0 of 3072 tokens)."""
    w = inputs.MNIST_RF256 if name == "mnist-rf256" else inputs.CIFAR_POLY2
    q, k, v = w.qkv()
    do = w.grad_out()
    dt = w.dtype
    Q, K, V, dO = dev(q, dt), dev(k, dt), dev(v, dt), dev(do, dt)
    C = w.features
    if w.fmap == "random":
        wp = w.projection()
        W = dev32(wp)
        fmap, fvjp = (lambda a: oracle.feature_performer(a, wp)), (lambda a, g: oracle.feature_performer_vjp(a, wp, g))
        gmap, gvjp = (lambda a: binding.feature_random(a, W)), (lambda a, g: binding.feature_random_vjp(a, W, g))
    else:
        fmap, fvjp = (lambda a: oracle.feature_poly2(a, C)), oracle.feature_poly2_vjp
        gmap, gvjp = (lambda a: binding.feature_poly2(a, C)), binding.feature_poly2_vjp
    fQ, fK = gmap(Q), gmap(K)
    out = binding.forward_causal(fQ, fK, V, feature=IDENT)
    dfq, dfk, dv = binding.backward_causal(fQ, fK, V, out["o"], out["den"], dO, ckpt=out["ckpt"], feature=IDENT)
    dq, dk = gvjp(Q, dfq), gvjp(K, dfk)
    torch.cuda.synchronize()
    nb = w.B if w.fmap == "random" else 1
    cut = lambda a: np.asarray(a)[:nb]  # noqa: E731
    hs = lambda t: cut(unsl(host(t))) if t.dim() == 5 else cut(host(t))  # noqa: E731
    q, k, v, do = cut(q), cut(k), cut(v), cut(do)
    fq, fk, gq, gk = hs(fQ), hs(fK), hs(dfq), hs(dfk)
    tol = TOL[dt]
    assert max(rowerr(fq, fmap(q)), rowerr(fk, fmap(k))) <= tol
    ro, rden, _, _ = oracle.forward_causal(fq, fk, v, feature=IDENT)
    rq, rk, rv = oracle.backward_causal(fq, fk, v, do, feature=IDENT)
    g = np.asarray(do, np.float64) / rden[..., None]
    u = np.empty(fq.shape)
    for b in range(fq.shape[0]):
        for h in range(fq.shape[1]):
            u[b, h] = oracle.numerator_backward(fq[b, h], fk[b, h], v[b, h], g[b, h])[0]
    errs = {"O": rowerr(hs(out["o"]), ro), "den": rowerr(hs(out["den"]), rden, False), "dV": rowerr(hs(dv), rv),
            "dPhiQ": rowerr(gq, rq, row_floor=CANCEL_FLOOR * np.abs(u).max(-1)), "dPhiK": rowerr(gk, rk),
            "dQ": rowerr(hs(dq), fvjp(q, gq)), "dK": rowerr(hs(dk), fvjp(k, gk))}
    assert max(errs.values()) <= tol, errs
