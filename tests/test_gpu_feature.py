"""GPU parity of the other feature maps (degree-2 polynomial, positive random features) and of the attention in
feature mode (Q, K taken as feature vectors) against the float64 oracle.

Gate: rowerr <= 1e-4 (float32 storage) / 2e-2 (bf16), each step checked at its own inputs (the attention on
the features the library produced, the chain rule through the map on the feature gradients it produced), and
end to end against a chain of oracle steps only (the oracle's features, rounded to the storage type as the
library stores them, its attention and its chain rule), also through autograd.  The chain rule of a feature map
is a signed sum over the features, so an error within the gate in each feature gradient (at most the gate times
the row's largest |dPhi_c|) reaches dX as at most the gate times sum_c |d phi_c / dx| max_c' |dPhi_c'|: the
end-to-end rows are judged against that size (the propagated per-step gate).  The feature gradients dPhi_Q are floored at 1e-2 of the
numerator term |S_i g_i| (the cancellation of the quotient rule, as for dQ of the plain method); the raw
query gradient of the composition at 1e-2 of that term carried through the same map.
"""
import numpy as np
import pytest
import torch

import oracle
from linear_rnn_layers_amd import binding, inputs
from tests import pins
from tests.feature_util import (CANCEL_FLOOR, IDENT, feat_cancel_scale, feat_key_cancel_terms, poly2_vjp_terms,
                                rf_vjp_terms, store)
from tests.gpu_util import TOL, dev, dev32, host, rowerr

pytestmark = pytest.mark.gpu

F32, BF16 = inputs.F32, inputs.BF16


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "the GPU tests need a GPU"
    binding.load()
    yield


def _x(shape, seed, sigma, dtype):
    return inputs.gaussian(shape, seed, sigma, dtype)


def _w(H, C, Din, seed):
    return inputs.gaussian((H, C, Din), seed, 1.0, F32)


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("Din,C", [(32, 32), (32, 64), (64, 32), (64, 64)])
def test_random_features(Din, C, dtype):
    B, H, N = 2, 3, 150
    x = _x((B, H, N, Din), 14000 + Din + C, 0.3, dtype)
    w = _w(H, C, Din, 14010)
    dphi = _x((B, H, N, C), 14020, 1.0, dtype)
    phi = binding.feature_random(dev(x, dtype), dev32(w))
    dx = binding.feature_random_vjp(dev(x, dtype), dev32(w), dev(dphi, dtype))
    torch.cuda.synchronize()
    assert rowerr(host(phi), oracle.feature_performer(x, w)) <= TOL[dtype]
    assert rowerr(host(dx), oracle.feature_performer_vjp(x, w, dphi)) <= TOL[dtype]


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_random_features_several_chunks_per_workgroup(dtype):
    """2 x 2 heads of 38417 tokens (601 chunks, the last of 17 tokens): about 2404 chunks over about 1024
    workgroups, so each workgroup maps three chunks of one head with the projection staged once, and the
    last workgroup of every head a single ragged chunk."""
    B, H, N, Din, C = 2, 2, 38417, 32, 64
    x = _x((B, H, N, Din), 14050, 0.3, dtype)
    w = _w(H, C, Din, 14051)
    dphi = _x((B, H, N, C), 14052, 1.0, dtype)
    phi = binding.feature_random(dev(x, dtype), dev32(w))
    dx = binding.feature_random_vjp(dev(x, dtype), dev32(w), dev(dphi, dtype))
    torch.cuda.synchronize()
    assert rowerr(host(phi), oracle.feature_performer(x, w)) <= TOL[dtype]
    assert rowerr(host(dx), oracle.feature_performer_vjp(x, w, dphi)) <= TOL[dtype]


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("Din,C", [(3, 32), (5, 32), (7, 64), (4, 64)])
def test_poly2_features(Din, C, dtype):
    B, H, N = 2, 3, 150
    x = _x((B, H, N, Din), 14100 + Din + C, 1.0, dtype)
    dphi = _x((B, H, N, C), 14120, 1.0, dtype)
    phi = binding.feature_poly2(dev(x, dtype), C)
    dx = binding.feature_poly2_vjp(dev(x, dtype), dev(dphi, dtype))
    torch.cuda.synchronize()
    assert rowerr(host(phi), oracle.feature_poly2(x, C)) <= TOL[dtype]
    assert rowerr(host(dx), oracle.feature_poly2_vjp(x, dphi)) <= TOL[dtype]


def _attend(fq, fk, v, do, dtype, causal):
    """GPU attention in feature mode on device features: (O, dPhiQ, dPhiK, dV) as device tensors."""
    if causal:
        out = binding.forward_causal(fq, fk, v, feature=IDENT)
        g = binding.backward_causal(fq, fk, v, out["o"], out["den"], do, ckpt=out["ckpt"], feature=IDENT)
        return (out["o"],) + tuple(g)
    o = binding.forward_noncausal(fq, fk, v, feature=IDENT)
    return (o,) + tuple(binding.backward_noncausal(fq, fk, v, do, feature=IDENT))


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("which", ["random", "poly2"])
def test_feature_mode_attention(which, causal, dtype):
    """Features on the GPU, attention in feature mode, gradients through the features: against the oracle's
    float64 composition of the same steps."""
    B, H, N, M = 2, 2, 200, 32
    if which == "random":
        Din, C, sig = 32, 64, 0.3
        w = _w(H, C, Din, 14210)
        fmap = lambda a: oracle.feature_performer(a, w)  # noqa: E731
        fvjp = lambda a, g: oracle.feature_performer_vjp(a, w, g)  # noqa: E731
        gmap = lambda a: binding.feature_random(a, dev32(w))  # noqa: E731
        gvjp = lambda a, g: binding.feature_random_vjp(a, dev32(w), g)  # noqa: E731
    else:
        Din, C, sig = 5, 32, 0.6
        fmap = lambda a: oracle.feature_poly2(a, C)  # noqa: E731
        fvjp = oracle.feature_poly2_vjp
        gmap = lambda a: binding.feature_poly2(a, C)  # noqa: E731
        gvjp = binding.feature_poly2_vjp
    q, k = _x((B, H, N, Din), 14200, sig, dtype), _x((B, H, N, Din), 14201, sig, dtype)
    v, do = _x((B, H, N, M), 14202, 1.0, dtype), _x((B, H, N, M), 14203, 1.0, dtype)
    Q, K, V, dO = dev(q, dtype), dev(k, dtype), dev(v, dtype), dev(do, dtype)
    fQ, fK = gmap(Q), gmap(K)
    o, dfq, dfk, dv = _attend(fQ, fK, V, dO, dtype, causal)
    dq, dk = gvjp(Q, dfq), gvjp(K, dfk)
    torch.cuda.synchronize()
    # each step against the oracle at that step's own inputs: the features from the stored inputs, the attention
    # on the features the library produced, the feature gradients' chain rule on the gradients it produced
    fq, fk = host(fQ), host(fK)
    assert max(rowerr(fq, fmap(q)), rowerr(fk, fmap(k))) <= TOL[dtype]
    if causal:
        ro = oracle.forward_causal(fq, fk, v, feature=IDENT)[0]
        rfq, rfk, rv = oracle.backward_causal(fq, fk, v, do, feature=IDENT)
    else:
        ro = oracle.forward_noncausal(fq, fk, v, feature=IDENT)
        rfq, rfk, rv = oracle.backward_noncausal(fq, fk, v, do, feature=IDENT)
    u = feat_cancel_scale(fq, fk, v, do, causal)
    errs = {"O": rowerr(host(o), ro), "dV": rowerr(host(dv), rv),
            "dPhiQ": rowerr(host(dfq), rfq, row_floor=CANCEL_FLOOR * np.abs(u).max(-1)),
            "dPhiK": rowerr(host(dfk), rfk),
            "dQ": rowerr(host(dq), fvjp(q, host(dfq))), "dK": rowerr(host(dk), fvjp(k, host(dfk)))}
    assert max(errs.values()) <= TOL[dtype], errs
    # end to end, from the oracle alone: its features of the stored inputs (rounded to the storage type, as the
    # library stores them), its attention gradients on them, its chain rule -- nothing the library produced
    # enters the reference.  The chain rule is a signed sum over the features: its rows are judged against the
    # size of the summed terms at 1e-2, as the quotient rule's cancellation in dQ is.
    ofq, ofk = store(fmap(q), dtype), store(fmap(k), dtype)
    terms = (lambda a, g: rf_vjp_terms(a, w, g)) if which == "random" else poly2_vjp_terms
    if causal:
        oo = oracle.forward_causal(ofq, ofk, v, feature=IDENT)[0]
        ofq_g, ofk_g, ov = oracle.backward_causal(ofq, ofk, v, do, feature=IDENT)
    else:
        oo = oracle.forward_noncausal(ofq, ofk, v, feature=IDENT)
        ofq_g, ofk_g, ov = oracle.backward_noncausal(ofq, ofk, v, do, feature=IDENT)
    ou = feat_cancel_scale(ofq, ofk, v, do, causal)
    # each feature gradient's own floor (1e-2 of the numerator term its denominator share cancels) carried along
    # (the per-step gate bounds each element's error by the row's largest magnitude, so that is what every
    # feature's term carries)
    fq_abs = np.abs(ofq_g).max(-1, keepdims=True) + CANCEL_FLOOR * np.abs(ou).max(-1, keepdims=True)
    fq_abs = np.broadcast_to(fq_abs, ofq_g.shape)
    fk_abs = np.broadcast_to(np.abs(ofk_g).max(-1, keepdims=True), ofk_g.shape)
    if causal:
        fk_abs = fk_abs + CANCEL_FLOOR * feat_key_cancel_terms(ofq, ofk, v, do).max(-1, keepdims=True)
    chain = {"O": rowerr(host(o), oo), "dV": rowerr(host(dv), ov),
             "dQ": rowerr(host(dq), fvjp(q, ofq_g), row_floor=terms(q, fq_abs)),
             "dK": rowerr(host(dk), fvjp(k, ofk_g), row_floor=terms(k, fk_abs))}
    assert max(chain.values()) <= TOL[dtype], chain


def test_mnist_random_features_workload():
    """B=16 H=8 N=784 Din=32 float32 with 64 positive random features, every head, as the training step runs
    it: the features of Q and K, the causal attention in feature mode (checkpointed forward, backward), the
    chain rule back through the features; each step against the oracle at that step's own inputs."""
    w = inputs.MNIST_RF
    q, k, v = w.qkv()
    do = w.grad_out()
    wp = w.projection()
    Q, K, V, dO, W = dev(q), dev(k), dev(v), dev(do), dev32(wp)
    fQ, fK = binding.feature_random(Q, W), binding.feature_random(K, W)
    o, dfq, dfk, dv = _attend(fQ, fK, V, dO, F32, True)
    dq, dk = binding.feature_random_vjp(Q, W, dfq), binding.feature_random_vjp(K, W, dfk)
    torch.cuda.synchronize()
    fq, fk = host(fQ), host(fK)
    assert max(rowerr(fq, oracle.feature_performer(q, wp)), rowerr(fk, oracle.feature_performer(k, wp))) <= 1e-4
    ro = oracle.forward_causal(fq, fk, v, feature=IDENT)[0]
    rfq, rfk, rv = oracle.backward_causal(fq, fk, v, do, feature=IDENT)
    u = feat_cancel_scale(fq, fk, v, do)
    errs = {"O": rowerr(host(o), ro), "dV": rowerr(host(dv), rv),
            "dPhiQ": rowerr(host(dfq), rfq, row_floor=CANCEL_FLOOR * np.abs(u).max(-1)),
            "dPhiK": rowerr(host(dfk), rfk),
            "dQ": rowerr(host(dq), oracle.feature_performer_vjp(q, wp, host(dfq))),
            "dK": rowerr(host(dk), oracle.feature_performer_vjp(k, wp, host(dfk)))}
    assert max(errs.values()) <= 1e-4, errs
    # end to end from the oracle alone (its features, attention gradients and chain rule; the chain rule's rows
    # judged against the size of the terms it sums, as above)
    ofq, ofk = store(oracle.feature_performer(q, wp), F32), store(oracle.feature_performer(k, wp), F32)
    oo = oracle.forward_causal(ofq, ofk, v, feature=IDENT)[0]
    gq, gk, gv = oracle.backward_causal(ofq, ofk, v, do, feature=IDENT)
    ou = feat_cancel_scale(ofq, ofk, v, do)
    # each feature gradient's own floor carried along: 1e-2 of the numerator term its denominator share
    # cancels, or -- where larger -- the library's features' deviation from the oracle's (measured above, in
    # units of the gate) times that term: the attention's inputs differ by that much between the two chains,
    # and the cancellation passes the difference on at the scale of the cancelled term
    eps = max(rowerr(fq, ofq), rowerr(fk, ofk)) / 1e-4
    fac = max(CANCEL_FLOOR, eps)
    # (the per-step gate bounds each element's error by the row's largest magnitude, so that is what every
    # feature's term carries)
    rowmax = lambda a: np.broadcast_to(np.abs(a).max(-1, keepdims=True), a.shape)  # noqa: E731
    gq_abs = rowmax(gq) + fac * np.abs(ou).max(-1, keepdims=True)
    gk_abs = rowmax(gk) + fac * feat_key_cancel_terms(ofq, ofk, v, do).max(-1, keepdims=True)
    chain = {"O": rowerr(host(o), oo), "dV": rowerr(host(dv), gv),
             "dQ": rowerr(host(dq), oracle.feature_performer_vjp(q, wp, gq), row_floor=rf_vjp_terms(q, wp, gq_abs)),
             "dK": rowerr(host(dk), oracle.feature_performer_vjp(k, wp, gk), row_floor=rf_vjp_terms(k, wp, gk_abs))}
    assert max(chain.values()) <= 1e-4, chain


def test_feature_mode_with_elu_features_matches_the_method():
    """elu + 1 applied by torch, then feature mode, equals the library's own elu + 1 path."""
    B, H, N, D, M = 2, 2, 300, 64, 32
    q, k, v = (inputs.gaussian((B, H, N, d), 14300 + i, 1.0, F32) for i, d in enumerate((D, D, M)))
    do = inputs.gaussian((B, H, N, M), 14303)
    Q, K, V, dO = dev(q), dev(k), dev(v), dev(do)
    fQ, fK = torch.nn.functional.elu(Q) + 1.0, torch.nn.functional.elu(K) + 1.0
    a = binding.forward_causal(Q, K, V)
    b = binding.forward_causal(fQ, fK, V, feature=IDENT)
    ga = binding.backward_causal(Q, K, V, a["o"], a["den"], dO, ckpt=a["ckpt"])
    gb = binding.backward_causal(fQ, fK, V, b["o"], b["den"], dO, ckpt=b["ckpt"], feature=IDENT)
    torch.cuda.synchronize()
    dphi = lambda x: torch.where(x > 0, torch.ones_like(x), torch.exp(x))  # noqa: E731
    assert rowerr(host(b["o"]), host(a["o"])) <= 1e-5
    assert rowerr(host(gb[1] * dphi(K)), host(ga[1])) <= 1e-5
    assert rowerr(host(gb[2]), host(ga[2])) <= 1e-5


def test_feature_autograd_composition():
    """torch.autograd through random features and the causal attention in feature mode."""
    B, H, N, Din, C, M = 2, 2, 180, 32, 32, 64
    q, k = _x((B, H, N, Din), 14400, 0.3, F32), _x((B, H, N, Din), 14401, 0.3, F32)
    v, do = _x((B, H, N, M), 14402, 1.0, F32), _x((B, H, N, M), 14403, 1.0, F32)
    w = _w(H, C, Din, 14410)
    Q, K, V = (dev(a).requires_grad_(True) for a in (q, k, v))
    W = dev32(w)
    o = binding.causal_linear_attention(binding.random_features(Q, W), binding.random_features(K, W), V,
                                        feature=IDENT)
    (o * dev(do)).sum().backward()
    torch.cuda.synchronize()
    fq, fk = oracle.feature_performer(q, w), oracle.feature_performer(k, w)
    rfq, rfk, rv = oracle.backward_causal(fq, fk, v, do, feature=IDENT)
    u = feat_cancel_scale(fq, fk, v, do)
    rq, rk = oracle.feature_performer_vjp(q, w, rfq), oracle.feature_performer_vjp(k, w, rfk)
    errs = [rowerr(host(Q.grad), rq, row_floor=CANCEL_FLOOR * np.abs(oracle.feature_performer_vjp(q, w, u)).max(-1)),
            rowerr(host(K.grad), rk), rowerr(host(V.grad), rv)]
    assert max(errs) <= 1e-4, errs


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_feature_mode_with_decay(dtype):
    """Random features through the decayed recurrence (feature mode with logA): forward, the feature gradients
    and dlogA against the oracle at the same features; dPhi_Q and dlogA floored as in the decay tests."""
    B, H, N, Din, C, M = 2, 2, 300, 32, 32, 64
    q, k = _x((B, H, N, Din), 14500, 0.3, dtype), _x((B, H, N, Din), 14501, 0.3, dtype)
    v, do = _x((B, H, N, M), 14502, 1.0, dtype), _x((B, H, N, M), 14503, 1.0, dtype)
    w = _w(H, C, Din, 14510)
    la = (-np.log1p(np.exp(-(inputs.gaussian((B, H, N), 14511).astype(np.float64) + 2.0)))).astype(np.float32)
    Q, K, V, dO, LA = dev(q, dtype), dev(k, dtype), dev(v, dtype), dev(do, dtype), dev32(la)
    fQ, fK = binding.feature_random(Q, dev32(w)), binding.feature_random(K, dev32(w))
    out = binding.forward_causal(fQ, fK, V, feature=IDENT, log_a=LA)
    dfq, dfk, dv, dla = binding.backward_causal(fQ, fK, V, out["o"], out["den"], dO, ckpt=out["ckpt"],
                                                feature=IDENT, log_a=LA)
    torch.cuda.synchronize()
    fq, fk = host(fQ), host(fK)
    la = la.astype(np.float64)
    ro = oracle.forward_decay(fq, fk, v, la, feature=IDENT)[0]
    rfq, rfk, rv, rla, _, _ = oracle.backward_decay(fq, fk, v, la, do, feature=IDENT)
    # cancellation scales from the plain decayed recurrences on the features
    a = np.exp(la)
    S = np.zeros((B, H, C, M))
    Z = np.zeros((B, H, C))
    sq = np.empty((B, H, N))
    for t in range(N):
        S = a[:, :, t, None, None] * S + fk[:, :, t, :, None] * v[:, :, t, None, :]
        Z = a[:, :, t, None] * Z + fk[:, :, t]
        g = do[:, :, t] / (fq[:, :, t] * Z).sum(-1)[..., None]
        sq[:, :, t] = np.abs(np.einsum("bhcm,bhm->bhc", S, g)).max(-1)
    x = np.abs((fk * rfk).sum(-1))
    dla_floor = CANCEL_FLOOR * np.flip(np.cumsum(np.flip(x, -1), -1), -1)
    errs = {"O": rowerr(host(out["o"]), ro), "dV": rowerr(host(dv), rv), "dPhiK": rowerr(host(dfk), rfk),
            "dPhiQ": rowerr(host(dfq), rfq, row_floor=CANCEL_FLOOR * sq),
            "dlogA": rowerr(host(dla), rla, False, row_floor=dla_floor)}
    assert max(errs.values()) <= TOL[dtype], errs
