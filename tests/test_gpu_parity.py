"""GPU parity: the HIP library against the float64 oracle, element by element.

Gate (per output tensor): rowerr <= 1e-4 for float32 storage and <= 2e-2
for bf16 storage (tests/gpu_util.py defines rowerr).  Every call goes through
the C ABI via the ctypes binding; the oracle runs on the host CPU.
"""
import numpy as np
import pytest
import torch

import oracle
from linear_rnn_layers_amd import binding, inputs
from tests import pins
from tests.gpu_util import TOL, dev, dev32, host, rowerr

pytestmark = pytest.mark.gpu

F32, BF16 = inputs.F32, inputs.BF16


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "the GPU tests need a GPU"
    binding.load()
    yield


def _qkv(B, H, N, D, M, dtype, seed, sigma=1.0):
    q = inputs.gaussian((B, H, N, D), seed, sigma, dtype)
    k = inputs.gaussian((B, H, N, D), seed + 1, sigma, dtype)
    v = inputs.gaussian((B, H, N, M), seed + 2, sigma, dtype)
    return q, k, v


def gpu_forward(q, k, v, dtype, s0=None, z0=None, opts=None):
    out = binding.forward_causal(dev(q, dtype), dev(k, dtype), dev(v, dtype),
                                 s0=None if s0 is None else dev32(s0), z0=None if z0 is None else dev32(z0),
                                 return_state=True, checkpoint=True, opts=opts)
    torch.cuda.synchronize()
    return out


def check_forward(q, k, v, dtype, s0=None, z0=None, tol=None, opts=None):
    tol = TOL[dtype] if tol is None else tol
    out = gpu_forward(q, k, v, dtype, s0, z0, opts)
    o, den, s, z = oracle.forward_causal(q, k, v, s0, z0)
    errs = {"O": rowerr(host(out["o"]), o), "den": rowerr(host(out["den"]), den, False),
            "S_N": rowerr(host(out["s"]), s), "Z_N": rowerr(host(out["z"]), z, False)}
    assert max(errs.values()) <= tol, errs
    return out


SWEEP_N = [1, 2, 15, 16, 17, 63, 64, 65, 129, 784]
DM = [(32, 32), (64, 64), (32, 64), (64, 32)]


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("D,M", DM)
@pytest.mark.parametrize("N", SWEEP_N)
def test_forward_causal_sweep(N, D, M, dtype):
    q, k, v = _qkv(2, 3, N, D, M, dtype, 1000 + N)
    check_forward(q, k, v, dtype)


def test_small_workload_forward():
    """B=1 H=1 N=64 D=M=32 float32, against the oracle and the quadratic eq. 8."""
    w = inputs.SMALL
    q, k, v = w.qkv()
    out = check_forward(q, k, v, F32)
    ob, denb = pins.brute_causal(q, k, v)
    assert rowerr(host(out["o"]), ob) <= 1e-4
    assert rowerr(host(out["den"]), denb, False) <= 1e-4


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_forward_initial_state_and_split(dtype):
    """Continuing from (S0, Z0) matches the oracle and the unsplit sequence."""
    B, H, N, D, M = 2, 2, 300, 64, 32
    q, k, v = _qkv(B, H, N, D, M, dtype, 2000)
    _, _, s0, z0 = oracle.forward_causal(q[:, :, :111], k[:, :, :111], v[:, :, :111])
    check_forward(q[:, :, 111:], k[:, :, 111:], v[:, :, 111:], dtype, s0, z0)


@pytest.mark.parametrize("chunks", [1, 2, 3, 5])
def test_segment_length_invariance(chunks):
    """Results do not depend on how the sequence is cut into segments."""
    B, H, N, D, M = 2, 2, 784, 32, 32
    q, k, v = _qkv(B, H, N, D, M, F32, 3000)
    do = inputs.gaussian((B, H, N, M), 3004)
    opts = binding.options(segment_chunks=chunks)
    assert binding.segment_length(B, H, N, D, M, opts) == 64 * chunks
    out = check_forward(q, k, v, F32, opts=opts)
    dq, dk, dv = binding.backward_causal(dev(q), dev(k), dev(v), out["o"], out["den"], dev(do), ckpt=out["ckpt"],
                                         opts=opts)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.backward_causal(q, k, v, do)
    errs = [rowerr(host(dq), rq, row_floor=CANCEL_FLOOR * dq_cancel_scale(q, k, v, do)), rowerr(host(dk), rk),
            rowerr(host(dv), rv)]
    assert max(errs) <= 1e-4, errs


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("D,M", DM)
@pytest.mark.parametrize("N", [1, 17, 64, 200, 784])
def test_forward_noncausal_sweep(N, D, M, dtype):
    q, k, v = _qkv(2, 3, N, D, M, dtype, 4000 + N)
    o = binding.forward_noncausal(dev(q, dtype), dev(k, dtype), dev(v, dtype))
    torch.cuda.synchronize()
    assert rowerr(host(o), oracle.forward_noncausal(q, k, v)) <= TOL[dtype]


# The query gradient of eq. 13 with the denominator's share,
#   dphiQ_i = S_i g_i + c_i Z_i,
# is a cancellation: its first term S_i g_i is removed along Z_i, exactly so
# for token 1 (pin P4: O_1 = V_1 whatever Q, K are) and nearly so for rows
# that happen to be small.  A relative error of such a row is limited by the
# working precision of the terms it cancels, so each dQ row is measured
# against the largest of |row|, 1e-3 x its head's largest row, and
# CANCEL_FLOOR x |S_i g_i * phi'(Q_i)| (the oracle's eq. 13 first term).  At
# the float32 gate this allows 1e-6 of the cancelled terms, i.e. about 16
# float32 ulps.
CANCEL_FLOOR = 1e-2


def dq_cancel_scale(q, k, v, do, s0=None, z0=None):
    """Per-row |S_i g_i * phi'(Q_i)|_inf from the oracle (eq. 13's first term, g_i = dO_i / den_i)."""
    _, den, _, _ = oracle.forward_causal(q, k, v, s0, z0)
    pq, pk = pins.phi_lib(q), pins.phi_lib(k)
    g = do.astype(np.float64) / den[..., None]
    u = np.empty(q.shape)
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            u[b, h] = oracle.numerator_backward(pq[b, h], pk[b, h], v[b, h], g[b, h])[0]
    if s0 is not None:
        u += np.einsum("bhdm,bhnm->bhnd", s0, g)
    return np.abs(u * np.minimum(pq, 1.0)).max(-1)


def check_backward(q, k, v, do, dtype, s0=None, z0=None, use_ckpt=True, tol=None):
    tol = TOL[dtype] if tol is None else tol
    out = gpu_forward(q, k, v, dtype, s0, z0)
    Q, K, V = dev(q, dtype), dev(k, dtype), dev(v, dtype)
    dq, dk, dv = binding.backward_causal(Q, K, V, out["o"], out["den"], dev(do, dtype),
                                         s0=None if s0 is None else dev32(s0), z0=None if z0 is None else dev32(z0),
                                         ckpt=out["ckpt"] if use_ckpt else None)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.backward_causal(q, k, v, do, s0, z0)
    dq, dk, dv = host(dq), host(dk), host(dv)
    errs = {"dV": rowerr(dv, rv),
            "dQ": rowerr(dq, rq, row_floor=CANCEL_FLOOR * dq_cancel_scale(q, k, v, do, s0, z0))}
    if s0 is None and q.shape[2] == 1:
        # N = 1: dK_1 = phi(Q_1) g_1.(V_1 - O_1) is an exact zero too; terms of size |phi(Q_1)| |g_1.V_1|
        pq, pk = pins.phi_lib(q[:, :, 0]), pins.phi_lib(k[:, :, 0])
        scale = np.abs((v[:, :, 0].astype(np.float64) * do[:, :, 0]).sum(-1)) / (pq * pk).sum(-1) * pq.max(-1)
        errs["dK"] = float((np.abs(dk[:, :, 0]).max(-1) / (CANCEL_FLOOR * scale)).max())
    else:
        errs["dK"] = rowerr(dk, rk)
    assert max(errs.values()) <= tol, errs
    return dq, dk, dv


def test_first_token_query_gradient_vanishes():
    """Pin P4 on the GPU path: dQ of token 1 is zero to working precision of the cancelled terms."""
    for dtype, kappa in ((F32, 1e-5), (BF16, 1e-3)):
        q, k, v = _qkv(3, 4, 40, 64, 32, dtype, 7100)
        do = inputs.gaussian((3, 4, 40, 32), 7104, 1.0, dtype)
        dq, _, _ = check_backward(q, k, v, do, dtype)
        scale = dq_cancel_scale(q, k, v, do)[:, :, 0]
        assert (np.abs(dq[:, :, 0]).max(-1) / scale).max() <= kappa


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("D,M", DM)
@pytest.mark.parametrize("N", [1, 2, 17, 64, 65, 200, 784])
def test_backward_causal_sweep(N, D, M, dtype):
    q, k, v = _qkv(2, 3, N, D, M, dtype, 5000 + N)
    do = inputs.gaussian((2, 3, N, M), 5999, 1.0, dtype)
    check_backward(q, k, v, do, dtype)


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("use_ckpt", [True, False])
def test_backward_with_initial_state(dtype, use_ckpt):
    B, H, N, D, M = 2, 2, 333, 32, 64
    q, k, v = _qkv(B, H, N, D, M, dtype, 6000)
    do = inputs.gaussian((B, H, N, M), 6003, 1.0, dtype)
    _, _, s0, z0 = oracle.forward_causal(*_qkv(B, H, 50, D, M, dtype, 6100))
    check_backward(q, k, v, do, dtype, s0, z0, use_ckpt)


def test_backward_first_row_and_euler_identity():
    """sum_d dQ_id rho(Q_id) = 0 per row (phi-homogeneity of O_i in phi(Q_i)), on GPU outputs."""
    B, H, N, D, M = 2, 2, 256, 32, 32
    q, k, v = _qkv(B, H, N, D, M, F32, 7000)
    do = inputs.gaussian((B, H, N, M), 7003)
    dq, _, _ = check_backward(q, k, v, do, F32)
    scale = np.abs(dq).max()
    rho = np.where(q > 0, q + 1.0, 1.0)
    assert np.abs((dq * rho).sum(-1)).max() <= 1e-5 * scale * D


def test_determinism():
    """Two runs of forward + backward give bit-identical results."""
    B, H, N, D, M = 4, 4, 1000, 64, 64
    q, k, v = _qkv(B, H, N, D, M, BF16, 8000)
    do = inputs.gaussian((B, H, N, M), 8003, 1.0, BF16)
    Q, K, V, dO = dev(q, BF16), dev(k, BF16), dev(v, BF16), dev(do, BF16)
    res = []
    for _ in range(2):
        out = binding.forward_causal(Q, K, V)
        grads = binding.backward_causal(Q, K, V, out["o"], out["den"], dO, ckpt=out["ckpt"])
        torch.cuda.synchronize()
        res.append([out["o"].clone(), out["den"].clone()] + [g.clone() for g in grads])
    for a, b in zip(*res):
        assert torch.equal(a, b)


# ------------------------------------------------------------ decode steps
@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("D,M", DM)
def test_decode_steps(D, M, dtype):
    B, H, T = 3, 5, 20
    q, k, v = _qkv(B, H, T, D, M, dtype, 9000 + D + M)
    s = torch.zeros((B, H, D, M), device="cuda")
    z = torch.zeros((B, H, D), device="cuda")
    ys = []
    for t in range(T):
        y = binding.decode_step(dev(q[:, :, t], dtype), dev(k[:, :, t], dtype), dev(v[:, :, t], dtype), s, z)
        ys.append(host(y))
    torch.cuda.synchronize()
    o, _, so, zo = oracle.forward_causal(q, k, v)
    assert rowerr(np.stack(ys, axis=2), o) <= TOL[dtype]
    assert rowerr(host(s), so) <= 1e-4 and rowerr(host(z), zo, False) <= 1e-4


def test_prefill_then_decode_equals_forward():
    """A GPU prefill's final state continued by GPU decode steps matches the oracle's one-pass forward."""
    B, H, N, D, M, P = 2, 3, 100, 64, 64, 70
    q, k, v = _qkv(B, H, N, D, M, BF16, 9500)
    out = gpu_forward(q[:, :, :P], k[:, :, :P], v[:, :, :P], BF16)
    s, z = out["s"], out["z"]
    o, _, so, zo = oracle.forward_causal(q, k, v)
    for t in range(P, N):
        y = binding.decode_step(dev(q[:, :, t], BF16), dev(k[:, :, t], BF16), dev(v[:, :, t], BF16), s, z)
        assert rowerr(host(y), o[:, :, t]) <= 2e-2
    assert rowerr(host(s), so) <= 1e-4


# --------------------------------------------------------- full workloads
def test_mnist_workload():
    """B=16 H=8 N=784 D=M=32 float32, every head element by element: causal forward (O, den, S_N, Z_N), causal
    backward and non-causal forward."""
    w = inputs.MNIST
    q, k, v = w.qkv()
    do = w.grad_out()
    check_forward(q, k, v, F32)
    check_backward(q, k, v, do, F32)
    o = binding.forward_noncausal(dev(q), dev(k), dev(v))
    torch.cuda.synchronize()
    assert rowerr(host(o), oracle.forward_noncausal(q, k, v)) <= 1e-4


@pytest.mark.parametrize("layer", [0, 15])
def test_cifar_workload_layer(layer):
    """B=4 H=8 N=3072 D=M=32 bf16, sigma = 0.5: forward + backward of one layer of the stack."""
    w = inputs.CIFAR
    q, k, v = w.qkv(layer)
    do = w.grad_out(layer)
    check_forward(q, k, v, BF16)
    check_backward(q, k, v, do, BF16)


def test_long_workload():
    """B=1 H=16 N=65536 D=M=64 bf16, inputs scaled by 1/sqrt(D), all heads element by element: forward (O, den,
    S_N, Z_N) and backward (dQ, dK, dV), in the segment plan and launch configuration the benchmark times."""
    w = inputs.LONG
    q, k, v = w.qkv()
    do = w.grad_out()
    check_forward(q, k, v, BF16)
    check_backward(q, k, v, do, BF16)


@pytest.mark.parametrize("mean", [4.0, -3.0])
def test_backward_values_around_a_nonzero_mean(mean):
    """bf16, many segments (64 chunks per head, reverse aggregates scanned), V ~ N(mean, 1): every output row
    O_i is then close to every V_j, so the key-gradient weights (dO_i.V_j - O_i.dO_i)/den_i cancel strongly --
    in the chunk that holds both tokens and, through the reverse aggregates, across segments."""
    B, H, N, D, M = 1, 2, 64 * 64, 64, 64
    q, k, _ = _qkv(B, H, N, D, M, BF16, 9900, sigma=1.0 / 8.0)
    v = inputs.round_to_bf16(inputs.gaussian((B, H, N, M), 9902) + np.float32(mean))
    do = inputs.gaussian((B, H, N, M), 9903, 1.0, BF16)
    assert -(-N // binding.segment_length(B, H, N, D, M)) > 1
    check_forward(q, k, v, BF16)
    check_backward(q, k, v, do, BF16)


def test_single_segment_heads_sampled():
    """The sequence sweep's N = 2048 point: B=32 H=16 N=2048 D=M=64 bf16 (512 heads, so each head is one
    segment and the aggregate passes are skipped), inputs scaled by 1/8.  Forward and backward run on all
    heads; eight sampled heads are checked against the oracle (heads are independent)."""
    B, H, N, D, M = 32, 16, 2048, 64, 64
    assert binding.segment_length(B, H, N, D, M) == N
    q, k, v = _qkv(B, H, N, D, M, BF16, 9800, sigma=1.0 / 8.0)
    do = inputs.gaussian((B, H, N, M), 9803, 1.0, BF16)
    Q, K, V, dO = dev(q, BF16), dev(k, BF16), dev(v, BF16), dev(do, BF16)
    out = binding.forward_causal(Q, K, V)
    dq, dk, dv = binding.backward_causal(Q, K, V, out["o"], out["den"], dO, ckpt=out["ckpt"])
    torch.cuda.synchronize()
    o, den, dq, dk, dv = (host(t) for t in (out["o"], out["den"], dq, dk, dv))
    rng = np.random.default_rng(9804)
    for b, h in zip(rng.integers(0, B, 8), rng.integers(0, H, 8)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        qs, ks, vs, dos = q[sl], k[sl], v[sl], do[sl]
        ro, rden, _, _ = oracle.forward_causal(qs, ks, vs)
        rq, rk, rv = oracle.backward_causal(qs, ks, vs, dos)
        errs = {"O": rowerr(o[sl], ro), "den": rowerr(den[sl], rden, False), "dK": rowerr(dk[sl], rk),
                "dV": rowerr(dv[sl], rv),
                "dQ": rowerr(dq[sl], rq, row_floor=CANCEL_FLOOR * dq_cancel_scale(qs, ks, vs, dos))}
        assert max(errs.values()) <= TOL[BF16], (b, h, errs)


@pytest.mark.parametrize("layer", [0, 8])
def test_speech_workload_layer(layer):
    """B=16 H=6 N=800 D=M=32 float32: one layer of the 9-layer encoder as a training step runs it, the
    non-causal forward returning its totals and the backward taking them, every head."""
    w = inputs.SPEECH
    q, k, v = w.qkv(layer)
    do = w.grad_out(layer)
    o = binding.forward_noncausal(dev(q), dev(k), dev(v))
    torch.cuda.synchronize()
    assert rowerr(host(o), oracle.forward_noncausal(q, k, v)) <= 1e-4
    check_backward_noncausal(q, k, v, do, F32, totals=True)


def test_beyond_32bit_offsets_constant_values():
    """One head of 2^25 + 17 tokens at D = M = 64 bf16 (2^31 elements per tensor, so element offsets pass
    2^31) with every V row equal to one vector v: properties that hold at any size, since the attention
    weights of a row are positive and sum to one.  Causal and non-causal O equal v; the final state is
    S_N = Z_N v^T; dQ and dK vanish (O no longer depends on Q, K) up to rounding of the terms that cancel,
    bounded per row from cumulative sums of scalars: |dphiQ_i| <= |v| |dO_i| / min_d phi(Q_i)_d and
    |dphiK_j| <= sum_{i >= j} max_d phi(Q_i)_d |v| |dO_i| / den_i with den_i >= min_d phi(Q_i)_d sum_d Z_i,d;
    column sums of dV equal those of dO.  Inputs drawn on the GPU (seeded Philox), Q and K ~ N(0, 1/64)."""
    N, D, M = (1 << 25) + 17, 64, 64
    gen = torch.Generator(device="cuda")
    gen.manual_seed(9700)
    bf = torch.bfloat16
    q = (torch.randn((1, 1, N, D), generator=gen, device="cuda") / 8).to(bf)
    k = (torch.randn((1, 1, N, D), generator=gen, device="cuda") / 8).to(bf)
    v0 = torch.randn((M,), generator=gen, device="cuda").to(bf)
    v = v0.expand(1, 1, N, M).contiguous()
    do = torch.randn((1, 1, N, M), generator=gen, device="cuda").to(bf)
    out = binding.forward_causal(q, k, v, return_state=True)
    o_nc = binding.forward_noncausal(q, k, v)
    dq, dk, dv = binding.backward_causal(q, k, v, out["o"], out["den"], do, ckpt=out["ckpt"])
    torch.cuda.synchronize()
    vf = v0.double()
    vn = vf.norm()

    def chunks(n=1 << 22):
        return [(a, min(N, a + n)) for a in range(0, N, n)]

    err_o = err_nc = 0.0
    for a, b in chunks():
        err_o = max(err_o, float((out["o"][0, 0, a:b].double() - vf).abs().max()))
        err_nc = max(err_nc, float((o_nc[0, 0, a:b].double() - vf).abs().max()))
    assert max(err_o, err_nc) <= 2e-2 * float(vf.abs().max()), (err_o, err_nc)
    s_n, z_n = out["s"][0, 0].double(), out["z"][0, 0].double()
    assert float((s_n - torch.outer(z_n, vf)).abs().max()) <= 2e-2 * float(s_n.abs().max())
    # per-token scalars for the bounds, float64
    pq_min = torch.empty(N, dtype=torch.float64, device="cuda")
    pq_max = torch.empty_like(pq_min)
    pk_sum = torch.empty_like(pq_min)
    don = torch.empty_like(pq_min)
    phi = lambda x: torch.where(x > 0, x + 1, torch.exp(x))  # noqa: E731
    for a, b in chunks():
        pq = phi(q[0, 0, a:b].double())
        pq_min[a:b], pq_max[a:b] = pq.min(-1).values, pq.max(-1).values
        pk_sum[a:b] = phi(k[0, 0, a:b].double()).sum(-1)
        don[a:b] = do[0, 0, a:b].double().norm(dim=-1)
    tq = vn * don / pq_min
    den_lb = pq_min * torch.cumsum(pk_sum, 0)
    tk = torch.flip(torch.cumsum(torch.flip(pq_max * vn * don / den_lb, [0]), 0), [0])
    rq = rk = 0.0
    for a, b in chunks():
        rq = max(rq, float((dq[0, 0, a:b].double().abs().max(-1).values / tq[a:b]).max()))
        rk = max(rk, float((dk[0, 0, a:b].double().abs().max(-1).values / tk[a:b]).max()))
    assert rq <= 1e-3 and rk <= 1e-3, (rq, rk)
    sdv = torch.zeros(M, dtype=torch.float64, device="cuda")
    sdo, sdo_abs = torch.zeros_like(sdv), torch.zeros_like(sdv)
    for a, b in chunks():
        sdv += dv[0, 0, a:b].double().sum(0)
        x = do[0, 0, a:b].double()
        sdo += x.sum(0)
        sdo_abs += x.abs().sum(0)
    assert float(((sdv - sdo).abs() / sdo_abs).max()) <= 2e-2


def test_decode_graph_replay():
    """Decode steps captured in a HIP graph, as a serving loop runs them, then replayed three times with eager
    work and synchronisations between the replays: every replay equals the eager launches bit for bit (y of
    every step, the final S and Z)."""
    B, H, D, M, P, T = 4, 3, 64, 64, 100, 12
    q, k, v = _qkv(B, H, P, D, M, BF16, 9600)
    out = gpu_forward(q, k, v, BF16)
    s0, z0 = out["s"].clone(), out["z"].clone()
    steps = [tuple(dev(inputs.gaussian(shape, 9610 + 3 * t + i, 1.0, BF16), BF16)
                   for i, shape in enumerate(((B, H, D), (B, H, D), (B, H, M)))) for t in range(T)]
    se, ze = s0.clone(), z0.clone()
    ye = torch.empty((T, B, H, M), dtype=torch.bfloat16, device="cuda")
    for t, (qt, kt, vt) in enumerate(steps):
        binding.la_decode_step(qt, kt, vt, se, ze, ye[t])
    torch.cuda.synchronize()
    sg, zg = s0.clone(), z0.clone()
    yg = torch.empty_like(ye)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for t, (qt, kt, vt) in enumerate(steps):
            binding.la_decode_step(qt, kt, vt, sg, zg, yg[t])
    torch.cuda.synchronize()
    for rep in range(3):
        sg.copy_(s0)
        zg.copy_(z0)
        yg.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(yg, ye), f"replay {rep}: y differs"
        assert torch.equal(sg, se) and torch.equal(zg, ze), f"replay {rep}: state differs"
        (torch.randn(1000, device="cuda") * 2).sum().item()  # unrelated eager work between replays


def test_decode_state_saved_to_host_and_restored():
    """Checkpoint and resume of a decode loop: after a prefill and 40 steps the state (S, Z) is copied to host
    memory and back into fresh device buffers; the next 40 steps from the restored state equal, bit for bit,
    those of the loop that kept its state on the device (the state is the whole carried context, eq. 16-19)."""
    B, H, D, M, P, T = 8, 4, 64, 32, 300, 80
    q, k, v = _qkv(B, H, P, D, M, BF16, 9700)
    out = gpu_forward(q, k, v, BF16)
    steps = [tuple(dev(inputs.gaussian(shape, 9710 + 3 * t + i, 1.0, BF16), BF16)
                   for i, shape in enumerate(((B, H, D), (B, H, D), (B, H, M)))) for t in range(T)]
    s, z = out["s"].clone(), out["z"].clone()
    ys = [binding.decode_step(*steps[t], s, z) for t in range(T)]
    torch.cuda.synchronize()
    s2, z2 = out["s"].clone(), out["z"].clone()
    for t in range(T // 2):
        binding.decode_step(*steps[t], s2, z2)
    torch.cuda.synchronize()
    saved = (s2.cpu().numpy().copy(), z2.cpu().numpy().copy())  # host copy, device buffers dropped
    del s2, z2
    s3, z3 = torch.from_numpy(saved[0]).to("cuda"), torch.from_numpy(saved[1]).to("cuda")
    for t in range(T // 2, T):
        y = binding.decode_step(*steps[t], s3, z3)
        assert torch.equal(y, ys[t]), t
    torch.cuda.synchronize()
    assert torch.equal(s3, s) and torch.equal(z3, z)


def test_decode_workload_sampled():
    """Batch 256, 16 heads, D=M=64, bf16 I/O: the 512-token prefill then all 4096 decode steps of the workload,
    on the per-step inputs the benchmark times (seeds 5,000,000 + 3 step + {0, 1, 2}); every step's y and the
    final state are checked on 32 sampled heads (the oracle follows those heads only: eq. 16-19 continued from
    the prefill's state, which equals decode steps from it)."""
    from concurrent.futures import ThreadPoolExecutor

    w = inputs.DECODE
    steps = w.steps
    B, H, D, M = w.B, w.H, w.D, w.M
    q, k, v = w.qkv()
    out = gpu_forward(q, k, v, BF16)
    s, z = out["s"], out["z"]
    rng = np.random.Generator(np.random.PCG64(77))
    flat = np.sort(rng.choice(B * H, size=32, replace=False))
    bi, hi = flat // H, flat % H
    _, _, so, zo = oracle.forward_causal(q[bi, hi][None], k[bi, hi][None], v[bi, hi][None])
    assert rowerr(host(s)[bi, hi][None], so) <= 1e-4
    ys = torch.empty((steps, len(flat), M), device="cuda", dtype=torch.bfloat16)
    idx_b = torch.from_numpy(bi).cuda()
    idx_h = torch.from_numpy(hi).cuda()
    qs, ks, vs = [], [], []
    widen = lambda a: (a.astype(np.uint32) << np.uint32(16)).view(np.float32)  # noqa: E731
    chunk = 256
    with ThreadPoolExecutor(16) as ex:
        for t0 in range(0, steps, chunk):
            trip = list(ex.map(w.decode_step_bits, range(t0, min(steps, t0 + chunk))))
            for j, (qt, kt, vt) in enumerate(trip):
                qd, kd, vd = (torch.from_numpy(a).view(torch.bfloat16).to("cuda") for a in (qt, kt, vt))
                y = binding.decode_step(qd, kd, vd, s, z)
                ys[t0 + j] = y[idx_b, idx_h]
                qs.append(widen(qt[bi, hi]))
                ks.append(widen(kt[bi, hi]))
                vs.append(widen(vt[bi, hi]))
            torch.cuda.synchronize()
    qn, kn, vn = (np.stack(a, axis=1)[None] for a in (qs, ks, vs))  # [1, 32, steps, D]
    yo, _, sn, zn = oracle.forward_causal(qn, kn, vn, so, zo)
    assert rowerr(host(ys).transpose(1, 0, 2)[None], yo) <= 2e-2
    assert rowerr(host(s)[bi, hi][None], sn) <= 1e-4
    assert rowerr(host(z)[bi, hi][None], zn, False) <= 1e-4


# ------------------------------------------------ non-causal backward
def nc_cancel_scales(q, k, v, do):
    """Per-row sizes of the terms the non-causal gradients cancel: |S g_i * phi'(Q_i)|_inf for dQ and
    |R V_j * phi'(K_j)|_inf for dK (S, R the totals of the reading notes' eq. 5-6 and its reverse sum)."""
    pq, pk = pins.phi_lib(q), pins.phi_lib(k)
    v64, do64 = v.astype(np.float64), do.astype(np.float64)
    S = np.einsum("bhnd,bhnm->bhdm", pk, v64)
    den = np.einsum("bhnd,bhd->bhn", pq, pk.sum(axis=2))
    g = do64 / den[..., None]
    R = np.einsum("bhnd,bhnm->bhdm", pq, g)
    uq = np.einsum("bhdm,bhnm->bhnd", S, g) * np.minimum(pq, 1.0)
    uk = np.einsum("bhdm,bhnm->bhnd", R, v64) * np.minimum(pk, 1.0)
    return np.abs(uq).max(-1), np.abs(uk).max(-1)


def check_backward_noncausal(q, k, v, do, dtype, tol=None, totals=False, opts=None):
    tol = TOL[dtype] if tol is None else tol
    Q, K, V = dev(q, dtype), dev(k, dtype), dev(v, dtype)
    s = z = None
    if totals:  # the forward's totals, checked against the plain sums, passed on to the backward
        _, s, z = binding.forward_noncausal(Q, K, V, return_state=True, opts=opts)
        torch.cuda.synchronize()
        _, _, rs, rz = oracle.forward_causal(q, k, v)
        assert max(rowerr(host(s), rs), rowerr(host(z), rz, False)) <= tol
    dq, dk, dv = binding.backward_noncausal(Q, K, V, dev(do, dtype), s=s, z=z, opts=opts)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.backward_noncausal(q, k, v, do)
    dq, dk, dv = host(dq), host(dk), host(dv)
    sq, sk = nc_cancel_scales(q, k, v, do)
    if q.shape[2] == 1:
        # N = 1: O_1 = V_1, so dQ_1 and dK_1 are exact zeros.  The library forms them through the totals
        # S = phi(K) V^T and R = phi(Q) g^T, whose elements are rounded before the products with g and V,
        # so the attainable error is the dot-product bound sum_m |S_dm| |g_m| (resp. |R_dm| |V_m|), not the
        # size of the (possibly cancelling) dot product itself.  The bar is the one the causal first-token
        # query gradient meets: a residual below kappa of that bound.
        kappa = {F32: 1e-5, BF16: 1e-3}[dtype]
        pq, pk = pins.phi_lib(q[:, :, 0]), pins.phi_lib(k[:, :, 0])
        v1, do1 = v[:, :, 0].astype(np.float64), do[:, :, 0].astype(np.float64)
        den = (pq * pk).sum(-1, keepdims=True)
        bq = (pk * (np.abs(v1) * np.abs(do1)).sum(-1, keepdims=True) / den * np.minimum(pq, 1.0)).max(-1)
        bk = (pq * (np.abs(do1) * np.abs(v1)).sum(-1, keepdims=True) / den * np.minimum(pk, 1.0)).max(-1)
        errs = {"dQ": float((np.abs(dq[:, :, 0]).max(-1) / bq).max()) * tol / kappa,
                "dK": float((np.abs(dk[:, :, 0]).max(-1) / bk).max()) * tol / kappa,
                "dV": rowerr(dv, rv)}
    else:
        errs = {"dQ": rowerr(dq, rq, row_floor=CANCEL_FLOOR * sq), "dK": rowerr(dk, rk, row_floor=CANCEL_FLOOR * sk),
                "dV": rowerr(dv, rv)}
    assert max(errs.values()) <= tol, errs
    return dq, dk, dv


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("D,M", DM)
@pytest.mark.parametrize("N", [1, 2, 17, 64, 65, 200, 784])
def test_backward_noncausal_sweep(N, D, M, dtype):
    q, k, v = _qkv(2, 3, N, D, M, dtype, 9000 + N)
    do = inputs.gaussian((2, 3, N, M), 9999, 1.0, dtype)
    check_backward_noncausal(q, k, v, do, dtype)


@pytest.mark.parametrize("chunks", [1, 3])
def test_backward_noncausal_segment_invariance(chunks):
    """Segment lengths change only the summation order of the totals."""
    q, k, v = _qkv(2, 2, 700, 64, 32, F32, 9100)
    do = inputs.gaussian((2, 2, 700, 32), 9104, 1.0, F32)
    check_backward_noncausal(q, k, v, do, F32, opts=binding.options(segment_chunks=chunks))


def test_backward_noncausal_mnist_shape():
    """B=16 H=8 N=784 D=M=32 float32 (the MNIST-shaped layer, non-causal), every head."""
    w = inputs.MNIST
    q, k, v = w.qkv()
    check_backward_noncausal(q, k, v, w.grad_out(), F32)


def test_backward_noncausal_long_shape_sampled():
    """B=1 H=16 N=65536 D=M=64 bf16: the whole problem on the GPU, the oracle on two heads."""
    w = inputs.LONG
    q, k, v = w.qkv()
    do = w.grad_out()
    dq, dk, dv = binding.backward_noncausal(dev(q, BF16), dev(k, BF16), dev(v, BF16), dev(do, BF16))
    torch.cuda.synchronize()
    hs = [0, 11]
    sub = lambda a: a[:, hs]  # noqa: E731
    rq, rk, rv = oracle.backward_noncausal(sub(q), sub(k), sub(v), sub(do))
    sq, sk = nc_cancel_scales(sub(q), sub(k), sub(v), sub(do))
    errs = {"dQ": rowerr(sub(host(dq)), rq, row_floor=CANCEL_FLOOR * sq),
            "dK": rowerr(sub(host(dk)), rk, row_floor=CANCEL_FLOOR * sk), "dV": rowerr(sub(host(dv)), rv)}
    assert max(errs.values()) <= TOL[BF16], errs


def test_noncausal_autograd_wrapper():
    """torch.autograd through the library's non-causal forward and backward equals the oracle."""
    q, k, v = _qkv(2, 2, 150, 32, 64, F32, 9200)
    do = inputs.gaussian((2, 2, 150, 64), 9204, 1.0, F32)
    Q, K, V = (dev(a).requires_grad_(True) for a in (q, k, v))
    out = binding.noncausal_linear_attention(Q, K, V)
    out.backward(dev(do))
    torch.cuda.synchronize()
    rq, rk, rv = oracle.backward_noncausal(q, k, v, do)
    sq, sk = nc_cancel_scales(q, k, v, do)
    errs = [rowerr(host(Q.grad), rq, row_floor=CANCEL_FLOOR * sq), rowerr(host(K.grad), rk, row_floor=CANCEL_FLOOR * sk),
            rowerr(host(V.grad), rv), rowerr(host(out), oracle.forward_noncausal(q, k, v))]
    assert max(errs) <= 1e-4, errs


# ------------------------------------------------------- state gradients
def _state_inputs(B, H, D, M, dtype, seed, sigma=0.1):
    """A realistic initial state (the final state of a 50-token prefix) and final-state gradients."""
    _, _, s0, z0 = oracle.forward_causal(*_qkv(B, H, 50, D, M, dtype, seed))
    s0, z0 = (a.astype(np.float32).astype(np.float64) for a in (s0, z0))  # what the library receives
    dsn = inputs.gaussian((B, H, D, M), seed + 10, sigma)
    dzn = inputs.gaussian((B, H, D), seed + 11, sigma)
    return s0, z0, dsn, dzn


def gpu_backward_state(q, k, v, do, dtype, s0, z0, dsn, dzn, use_ckpt=True, opts=None):
    out = gpu_forward(q, k, v, dtype, s0, z0, opts)
    Q, K, V = dev(q, dtype), dev(k, dtype), dev(v, dtype)
    g = binding.backward_causal(Q, K, V, out["o"], out["den"], dev(do, dtype),
                                s0=None if s0 is None else dev32(s0), z0=None if z0 is None else dev32(z0),
                                ckpt=out["ckpt"] if use_ckpt else None,
                                ds_n=None if dsn is None else dev32(dsn), dz_n=None if dzn is None else dev32(dzn),
                                state_grad=True, opts=opts)
    torch.cuda.synchronize()
    return [host(t) for t in g]


def state_grad_errors(got, q, k, v, do, s0, z0, dsn, dzn):
    dq, dk, dv, ds0, dz0 = got
    rq, rk, rv, rs, rz = oracle.backward_causal(q, k, v, do, s0, z0, dsn, dzn, state_grad=True)
    return {"dQ": rowerr(dq, rq, row_floor=CANCEL_FLOOR * dq_cancel_scale(q, k, v, do, s0, z0)),
            "dK": rowerr(dk, rk), "dV": rowerr(dv, rv), "dS0": rowerr(ds0, rs),
            # dZ0 = dZ_N + sum_i c_i phi(Q_i) is a signed sum, one D-vector per head like a row of dK
            "dZ0": rowerr(dz0[:, :, None, :], rz[:, :, None, :])}


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("D,M", DM)
@pytest.mark.parametrize("N", [1, 64, 65, 200, 784])
def test_state_gradient_sweep(N, D, M, dtype):
    """Gradients with an initial state and a final-state gradient: dQ, dK, dV and dS0, dZ0."""
    B, H = 2, 3
    q, k, v = _qkv(B, H, N, D, M, dtype, 9300 + N)
    do = inputs.gaussian((B, H, N, M), 9390, 1.0, dtype)
    s0, z0, dsn, dzn = _state_inputs(B, H, D, M, dtype, 9400)
    got = gpu_backward_state(q, k, v, do, dtype, s0, z0, dsn, dzn)
    errs = state_grad_errors(got, q, k, v, do, s0, z0, dsn, dzn)
    assert max(errs.values()) <= TOL[dtype], errs


@pytest.mark.parametrize("D,M", [(32, 32), (64, 64)])
@pytest.mark.parametrize("chunks", [1, 3])
@pytest.mark.parametrize("use_ckpt", [True, False])
def test_state_gradient_segments(D, M, chunks, use_ckpt):
    """Many segments (reverse aggregates summed in the workgroup for D=M=32, scanned for 64) with the
    final-state gradient added to every segment's start; initial-state gradient from the first segment."""
    B, H, N = 1, 2, 784
    q, k, v = _qkv(B, H, N, D, M, F32, 9500 + chunks)
    do = inputs.gaussian((B, H, N, M), 9590)
    s0, z0, dsn, dzn = _state_inputs(B, H, D, M, F32, 9600)
    got = gpu_backward_state(q, k, v, do, F32, s0, z0, dsn, dzn, use_ckpt, binding.options(segment_chunks=chunks))
    errs = state_grad_errors(got, q, k, v, do, s0, z0, dsn, dzn)
    assert max(errs.values()) <= TOL[F32], errs


def test_state_gradient_without_initial_state():
    """No S0, Z0 (zero initial state): dS0, dZ0 are still the gradient with respect to it."""
    B, H, N, D, M = 2, 2, 300, 64, 32
    q, k, v = _qkv(B, H, N, D, M, BF16, 9700)
    do = inputs.gaussian((B, H, N, M), 9703, 1.0, BF16)
    _, _, dsn, dzn = _state_inputs(B, H, D, M, BF16, 9710)
    got = gpu_backward_state(q, k, v, do, BF16, None, None, dsn, dzn)
    errs = state_grad_errors(got, q, k, v, do, None, None, dsn, dzn)
    assert max(errs.values()) <= TOL[BF16], errs
    # and without a final-state gradient the initial-state gradient is the reverse sum alone
    got = gpu_backward_state(q, k, v, do, BF16, None, None, None, None)
    errs = state_grad_errors(got, q, k, v, do, None, None, None, None)
    assert max(errs.values()) <= TOL[BF16], errs


def test_state_gradient_empty_sequence():
    """N = 0: dS0, dZ0 receive dS_N, dZ_N unchanged (zeros when absent)."""
    B, H, D, M = 2, 3, 32, 64
    e = torch.empty((B, H, 0, D), device="cuda")
    ev = torch.empty((B, H, 0, M), device="cuda")
    dsn = dev32(inputs.gaussian((B, H, D, M), 9800))
    dzn = dev32(inputs.gaussian((B, H, D), 9801))
    ds0 = torch.full((B, H, D, M), 7.0, device="cuda")
    dz0 = torch.full((B, H, D), 7.0, device="cuda")
    binding.la_backward_causal(e, e, ev, ev, None, ev, e, e, ev, dS_N=dsn, dZ_N=dzn, dS0=ds0, dZ0=dz0)
    torch.cuda.synchronize()
    assert torch.equal(ds0, dsn) and torch.equal(dz0, dzn)
    binding.la_backward_causal(e, e, ev, ev, None, ev, e, e, ev, dS0=ds0, dZ0=dz0)
    torch.cuda.synchronize()
    assert not torch.any(ds0) and not torch.any(dz0)


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_state_gradient_chains_across_a_split(dtype):
    """A sequence cut in two: the second part's backward (with the final-state gradient) gives dS0, dZ0 that,
    as the first part's final-state gradient, reproduce the whole sequence's gradients."""
    B, H, N, D, M, cut = 2, 2, 700, 64, 64, 300
    q, k, v = _qkv(B, H, N, D, M, dtype, 9900)
    do = inputs.gaussian((B, H, N, M), 9903, 1.0, dtype)
    s0, z0, dsn, dzn = _state_inputs(B, H, D, M, dtype, 9910)
    _, _, s_mid, z_mid = oracle.forward_causal(q[:, :, :cut], k[:, :, :cut], v[:, :, :cut], s0, z0)
    sl2, sl1 = slice(cut, None), slice(None, cut)
    g2 = gpu_backward_state(q[:, :, sl2], k[:, :, sl2], v[:, :, sl2], do[:, :, sl2], dtype, s_mid, z_mid, dsn, dzn)
    g1 = gpu_backward_state(q[:, :, sl1], k[:, :, sl1], v[:, :, sl1], do[:, :, sl1], dtype, s0, z0, g2[3], g2[4])
    got = [np.concatenate((a, b), 2) for a, b in zip(g1[:3], g2[:3])] + g1[3:]
    errs = state_grad_errors(got, q, k, v, do, s0, z0, dsn, dzn)
    assert max(errs.values()) <= TOL[dtype], errs


def test_state_gradient_autograd_wrapper():
    """torch.autograd through the library with an initial state and the final state in the loss."""
    B, H, N, D, M = 2, 2, 260, 32, 32
    q, k, v = _qkv(B, H, N, D, M, F32, 9950)
    do = inputs.gaussian((B, H, N, M), 9953)
    s0, z0, dsn, dzn = _state_inputs(B, H, D, M, F32, 9960)
    Q, K, V, S0, Z0 = (dev32(a).requires_grad_(True) for a in (q, k, v, s0, z0))
    o, s, z = binding.causal_linear_attention(Q, K, V, S0, Z0, return_state=True)
    ((o * dev32(do)).sum() + (s * dev32(dsn)).sum() + (z * dev32(dzn)).sum()).backward()
    torch.cuda.synchronize()
    got = [host(t.grad) for t in (Q, K, V, S0, Z0)]
    errs = state_grad_errors(got, q, k, v, do, s0, z0, dsn, dzn)
    assert max(errs.values()) <= TOL[F32], errs


def test_state_gradient_long_shape_sampled():
    """B=1 H=16 N=65536 D=M=64 bf16 with an initial state and a final-state gradient; the oracle follows
    heads 0 and 11."""
    w = inputs.LONG
    q, k, v = w.qkv()
    do = w.grad_out()
    s0, z0, dsn, dzn = _state_inputs(w.B, w.H, w.D, w.M, BF16, 9990)
    got = gpu_backward_state(q, k, v, do, BF16, s0, z0, dsn, dzn)
    hs = [0, 11]
    sub = lambda a: a[:, hs]  # noqa: E731
    errs = state_grad_errors([sub(a) for a in got], sub(q), sub(k), sub(v), sub(do), sub(s0), sub(z0), sub(dsn),
                             sub(dzn))
    assert max(errs.values()) <= TOL[BF16], errs


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("D,M", DM)
@pytest.mark.parametrize("N", [1, 65, 784])
def test_backward_noncausal_with_forward_totals(N, D, M, dtype):
    """The non-causal forward's totals (S, Z) handed to the backward in place of forming them again."""
    q, k, v = _qkv(2, 3, N, D, M, dtype, 15000 + N)
    do = inputs.gaussian((2, 3, N, M), 15099, 1.0, dtype)
    check_backward_noncausal(q, k, v, do, dtype, totals=True)


def test_noncausal_totals_of_empty_sequence():
    s = torch.full((2, 2, 32, 64), 3.0, device="cuda")
    z = torch.full((2, 2, 32), 3.0, device="cuda")
    e, ev = torch.empty((2, 2, 0, 32), device="cuda"), torch.empty((2, 2, 0, 64), device="cuda")
    binding.la_forward_noncausal(e, e, ev, ev, S_out=s, Z_out=z)
    torch.cuda.synchronize()
    assert not torch.any(s) and not torch.any(z)
