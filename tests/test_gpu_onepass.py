"""GPU parity of the one-pass causal forward (segments of at most four chunks
whose aggregates every workgroup sums itself) against the float64 oracle and
against the two-launch form (aggregate pass, then the forward).

The one-pass form defers each segment's carry: a workgroup walks its segment
from a zero state, publishes the segment aggregate behind a flag, and adds
phi(Q).(sum of the earlier aggregates) to its numerators and denominators at
the end.  These tests run it on ragged sequences over one to four chunks per
segment, with and without an initial state, check the checkpoint entries it
writes (the states at the segment starts, eq. 10-11 summed over the earlier
tokens) and that a backward from its checkpoint is unchanged, and call it
twice on one workspace pre-filled with non-zero bytes (the flags must be
cleared by the call itself).
"""
import numpy as np
import pytest
import torch

import oracle
from linear_rnn_layers_amd import binding, inputs
from tests.gpu_util import TOL, dev, dev32, host, rowerr

pytestmark = pytest.mark.gpu

F32, BF16 = inputs.F32, inputs.BF16
DM = [(32, 32), (64, 64), (32, 64), (64, 32)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "the GPU tests need a GPU"
    binding.load()
    binding.set_segment_chunks(0)
    binding.set_forward_onepass(2)
    yield
    binding.set_segment_chunks(0)
    binding.set_forward_onepass(1)


def _qkv(B, H, N, D, M, dtype, seed, sigma=1.0):
    q = inputs.gaussian((B, H, N, D), seed, sigma, dtype)
    k = inputs.gaussian((B, H, N, D), seed + 1, sigma, dtype)
    v = inputs.gaussian((B, H, N, M), seed + 2, sigma, dtype)
    return q, k, v


def _run(q, k, v, dtype, s0=None, z0=None, onepass=True):
    """Forward with checkpoint and final state; returns the outputs and whether the one-pass form ran."""
    prev = binding.set_forward_onepass(2 if onepass else 0)
    binding.prof_select("sync_clear")
    try:
        out = binding.forward_causal(dev(q, dtype), dev(k, dtype), dev(v, dtype),
                                     s0=None if s0 is None else dev32(s0), z0=None if z0 is None else dev32(z0),
                                     return_state=True, checkpoint=True)
        _, launches, _ = binding.prof_collect()
    finally:
        binding.prof_select(None)
        binding.set_forward_onepass(prev)
    return out, launches > 0


def _ckpt_ref(q, k, v, L, s0=None, z0=None):
    """Oracle states at the segment starts 0, L, 2L, ... and at N: [B, H, nseg + 1, D*M + D]."""
    B, H, N, D = q.shape
    M = v.shape[-1]
    starts = list(range(0, N, L)) + [N]
    ref = np.zeros((B, H, len(starts), D * M + D))
    for e, t in enumerate(starts):
        if t == 0:
            s = np.zeros((B, H, D, M)) if s0 is None else s0
            z = np.zeros((B, H, D)) if z0 is None else z0
        else:
            _, _, s, z = oracle.forward_causal(q[:, :, :t], k[:, :, :t], v[:, :, :t], s0, z0)
        ref[:, :, e, :D * M] = np.asarray(s, dtype=np.float64).reshape(B, H, D * M)
        ref[:, :, e, D * M:] = z
    return ref


def _error_word(ws, B, H, N, D, M):
    """Word 0 of the one-launch forward's flag region: after the aggregates and the prefix states of the workspace."""
    L = binding.segment_length(B, H, N, D, M)
    nseg, sv = -(-N // L), D * M + D
    off = sum((x + 255) // 256 * 256 for x in (B * H * nseg * sv * 4, B * H * (nseg + 1) * sv * 4))
    return int(ws[off:off + 4].view(torch.int32).item())


def _check(out, q, k, v, dtype, s0=None, z0=None):
    o, den, s, z = oracle.forward_causal(q, k, v, s0, z0)
    errs = {"O": rowerr(host(out["o"]), o), "den": rowerr(host(out["den"]), den, False),
            "S_N": rowerr(host(out["s"]), s), "Z_N": rowerr(host(out["z"]), z, False)}
    assert max(errs.values()) <= TOL[dtype], errs


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("D,M", DM)
@pytest.mark.parametrize("chunks", [1, 2, 3, 4])
def test_onepass_segments(chunks, D, M, dtype):
    """One to four chunks per segment, ragged last segment: outputs, final state and checkpoint entries."""
    B, H = 2, 2
    N = 3 * 64 * chunks + 37 if D * M <= 1024 else 64 * chunks + 29  # few enough aggregates to sum per workgroup
    q, k, v = _qkv(B, H, N, D, M, dtype, 7000 + 10 * chunks + D + M)
    prev = binding.set_segment_chunks(chunks)
    try:
        out, onepass = _run(q, k, v, dtype)
        L = binding.segment_length(B, H, N, D, M)
    finally:
        binding.set_segment_chunks(prev)
    assert onepass, "the one-pass forward did not run"
    assert L == 64 * chunks
    _check(out, q, k, v, dtype)
    nseg = -(-N // L)
    ck = host(out["ckpt"]).reshape(B, H, nseg + 1, D * M + D)
    ref = _ckpt_ref(q, k, v, L)
    assert rowerr(ck[:, :, 1:, :D * M].reshape(B, H, -1, M), ref[:, :, 1:, :D * M].reshape(B, H, -1, M)) <= TOL[dtype]
    assert rowerr(ck[:, :, 1:, D * M:], ref[:, :, 1:, D * M:]) <= TOL[dtype]
    assert np.all(ck[:, :, 0] == 0.0)


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_onepass_initial_state(dtype):
    """The carry of every segment starts from (S0, Z0), so the first segment's rows see it too."""
    B, H, N, D, M = 2, 3, 500, 32, 64
    q, k, v = _qkv(B, H, N + 90, D, M, dtype, 7500)
    _, _, s0, z0 = oracle.forward_causal(q[:, :, :90], k[:, :, :90], v[:, :, :90])
    q, k, v = q[:, :, 90:], k[:, :, 90:], v[:, :, 90:]
    prev = binding.set_segment_chunks(2)
    try:
        out, onepass = _run(q, k, v, dtype, s0, z0)
    finally:
        binding.set_segment_chunks(prev)
    assert onepass
    _check(out, q, k, v, dtype, s0, z0)


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_onepass_matches_two_launch_form(dtype):
    """Both forms of the forward agree within the tolerance, and the backward from either checkpoint matches."""
    B, H, N, D, M = 4, 4, 784, 32, 32
    q, k, v = _qkv(B, H, N, D, M, dtype, 7600)
    do = inputs.gaussian((B, H, N, M), 7604, 1.0, dtype)
    a, ra = _run(q, k, v, dtype, onepass=True)
    b, rb = _run(q, k, v, dtype, onepass=False)
    assert ra and not rb
    for key in ("o", "s"):
        assert rowerr(host(a[key]), host(b[key])) <= TOL[dtype], key
    for key in ("den", "z"):
        assert rowerr(host(a[key]), host(b[key]), False) <= TOL[dtype], key
    Q, K, V, dO = dev(q, dtype), dev(k, dtype), dev(v, dtype), dev(do, dtype)
    ga = binding.backward_causal(Q, K, V, a["o"], a["den"], dO, ckpt=a["ckpt"])
    gb = binding.backward_causal(Q, K, V, b["o"], b["den"], dO, ckpt=b["ckpt"])
    torch.cuda.synchronize()
    rq, rk, rv = oracle.backward_causal(q, k, v, do)
    for x, y, r in zip(ga, gb, (rq, rk, rv)):
        # dQ of the first token is an exact cancellation (zero): rows are judged against the tensor's scale
        assert rowerr(host(x), host(y), row_floor=np.full(r.shape[:-1], 1e-3 * np.abs(r).max())) <= TOL[dtype]


def test_onepass_rule():
    """By default the one-launch form runs for states of D*M >= 2048 and the two-launch form below that."""
    prev = binding.set_forward_onepass(1)
    try:
        for (D, M), want in (((32, 32), False), ((64, 32), True), ((64, 64), True)):
            q, k, v = _qkv(2, 2, 300, D, M, F32, 7900)
            binding.prof_select("sync_clear")
            binding.forward_causal(dev(q), dev(k), dev(v))
            _, launches, _ = binding.prof_collect()
            binding.prof_select(None)
            assert (launches > 0) == want, (D, M)
    finally:
        binding.set_forward_onepass(prev)


def test_onepass_reused_dirty_workspace():
    """Two calls on one workspace that starts filled with 0xff bytes: the call clears its own flags."""
    B, H, N, D, M = 8, 8, 784, 32, 32
    q, k, v = _qkv(B, H, N, D, M, F32, 7700)
    Q, K, V = dev(q), dev(k), dev(v)
    ws = binding.alloc_workspace(binding.LA_OP_FWD_CAUSAL, B, H, N, D, M, binding.dtype_code(torch.float32), "cuda")
    ws.fill_(255)
    ref = oracle.forward_causal(q, k, v)
    binding.prof_select("sync_clear")
    assert binding.segment_length(B, H, N, D, M) <= 4 * 64
    for _ in range(2):
        O = torch.empty((B, H, N, M), device="cuda")
        den = torch.empty((B, H, N), device="cuda")
        binding.la_forward_causal(Q, K, V, O, den, ws=ws)
        torch.cuda.synchronize()
        assert _error_word(ws, B, H, N, D, M) == 0  # no wait gave up
        assert rowerr(host(O), ref[0]) <= 1e-4
        assert rowerr(host(den), ref[1], False) <= 1e-4
    _, launches, _ = binding.prof_collect()
    binding.prof_select(None)
    assert launches == 2


def test_onepass_wait_limit():
    """With the poll limit at 0 every wait gives up at once (forced from the host: no wave spins): the first segment
    of each head needs no carry and stays exact, later segments' rows and the final state are NaN, the error word
    is set; the next call at the normal limit is exact again."""
    B, H, N, D, M = 2, 3, 5 * 64 + 11, 32, 32
    q, k, v = _qkv(B, H, N, D, M, F32, 7950)
    Q, K, V = dev(q), dev(k), dev(v)
    o_ref, den_ref, _, _ = oracle.forward_causal(q, k, v)
    prev_c = binding.set_segment_chunks(2)
    try:
        L = binding.segment_length(B, H, N, D, M)
        ws = binding.alloc_workspace(binding.LA_OP_FWD_CAUSAL, B, H, N, D, M, binding.dtype_code(torch.float32),
                                     "cuda")
        for polls in (0, 1 << 22):
            prev_p = binding.set_wait_polls(polls)
            try:
                O = torch.empty((B, H, N, M), device="cuda")
                den = torch.empty((B, H, N), device="cuda")
                S = torch.empty((B, H, D, M), device="cuda")
                Z = torch.empty((B, H, D), device="cuda")
                binding.la_forward_causal(Q, K, V, O, den, S_out=S, Z_out=Z, ws=ws)
                torch.cuda.synchronize()
            finally:
                binding.set_wait_polls(prev_p)
            o, d = host(O), host(den)
            if polls == 0:
                assert _error_word(ws, B, H, N, D, M) == 1
                assert rowerr(o[:, :, :L], o_ref[:, :, :L]) <= 1e-4
                assert rowerr(d[:, :, :L], den_ref[:, :, :L], False) <= 1e-4
                assert np.isnan(o[:, :, L:]).all() and np.isnan(d[:, :, L:]).all()
                assert np.isnan(host(S)).all() and np.isnan(host(Z)).all()
            else:
                assert _error_word(ws, B, H, N, D, M) == 0
                assert rowerr(o, o_ref) <= 1e-4
                assert rowerr(d, den_ref, False) <= 1e-4
    finally:
        binding.set_segment_chunks(prev_c)


def test_onepass_many_heads_full_shape():
    """The MNIST-shaped layer (B=16 H=8 N=784 D=M=32 float32): rows sampled from every head."""
    B, H, N, D, M = 16, 8, 784, 32, 32
    q, k, v = _qkv(B, H, N, D, M, F32, 7800)
    out, onepass = _run(q, k, v, F32)
    assert onepass
    o = host(out["o"])
    den = host(out["den"])
    rng = np.random.default_rng(7801)
    for b in range(B):
        for h in range(H):
            rows = np.unique(np.concatenate([rng.integers(0, N, 6), [0, 127, 128, N - 1]]))
            ro, rd, _, _ = oracle.forward_causal(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1])
            assert rowerr(o[b:b + 1, h:h + 1, rows], ro[:, :, rows]) <= 1e-4
            assert rowerr(den[b:b + 1, h:h + 1, rows], rd[:, :, rows], False) <= 1e-4
