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
    yield


def _qkv(B, H, N, D, M, dtype, seed, sigma=1.0):
    q = inputs.gaussian((B, H, N, D), seed, sigma, dtype)
    k = inputs.gaussian((B, H, N, D), seed + 1, sigma, dtype)
    v = inputs.gaussian((B, H, N, M), seed + 2, sigma, dtype)
    return q, k, v


def _opts(onepass=True, chunks=0, timer=None, **kw):
    form = binding.LA_FORM_ONE_LAUNCH if onepass else binding.LA_FORM_TWO_LAUNCH
    return binding.options(segment_chunks=chunks, forward_form=form, timer=timer, **kw)


def _resident(B, H, N, D, M, opts):
    """Forced one-launch tests keep the whole grid resident at once (at most one workgroup per compute unit), so
    no wait depends on the order in which workgroups are dispatched."""
    nseg = -(-N // binding.segment_length(B, H, N, D, M, opts))
    assert B * H * nseg <= 256, (B, H, N, nseg)


def _run(q, k, v, dtype, s0=None, z0=None, onepass=True, chunks=0):
    """Forward with checkpoint and final state; returns the outputs and whether the one-pass form ran (it is the
    form that launches the flag-clearing kernel)."""
    timer = binding.KernelTimer("sync_clear", 4)
    opts = _opts(onepass, chunks, timer)
    B, H, N, D = q.shape
    if onepass:
        _resident(B, H, N, D, v.shape[-1], opts)
    out = binding.forward_causal(dev(q, dtype), dev(k, dtype), dev(v, dtype),
                                 s0=None if s0 is None else dev32(s0), z0=None if z0 is None else dev32(z0),
                                 return_state=True, checkpoint=True, opts=opts)
    torch.cuda.synchronize()
    launches = timer.launches
    if launches:
        assert binding.forward_wait_status(out["ws"], B, H, N, D, v.shape[-1], binding.dtype_code(out["o"].dtype),
                                           opts) == 0
    out["opts"] = opts
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


def _error_word(ws, B, H, N, D, M, opts):
    """Word 0 of the one-launch forward's flag region: after the aggregates and the prefix states of the workspace."""
    L = binding.segment_length(B, H, N, D, M, opts)
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
    out, onepass = _run(q, k, v, dtype, chunks=chunks)
    L = binding.segment_length(B, H, N, D, M, out["opts"])
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
    out, onepass = _run(q, k, v, dtype, s0, z0, chunks=2)
    assert onepass
    _check(out, q, k, v, dtype, s0, z0)


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_onepass_matches_two_launch_form(dtype):
    """Both forms of the forward agree within the tolerance, and the backward from either checkpoint matches."""
    B, H, N, D, M = 2, 8, 784, 32, 32
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
    ga = binding.backward_causal(Q, K, V, a["o"], a["den"], dO, ckpt=a["ckpt"], opts=a["opts"])
    gb = binding.backward_causal(Q, K, V, b["o"], b["den"], dO, ckpt=b["ckpt"], opts=b["opts"])
    torch.cuda.synchronize()
    rq, rk, rv = oracle.backward_causal(q, k, v, do)
    for x, y, r in zip(ga, gb, (rq, rk, rv)):
        # dQ of the first token is an exact cancellation (zero): rows are judged against the tensor's scale
        assert rowerr(host(x), host(y), row_floor=np.full(r.shape[:-1], 1e-3 * np.abs(r).max())) <= TOL[dtype]


def test_onepass_rule():
    """By default the one-launch form runs for states of D*M >= 2048 and the two-launch form below that."""
    for (D, M), want in (((32, 32), False), ((64, 32), True), ((64, 64), True)):
        q, k, v = _qkv(2, 2, 300, D, M, F32, 7900)
        timer = binding.KernelTimer("sync_clear", 4)
        binding.forward_causal(dev(q), dev(k), dev(v), opts=binding.options(timer=timer))
        torch.cuda.synchronize()
        assert (timer.launches > 0) == want, (D, M)


def test_onepass_reused_dirty_workspace():
    """Two calls on one workspace that starts filled with 0xff bytes: the call clears its own flags."""
    B, H, N, D, M = 2, 8, 784, 32, 32
    q, k, v = _qkv(B, H, N, D, M, F32, 7700)
    Q, K, V = dev(q), dev(k), dev(v)
    timer = binding.KernelTimer("sync_clear", 4)
    opts = _opts(True, 0, timer)
    _resident(B, H, N, D, M, opts)
    ws = binding.alloc_workspace(binding.LA_OP_FWD_CAUSAL, B, H, N, D, M, binding.dtype_code(torch.float32), "cuda",
                                 opts)
    ws.fill_(255)
    ref = oracle.forward_causal(q, k, v)
    assert binding.segment_length(B, H, N, D, M, opts) <= 4 * 64
    for _ in range(2):
        O = torch.empty((B, H, N, M), device="cuda")
        den = torch.empty((B, H, N), device="cuda")
        binding.la_forward_causal(Q, K, V, O, den, ws=ws, opts=opts)
        torch.cuda.synchronize()
        assert _error_word(ws, B, H, N, D, M, opts) == 0  # no wait gave up
        assert binding.forward_wait_status(ws, B, H, N, D, M, binding.LA_F32, opts) == 0
        assert rowerr(host(O), ref[0]) <= 1e-4
        assert rowerr(host(den), ref[1], False) <= 1e-4
    assert timer.launches == 2


def test_onepass_wait_limit():
    """With the poll limit at 0 every wait gives up at once (forced from the host: no wave spins): the first segment
    of each head needs no carry and stays exact, later segments' rows and the final state are NaN, the error word
    is set; the next call at the normal limit is exact again."""
    B, H, N, D, M = 2, 3, 5 * 64 + 11, 32, 32
    q, k, v = _qkv(B, H, N, D, M, F32, 7950)
    Q, K, V = dev(q), dev(k), dev(v)
    o_ref, den_ref, _, _ = oracle.forward_causal(q, k, v)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    base = _opts(True, 2)
    L = binding.segment_length(B, H, N, D, M, base)
    _resident(B, H, N, D, M, base)
    ws = binding.alloc_workspace(binding.LA_OP_FWD_CAUSAL, B, H, N, D, M, binding.dtype_code(torch.float32), "cuda",
                                 base)
    for polls in (-1, 0):  # none at all (the failure path), then the default limit
        opts = _opts(True, 2, wait_polls=polls, status=status)
        O = torch.empty((B, H, N, M), device="cuda")
        den = torch.empty((B, H, N), device="cuda")
        S = torch.empty((B, H, D, M), device="cuda")
        Z = torch.empty((B, H, D), device="cuda")
        binding.la_forward_causal(Q, K, V, O, den, S_out=S, Z_out=Z, ws=ws, opts=opts)
        torch.cuda.synchronize()
        o, d = host(O), host(den)
        if polls < 0:
            assert _error_word(ws, B, H, N, D, M, opts) == 1
            assert binding.forward_wait_status(ws, B, H, N, D, M, binding.LA_F32, opts) == binding.LA_ERR_WAIT
            assert int(status.item()) == 1  # the caller's status word is set too
            status.zero_()
            assert rowerr(o[:, :, :L], o_ref[:, :, :L]) <= 1e-4
            assert rowerr(d[:, :, :L], den_ref[:, :, :L], False) <= 1e-4
            assert np.isnan(o[:, :, L:]).all() and np.isnan(d[:, :, L:]).all()
            assert np.isnan(host(S)).all() and np.isnan(host(Z)).all()
        else:
            assert _error_word(ws, B, H, N, D, M, opts) == 0
            assert binding.forward_wait_status(ws, B, H, N, D, M, binding.LA_F32, opts) == 0
            assert int(status.item()) == 0
            assert rowerr(o, o_ref) <= 1e-4
            assert rowerr(d, den_ref, False) <= 1e-4


def test_onepass_many_heads():
    """Sixteen heads of the MNIST-shaped layer (B=2 H=8 N=784 D=M=32 float32; the grid of 208 workgroups is
    resident at once): rows sampled from every head."""
    B, H, N, D, M = 2, 8, 784, 32, 32
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


def test_threads_with_different_options():
    """Two host threads run the causal forward and backward at the same time with different segment options and
    forms, each on its own stream: each gets exactly (bitwise) what the same call gives alone, and the oracle's
    outputs (the library keeps no state between calls)."""
    import threading

    B, H, N, D, M = 2, 4, 700, 64, 32
    q, k, v = _qkv(B, H, N, D, M, F32, 7990)
    do = inputs.gaussian((B, H, N, M), 7994)
    o_ref, den_ref, _, _ = oracle.forward_causal(q, k, v)
    cases = ((1, True), (3, False))

    def run(chunks, onepass):
        opts = _opts(onepass, chunks)
        Q, K, V, dO = dev(q), dev(k), dev(v), dev(do)
        out = binding.forward_causal(Q, K, V, opts=opts)
        g = binding.backward_causal(Q, K, V, out["o"], out["den"], dO, ckpt=out["ckpt"], opts=opts)
        return binding.segment_length(B, H, N, D, M, opts), [out["o"], out["den"]] + list(g)

    alone = {}
    for c in cases:
        L, ts = run(*c)
        torch.cuda.synchronize()
        alone[c] = (L, [host(t) for t in ts])
    results, errors = {}, []

    def worker(chunks, onepass):
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                for _ in range(5):
                    L, ts = run(chunks, onepass)
                stream.synchronize()
                results[(chunks, onepass)] = (L, [host(t) for t in ts])
        except Exception as e:  # noqa: BLE001
            errors.append(e)

    threads = [threading.Thread(target=worker, args=c) for c in cases]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for c in cases:
        L, got = results[c]
        assert L == 64 * c[0] == alone[c][0]
        for x, y in zip(got, alone[c][1]):
            assert np.array_equal(x, y)
        assert rowerr(got[0], o_ref) <= 1e-4
        assert rowerr(got[1], den_ref, False) <= 1e-4
