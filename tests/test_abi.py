"""The C-ABI library loads, exports what include/la.h declares, and rejects bad
arguments before launching anything.  CPU only: no call here reaches a kernel
(fake device addresses are never dereferenced by the host)."""
import ctypes
import os
import re

import pytest

from linear_rnn_layers_amd import binding
from linear_rnn_layers_amd import build as labuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "la.h")

OK, NULL, SHAPE, DTYPE, ALIGN, ALIAS, WORKSPACE, UNSUPPORTED, HIP, ARG, WAIT = range(11)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(la_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return binding.load()


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(lib, n), f"{n} declared in la.h but not exported"
    assert sorted(binding.ENTRY_POINTS) == names


def test_only_declared_symbols_are_exported():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", labuild.LIB], capture_output=True, text=True, check=True)
    exported = sorted({ln.split()[-1] for ln in out.stdout.splitlines() if " T " in ln})
    assert exported == declared_functions()


def test_version_and_strings(lib):
    assert lib.la_version() >= 100
    assert lib.la_status_string(0) == b"LA_OK"
    assert lib.la_status_string(WORKSPACE) == b"LA_ERR_WORKSPACE"
    assert lib.la_status_string(99) == b"LA_ERR_UNKNOWN"
    names = binding.kernel_names()
    assert "fwd_causal" in names and "bwd_query" in names and "bwd_kv" in names and "decode" in names


# Fake, 256-aligned, non-overlapping device addresses (never dereferenced).
BASE = 0x7F0000000000


def addr(i):
    return ctypes.c_void_p(BASE + i * (1 << 32))


def fwd(lib, B=2, H=2, N=100, D=32, M=32, dtype=0, ws=True, **over):
    args = dict(Q=addr(1), K=addr(2), V=addr(3), logA=None, O=addr(4), den=addr(5), S0=None, Z0=None, S_out=None,
                Z_out=None, ckpt=None)
    opts = over.pop("opts", None)
    args.update(over)
    need = lib.la_workspace_size(5 if args["logA"] else 0, B, H, N, D, M, dtype, None)
    wsp = addr(20) if ws else None
    nb = need if ws else 0
    if "ws_bytes" in over:
        nb = over.pop("ws_bytes")
        args.pop("ws_bytes")
    return lib.la_forward_causal(args["Q"], args["K"], args["V"], args["logA"], args["O"], args["den"], args["S0"],
                                 args["Z0"], args["S_out"], args["Z_out"], args["ckpt"], B, H, N, D, M, dtype,
                                 args.get("feature", 0), wsp, nb, None, opts)


def test_forward_validation(lib):
    assert fwd(lib, dtype=2) == DTYPE
    assert fwd(lib, B=0) == SHAPE
    assert fwd(lib, H=-1) == SHAPE
    assert fwd(lib, N=-5) == SHAPE
    assert fwd(lib, D=48) == UNSUPPORTED
    assert fwd(lib, M=128) == UNSUPPORTED
    assert fwd(lib, Q=None) == NULL
    assert fwd(lib, O=None) == NULL
    assert fwd(lib, S0=addr(6)) == ARG  # S0 without Z0
    assert fwd(lib, S_out=addr(7)) == ARG  # S_out without Z_out
    assert fwd(lib, K=ctypes.c_void_p(BASE + 2 * (1 << 32) + 8)) == ALIGN
    assert fwd(lib, O=addr(1)) == ALIAS  # output on top of Q
    assert fwd(lib, den=ctypes.c_void_p(BASE + 4 * (1 << 32) + 64)) == ALIAS  # den inside O
    assert fwd(lib, ws=False) == WORKSPACE
    assert fwd(lib, ws_bytes=16) == WORKSPACE
    assert b"workspace" in lib.la_last_error()


def test_noncausal_and_backward_validation(lib):
    ws = lib.la_workspace_size(1, 1, 1, 64, 64, 64, 1, None)
    assert lib.la_forward_noncausal(addr(1), addr(2), addr(3), None, None, None, 1, 1, 64, 64, 64, 1, 0, addr(20), ws, None, None) == NULL
    assert lib.la_forward_noncausal(addr(1), addr(2), addr(3), addr(4), None, None, 1, 1, 64, 64, 64, 1, 0, None, 0, None, None) == WORKSPACE
    assert lib.la_forward_noncausal(addr(1), addr(2), addr(3), addr(3), None, None, 1, 1, 64, 64, 64, 1, 0, addr(20), ws,
                                    None, None) == ALIAS
    # N = 0 is a no-op
    assert lib.la_forward_noncausal(None, None, None, None, None, None, 1, 1, 0, 64, 64, 1, 0, None, 0, None, None) == OK
    wsb = lib.la_workspace_size(2, 2, 2, 100, 32, 32, 0, None)
    names = ["Q", "K", "V", "logA", "O", "den", "dO", "S0", "Z0", "ckpt", "dS_N", "dZ_N", "dQ", "dK", "dV", "dlogA",
             "dS0", "dZ0"]
    base = dict(Q=addr(1), K=addr(2), V=addr(3), O=addr(4), den=addr(5), dO=addr(6), dQ=addr(7), dK=addr(8),
                dV=addr(9))

    def bwd(N=100, ws=addr(20), nb=wsb, **over):
        a = dict(base)
        a.update(over)
        return lib.la_backward_causal(*[a.get(n) for n in names], 2, 2, N, 32, 32, 0, a.get("feature", 0), ws, nb, None, None)

    assert bwd(den=None) == NULL  # den is required
    assert bwd(dQ=addr(6)) == ALIAS  # dQ on top of dO
    assert bwd(S0=addr(10)) == ARG  # S0 without Z0
    assert bwd(dS_N=addr(10)) == ARG  # dS_N without dZ_N
    assert bwd(dS0=addr(12)) == ARG  # dS0 without dZ0
    assert bwd(dS_N=addr(10), dZ_N=addr(11), dS0=addr(10), dZ0=addr(13)) == ALIAS  # dS0 on top of dS_N
    assert bwd(dS0=ctypes.c_void_p(BASE + 12 * (1 << 32) + 4), dZ0=addr(13)) == ALIGN
    assert bwd(nb=wsb - 1) == WORKSPACE
    assert bwd(N=0, ws=None, nb=0) == OK
    # N = 0 with a state gradient requested still validates that request (no launch happens on failure)
    assert bwd(N=0, ws=None, nb=0, dS0=addr(12), dZ0=addr(13), dS_N=addr(12), dZ_N=addr(11)) == ALIAS
    # decayed recurrence: logA and dlogA go together, dlogA is an output, the workspace grows
    assert bwd(logA=addr(14)) == ARG
    assert bwd(dlogA=addr(15)) == ARG
    wsd = lib.la_workspace_size(6, 2, 2, 100, 32, 32, 0, None)
    assert wsd > wsb
    assert bwd(logA=addr(14), dlogA=addr(15), nb=wsb) == WORKSPACE
    assert bwd(logA=addr(14), dlogA=addr(14), nb=wsd) == ALIAS
    assert bwd(logA=ctypes.c_void_p(BASE + 14 * (1 << 32) + 4), dlogA=addr(15), nb=wsd) == ALIGN


def test_feature_argument_validation(lib):
    assert fwd(lib, feature=2) == ARG
    assert fwd(lib, feature=-1) == ARG
    assert b"feature" in lib.la_last_error()
    assert lib.la_decode_step(addr(1), addr(2), addr(3), None, addr(4), addr(5), addr(6), 2, 2, 64, 64, 1, 5,
                              None, None) == ARG


def test_feature_map_validation(lib):
    # random features: Din, C in {32, 64}; W [H,C,Din] float32; outputs must not overlap inputs
    assert lib.la_feature_random(addr(1), addr(2), addr(3), 2, 2, 100, 48, 32, 0, None) == UNSUPPORTED
    assert lib.la_feature_random(addr(1), None, addr(3), 2, 2, 100, 32, 32, 0, None) == NULL
    assert lib.la_feature_random(addr(1), addr(2), addr(1), 2, 2, 100, 32, 32, 0, None) == ALIAS
    assert lib.la_feature_random_vjp(addr(1), addr(2), None, addr(4), 2, 2, 100, 32, 32, 0, None) == NULL
    assert lib.la_feature_random(None, None, None, 2, 2, 0, 32, 32, 0, None) == OK
    # degree-2 polynomial: 1 + Din + Din^2 <= C
    assert lib.la_feature_poly2(addr(1), addr(3), 2, 2, 100, 6, 32, 0, None) == UNSUPPORTED
    assert lib.la_feature_poly2(addr(1), addr(3), 2, 2, 100, 8, 64, 0, None) == UNSUPPORTED
    assert lib.la_feature_poly2(addr(1), addr(3), 2, 2, 100, 5, 48, 0, None) == UNSUPPORTED
    assert lib.la_feature_poly2(addr(1), addr(1), 2, 2, 100, 5, 32, 0, None) == ALIAS
    assert lib.la_feature_poly2_vjp(addr(1), None, addr(4), 2, 2, 100, 5, 32, 0, None) == NULL
    assert lib.la_feature_poly2(addr(1), addr(3), 2, 2, 100, 5, 32, 3, None) == DTYPE


def test_decay_forward_validation(lib):
    need = lib.la_workspace_size(5, 2, 2, 100, 32, 32, 0, None)  # the decayed forward's workspace
    assert need > 0
    assert fwd(lib, logA=addr(14), ws_bytes=need - 1) == WORKSPACE
    assert fwd(lib, logA=addr(4)) == ALIAS  # O on top of logA
    assert fwd(lib, logA=ctypes.c_void_p(BASE + 14 * (1 << 32) + 8)) == ALIGN


def test_noncausal_backward_validation(lib):
    ws = lib.la_workspace_size(4, 2, 2, 100, 32, 32, 0, None)
    assert ws > 0
    args = [addr(1), addr(2), addr(3), addr(4), None, None, addr(5), addr(6), addr(7)]
    a = list(args)
    a[6] = None
    assert lib.la_backward_noncausal(*a, 2, 2, 100, 32, 32, 0, 0, addr(20), ws, None, None) == NULL
    a = list(args)
    a[7] = addr(1)  # dK on top of Q
    assert lib.la_backward_noncausal(*a, 2, 2, 100, 32, 32, 0, 0, addr(20), ws, None, None) == ALIAS
    assert lib.la_backward_noncausal(*args, 2, 2, 100, 32, 32, 0, 0, addr(20), ws - 1, None, None) == WORKSPACE
    assert lib.la_backward_noncausal(*args, 2, 2, 100, 48, 32, 0, 0, addr(20), ws, None, None) == UNSUPPORTED
    assert lib.la_backward_noncausal(*args, 2, 2, 0, 32, 32, 0, 0, None, 0, None, None) == OK
    a = list(args)
    a[4] = addr(8)  # S_tot without Z_tot
    assert lib.la_backward_noncausal(*a, 2, 2, 100, 32, 32, 0, 0, addr(20), ws, None, None) == ARG
    a[5] = addr(9)
    a[6] = addr(8)  # dQ on top of S_tot
    assert lib.la_backward_noncausal(*a, 2, 2, 100, 32, 32, 0, 0, addr(20), ws, None, None) == ALIAS
    assert lib.la_forward_noncausal(addr(1), addr(2), addr(3), addr(4), addr(5), None, 2, 2, 100, 32, 32, 0, 0,
                                    addr(20), 1 << 30, None, None) == ARG


def test_decode_validation(lib):
    assert lib.la_decode_step(addr(1), addr(2), addr(3), None, addr(4), addr(5), None, 2, 2, 64, 64, 1, 0, None, None) == NULL
    assert lib.la_decode_step(addr(1), addr(2), addr(3), None, addr(4), addr(4), addr(6), 2, 2, 64, 64, 1, 0, None, None) == ALIAS
    assert lib.la_decode_step(addr(1), addr(2), addr(3), addr(4), addr(4), addr(5), addr(6), 2, 2, 64, 64, 1, 0,
                              None, None) == ALIAS  # S on top of logA
    assert lib.la_decode_step(addr(1), addr(2), addr(3), None, addr(4), addr(5), addr(6), 2, 2, 16, 64, 1, 0,
                              None, None) == UNSUPPORTED
    assert lib.la_decode_step(addr(1), addr(2), addr(3), None, addr(4), addr(5), addr(6), 2, 0, 64, 64, 1, 0, None, None) == SHAPE


def _plan(B, H, N, target=None, D=32, M=32):
    """The segment plan, restated: about `target` segments over all heads, each of whole 64-token chunks
    (512 for the non-causal ops and the decayed recurrence; for the causal ops 1024 when a head has at most
    16 chunks and D*M <= 1024, else 512)."""
    bh = B * H
    nch = -(-N // 64)
    if target is None:
        target = 1024 if nch <= 16 and D * M <= 1024 else 512
    segs = max(1, min(nch, -(-target // bh)))
    L = -(-nch // segs) * 64
    return L, -(-N // L)


@pytest.mark.parametrize("B,H,N,D,M", [(1, 1, 64, 32, 32), (16, 8, 784, 32, 32), (4, 8, 3072, 32, 32),
                                        (1, 16, 65536, 64, 64), (3, 5, 1000, 64, 32), (1, 1, 1, 32, 64)])
def test_plan_and_sizes(lib, B, H, N, D, M):
    L, nseg = _plan(B, H, N, D=D, M=M)
    assert lib.la_segment_length(B, H, N, D, M, None) == L
    sv = D * M + D
    assert lib.la_checkpoint_size(B, H, N, D, M, None) == B * H * (nseg + 1) * sv * 4
    # linear-memory bound: the checkpoint never exceeds B*H*N*max(D,M) floats by more than one state per head
    assert lib.la_checkpoint_size(B, H, N, D, M, None) <= 4 * B * H * (N * max(D, M) + 2 * sv)
    assert lib.la_workspace_size(3, B, H, N, D, M, 1, None) == 0
    # forward: segment aggregates, their prefix scan and the one-pass form's error word and per-segment flags
    # (32-bit words) when there is more than one segment
    agg, pref = _al(B * H * nseg * sv * 4), _al(B * H * (nseg + 1) * sv * 4)
    sync = _al((1 + B * H * nseg) * 4)
    assert lib.la_workspace_size(0, B, H, N, D, M, 0, None) == (0 if nseg == 1 else agg + pref + sync)
    _, nseg_nc = _plan(B, H, N, 512)
    agg_nc, pref_nc = _al(B * H * nseg_nc * sv * 4), _al(B * H * (nseg_nc + 1) * sv * 4)
    assert lib.la_workspace_size(1, B, H, N, D, M, 0, None) == agg_nc + pref_nc
    # backward: room to recompute the checkpoint, the reverse aggregates (more than one segment) and the
    # per-token pair (1/den, O.dO) the query pass hands to the key pass
    bwd = _al(B * H * nseg * sv * 4) + _al(B * H * (nseg + 1) * sv * 4) + (0 if nseg == 1 else _al(B * H * nseg * sv * 4))
    bwd += _al(B * H * N * 8)
    assert lib.la_workspace_size(2, B, H, N, D, M, 0, None) == bwd
    # non-causal backward: key aggregates + scan, reverse aggregates + scan
    assert lib.la_workspace_size(4, B, H, N, D, M, 0, None) == 2 * (agg_nc + pref_nc)
    # decayed forward: aggregates, prefix states, per-segment log-decay sums (more than one segment);
    # decayed backward: those, reverse aggregates and (1/den, c) per token
    dl = _al(B * H * nseg_nc * 4)  # the decayed recurrence plans like the non-causal ops
    assert lib.la_workspace_size(5, B, H, N, D, M, 0, None) == (0 if nseg_nc == 1 else agg_nc + pref_nc + dl)
    assert lib.la_workspace_size(6, B, H, N, D, M, 1, None) == agg_nc + pref_nc + dl + agg_nc + _al(B * H * N * 8) + dl
    assert lib.la_workspace_size(9, B, H, N, D, M, 0, None) == 0


def _al(x):
    return (x + 255) // 256 * 256


def opt(**kw):
    return ctypes.byref(binding.Options(**kw))


def test_per_call_options(lib):
    """The segment option changes the plan of that call only; invalid options are refused before any launch."""
    assert lib.la_segment_length(2, 2, 1000, 32, 32, opt(segment_chunks=3)) == 3 * 64
    assert lib.la_segment_length(2, 2, 1000, 32, 32, None) == _plan(2, 2, 1000)[0]
    assert lib.la_segment_length(2, 2, 1000, 32, 32, opt()) == _plan(2, 2, 1000)[0]
    # clamped to the sequence
    assert lib.la_segment_length(2, 2, 1000, 32, 32, opt(segment_chunks=99)) == 16 * 64
    sv = 32 * 32 + 32
    assert lib.la_checkpoint_size(2, 2, 1000, 32, 32, opt(segment_chunks=3)) == 4 * (-(-1000 // 192) + 1) * sv * 4
    assert fwd(lib, opts=opt(segment_chunks=-1)) == ARG
    assert b"segment_chunks" in lib.la_last_error()
    assert fwd(lib, opts=opt(forward_form=3)) == ARG
    assert fwd(lib, opts=opt(forward_form=-1)) == ARG
    t = binding.Options(timed_kernel=b"fwd_causal")  # timing without events
    assert fwd(lib, opts=ctypes.byref(t)) == ARG
    assert fwd(lib, opts=opt(status=BASE + 2)) == ALIGN
    assert lib.la_status_string(WAIT) == b"LA_ERR_WAIT"
    # the status query validates before it reads anything
    assert lib.la_forward_wait_status(addr(20), 16, 2, 2, 1000, 32, 32, 0, None, None) == WORKSPACE
    assert lib.la_forward_wait_status(addr(20), 1 << 30, 2, 2, 1000, 48, 32, 0, None, None) == UNSUPPORTED
    assert lib.la_forward_wait_status(None, 0, 1, 1, 64, 32, 32, 0, None, None) == OK  # one segment: no flags
    with pytest.raises(ValueError):
        binding.options(forward_form=5)
    with pytest.raises(ValueError):
        binding.options(segment_chunks=-2)


def test_threads_with_different_options_are_independent(lib):
    """Two host threads plan with different segment options at the same time: each sees only its own (the
    library keeps no state between calls).  The GPU counterpart runs the forward itself from two threads."""
    import threading

    B, H, N, D, M = 2, 3, 5000, 32, 32
    res = {}
    errors = []

    def worker(chunks):
        o = binding.Options(segment_chunks=chunks)
        try:
            for _ in range(2000):
                L = lib.la_segment_length(B, H, N, D, M, ctypes.byref(o))
                ck = lib.la_checkpoint_size(B, H, N, D, M, ctypes.byref(o))
                ws = lib.la_workspace_size(0, B, H, N, D, M, 0, ctypes.byref(o))
                # an invalid call on this thread leaves the other thread's error text alone
                assert fwd(lib, B=B, H=H, N=N, opts=ctypes.byref(binding.Options(forward_form=7))) == ARG
                res.setdefault(chunks, set()).add((L, ck, ws))
        except Exception as e:  # noqa: BLE001
            errors.append(e)

    ts = [threading.Thread(target=worker, args=(c,)) for c in (2, 5)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert not errors, errors
    for c in (2, 5):
        assert len(res[c]) == 1
        L, ck, ws = next(iter(res[c]))
        assert L == 64 * c
        nseg = -(-N // L)
        assert ck == B * H * (nseg + 1) * (D * M + D) * 4
    assert res[2] != res[5]


def test_binding_checks_tensor_agreement():
    """The binding compares every tensor with the sizes it passes to the C library (shape and dtype) before it
    touches a device pointer, so a mismatched call raises ValueError instead of reading past a buffer."""
    import torch

    B, H, N, D, M = 2, 3, 10, 32, 32
    f = lambda *s, dt=torch.float32: torch.zeros(*s, dtype=dt)  # noqa: E731
    q, k, v, o = f(B, H, N, D), f(B, H, N, D), f(B, H, N, M), f(B, H, N, M)
    cases = [
        lambda: binding.la_forward_causal(q, f(B, H, N - 1, D), v, o),  # short K
        lambda: binding.la_forward_causal(q, k, f(B, H, N + 1, M), o),  # V of another length
        lambda: binding.la_forward_causal(q, k, v.to(torch.bfloat16), o),  # mixed dtypes
        lambda: binding.la_forward_causal(q, k, v, f(B, H, N, D + 32)),  # O of the wrong width
        lambda: binding.la_forward_causal(q, k, v, o, den=f(B, H, N + 1)),
        lambda: binding.la_forward_causal(q, k, v, o, den=f(B, H, N, dt=torch.float64)),
        lambda: binding.la_forward_causal(q, k, v, o, S0=f(B, H, D, M, dt=torch.bfloat16), Z0=f(B, H, D)),
        lambda: binding.la_forward_causal(q, k, v, o, S_out=f(B, H, D, M), Z_out=f(B, H, D + 1)),
        lambda: binding.la_forward_causal(q, k, v, o, logA=f(B, H, N - 1)),
        lambda: binding.la_forward_causal(q, k, v, o, ckpt=f(7)),  # wrong checkpoint size
        lambda: binding.la_forward_causal(q, k, v, o, ws=f(100)),  # workspace not bytes
        lambda: binding.la_backward_causal(q, k, v, o, f(B, H, N), f(B, H, N, M), f(B, H, N, D), f(B, H, N, D),
                                           f(B, H, N - 1, M)),  # short dV
        lambda: binding.la_backward_causal(q, k, v, o, f(B, H, N), f(B, H, N, M, dt=torch.bfloat16), f(B, H, N, D),
                                           f(B, H, N, D), f(B, H, N, M)),  # dO of another dtype
        lambda: binding.la_backward_causal(q, k, v, o, f(B, H, N), f(B, H, N, M), f(B, H, N, D), f(B, H, N, D),
                                           f(B, H, N, M), dS_N=f(B, H, D, M), dZ_N=f(B, H, M + 1)),
        lambda: binding.la_backward_noncausal(q, k, v, f(B, H, N, M), f(B, H, N, D), f(B, H, N + 3, D),
                                              f(B, H, N, M)),
        lambda: binding.la_forward_noncausal(q, k, v, o, S_out=f(B, H, M, D + 32), Z_out=f(B, H, D)),
        lambda: binding.la_decode_step(f(B, H, D), f(B, H, D), f(B, H, M), f(B, H, D, M, dt=torch.bfloat16),
                                       f(B, H, D), f(B, H, M)),  # bf16 state would be overrun
        lambda: binding.la_decode_step(f(B, H, D), f(B, H, D), f(B, H, M), f(B, H, D, M), f(B, H, D), f(B, H, M),
                                       logA=f(B, H, 1)),
        lambda: binding.la_decode_step(f(B, H, D), f(B, H, D - 1), f(B, H, M), f(B, H, D, M), f(B, H, D),
                                       f(B, H, M)),
        lambda: binding.feature_random(q, f(H + 1, 64, D)),  # projection of another head count
        lambda: binding.feature_random_vjp(q, f(H, 64, D), f(B, H, N, 32)),
    ]
    for i, c in enumerate(cases):
        with pytest.raises(ValueError):
            c()
        # and the well-formed call only fails at the device check (no GPU here)
    with pytest.raises(ValueError, match="GPU"):
        binding.la_forward_causal(q, k, v, o, den=f(B, H, N))


@pytest.mark.parametrize("B,H,N,C,M", [(2, 2, 300, 128, 32), (4, 8, 3072, 1088, 32), (16, 8, 784, 256, 32),
                                        (1, 1, 1, 4096, 64), (1, 2, 5000, 192, 64)])
def test_wide_plan_and_sizes(lib, B, H, N, C, M):
    """Wide feature vectors (C = 64 ns): the plan of the B*H*ns feature slices as 64-feature heads; the
    checkpoint holds the slices' states; the workspaces add the slices' shares of the numerators and
    denominators (the forward), and of dV and of the pair (num . dO, den) per token (the backward)."""
    ns = C // 64
    L, nseg = _plan(B, H * ns, N, D=64, M=M)
    assert lib.la_segment_length(B, H, N, C, M, None) == L
    sv = 64 * M + 64
    bhs = B * H * ns
    assert lib.la_checkpoint_size(B, H, N, C, M, None) == bhs * (nseg + 1) * sv * 4
    pn, pd = _al(bhs * N * M * 4), _al(bhs * N * 4)
    agg, pref = _al(bhs * nseg * sv * 4), _al(bhs * (nseg + 1) * sv * 4)
    assert lib.la_workspace_size(0, B, H, N, C, M, 0, None) == (0 if nseg == 1 else agg + pref) + pn + pd
    _, nseg_nc = _plan(B, H * ns, N, 512)
    assert lib.la_workspace_size(1, B, H, N, C, M, 1, None) == (_al(bhs * nseg_nc * sv * 4) +
                                                                _al(bhs * (nseg_nc + 1) * sv * 4) + pn + pd)
    bwd = agg + pref + (0 if nseg == 1 else agg) + _al(B * H * N * 8) + pn + _al(bhs * N * 8)
    assert lib.la_workspace_size(2, B, H, N, C, M, 0, None) == bwd
    # non-causal backward: key and reverse aggregates with their scans, then the pair per token and the shares
    nc_st = _al(bhs * nseg_nc * sv * 4) + _al(bhs * (nseg_nc + 1) * sv * 4)
    assert lib.la_workspace_size(4, B, H, N, C, M, 0, None) == 2 * nc_st + _al(B * H * N * 8) + pn + _al(bhs * N * 8)
    for op in (3, 5, 6):  # decode needs none; no decayed form for wide features
        assert lib.la_workspace_size(op, B, H, N, C, M, 0, None) == 0


def test_wide_validation(lib):
    assert fwd(lib, D=96) == UNSUPPORTED
    assert fwd(lib, D=4160) == UNSUPPORTED
    assert fwd(lib, D=128) == UNSUPPORTED  # elu + 1 is applied to 32- or 64-wide heads only
    assert b"LA_FEATURE_IDENTITY" in lib.la_last_error()
    assert fwd(lib, D=128, feature=1, logA=addr(14)) == UNSUPPORTED
    assert b"decay" in lib.la_last_error()
    args = [addr(1), addr(2), addr(3), addr(4), None, None, addr(5), addr(6), addr(7)]
    assert lib.la_backward_noncausal(*args, 2, 2, 100, 128, 32, 0, 0, addr(20), 1 << 30, None, None) == UNSUPPORTED
    assert lib.la_decode_step(addr(1), addr(2), addr(3), None, addr(4), addr(5), addr(6), 2, 2, 128, 64, 1, 0,
                              None, None) == UNSUPPORTED
    assert lib.la_decode_step(addr(1), addr(2), addr(3), addr(8), addr(4), addr(5), addr(6), 2, 2, 128, 64, 1, 1,
                              None, None) == UNSUPPORTED
    # wide feature maps: C a multiple of 64 up to 4096; degree 2 needs 1 + Din + Din^2 <= C and Din <= 64
    assert lib.la_feature_random(addr(1), addr(2), addr(3), 2, 2, 100, 32, 96, 0, None) == UNSUPPORTED
    assert lib.la_feature_random(addr(1), addr(2), addr(3), 2, 2, 100, 32, 4160, 0, None) == UNSUPPORTED
    assert lib.la_feature_poly2(addr(1), addr(3), 2, 2, 100, 32, 1024, 0, None) == UNSUPPORTED
    assert lib.la_feature_poly2(addr(1), addr(3), 2, 2, 100, 65, 4096, 0, None) == UNSUPPORTED
    assert lib.la_feature_poly2(addr(1), addr(1), 2, 2, 100, 32, 1088, 0, None) == ALIAS
    names = binding.kernel_names()
    assert all(n in names for n in ("wide_combine", "bwd_query_shares", "nc_qr_shares", "wide_pairs", "wide_sum",
                                    "decode_wide",
                                    "feat_rf_vjp_wide", "feat_poly2_wide", "feat_poly2_vjp_wide"))


def test_binding_feature_sliced_layout():
    """Q, K wider than 64 features go in feature-sliced [B,H,D/64,N,64]; the plain layout is refused."""
    import torch

    q = torch.zeros((2, 3, 4, 10, 64))
    v = torch.zeros((2, 3, 10, 32))
    assert binding._sizes(q, q, v) == (2, 3, 10, 256, 32)
    with pytest.raises(ValueError, match="feature-sliced"):
        binding._sizes(torch.zeros((2, 3, 10, 256)), torch.zeros((2, 3, 10, 256)), v)
    with pytest.raises(ValueError):
        binding._sizes(torch.zeros((2, 3, 4, 10, 32)), torch.zeros((2, 3, 4, 10, 32)), v)
    x = torch.arange(2 * 3 * 10 * 256, dtype=torch.float32).reshape(2, 3, 10, 256)
    s = binding.to_sliced(x)
    assert tuple(s.shape) == (2, 3, 4, 10, 64)
    assert torch.equal(s[1, 2, 3, 7], x[1, 2, 7, 192:256])
    assert torch.equal(binding.from_sliced(s), x)
    assert binding.feature_shape(2, 3, 10, 64) == (2, 3, 10, 64)
    assert binding.feature_shape(2, 3, 10, 1088) == (2, 3, 17, 10, 64)
