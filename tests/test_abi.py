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

OK, NULL, SHAPE, DTYPE, ALIGN, ALIAS, WORKSPACE, UNSUPPORTED, HIP, ARG = range(10)


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
    assert "fwd_causal" in names and "bwd_causal" in names and "decode" in names


# Fake, 256-aligned, non-overlapping device addresses (never dereferenced).
BASE = 0x7F0000000000


def addr(i):
    return ctypes.c_void_p(BASE + i * (1 << 32))


def fwd(lib, B=2, H=2, N=100, D=32, M=32, dtype=0, ws=True, **over):
    args = dict(Q=addr(1), K=addr(2), V=addr(3), logA=None, O=addr(4), den=addr(5), S0=None, Z0=None, S_out=None,
                Z_out=None, ckpt=None)
    args.update(over)
    need = lib.la_workspace_size(5 if args["logA"] else 0, B, H, N, D, M, dtype)
    wsp = addr(20) if ws else None
    nb = need if ws else 0
    if "ws_bytes" in over:
        nb = over.pop("ws_bytes")
        args.pop("ws_bytes")
    return lib.la_forward_causal(args["Q"], args["K"], args["V"], args["logA"], args["O"], args["den"], args["S0"],
                                 args["Z0"], args["S_out"], args["Z_out"], args["ckpt"], B, H, N, D, M, dtype,
                                 args.get("feature", 0), wsp, nb, None)


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
    ws = lib.la_workspace_size(1, 1, 1, 64, 64, 64, 1)
    assert lib.la_forward_noncausal(addr(1), addr(2), addr(3), None, None, None, 1, 1, 64, 64, 64, 1, 0, addr(20), ws, None) == NULL
    assert lib.la_forward_noncausal(addr(1), addr(2), addr(3), addr(4), None, None, 1, 1, 64, 64, 64, 1, 0, None, 0, None) == WORKSPACE
    assert lib.la_forward_noncausal(addr(1), addr(2), addr(3), addr(3), None, None, 1, 1, 64, 64, 64, 1, 0, addr(20), ws,
                                    None) == ALIAS
    # N = 0 is a no-op
    assert lib.la_forward_noncausal(None, None, None, None, None, None, 1, 1, 0, 64, 64, 1, 0, None, 0, None) == OK
    wsb = lib.la_workspace_size(2, 2, 2, 100, 32, 32, 0)
    names = ["Q", "K", "V", "logA", "O", "den", "dO", "S0", "Z0", "ckpt", "dS_N", "dZ_N", "dQ", "dK", "dV", "dlogA",
             "dS0", "dZ0"]
    base = dict(Q=addr(1), K=addr(2), V=addr(3), O=addr(4), den=addr(5), dO=addr(6), dQ=addr(7), dK=addr(8),
                dV=addr(9))

    def bwd(N=100, ws=addr(20), nb=wsb, **over):
        a = dict(base)
        a.update(over)
        return lib.la_backward_causal(*[a.get(n) for n in names], 2, 2, N, 32, 32, 0, a.get("feature", 0), ws, nb, None)

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
    wsd = lib.la_workspace_size(6, 2, 2, 100, 32, 32, 0)
    assert wsd > wsb
    assert bwd(logA=addr(14), dlogA=addr(15), nb=wsb) == WORKSPACE
    assert bwd(logA=addr(14), dlogA=addr(14), nb=wsd) == ALIAS
    assert bwd(logA=ctypes.c_void_p(BASE + 14 * (1 << 32) + 4), dlogA=addr(15), nb=wsd) == ALIGN


def test_feature_argument_validation(lib):
    assert fwd(lib, feature=2) == ARG
    assert fwd(lib, feature=-1) == ARG
    assert b"feature" in lib.la_last_error()
    assert lib.la_decode_step(addr(1), addr(2), addr(3), None, addr(4), addr(5), addr(6), 2, 2, 64, 64, 1, 5,
                              None) == ARG


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
    need = lib.la_workspace_size(5, 2, 2, 100, 32, 32, 0)  # the decayed forward's workspace
    assert need > 0
    assert fwd(lib, logA=addr(14), ws_bytes=need - 1) == WORKSPACE
    assert fwd(lib, logA=addr(4)) == ALIAS  # O on top of logA
    assert fwd(lib, logA=ctypes.c_void_p(BASE + 14 * (1 << 32) + 8)) == ALIGN


def test_noncausal_backward_validation(lib):
    ws = lib.la_workspace_size(4, 2, 2, 100, 32, 32, 0)
    assert ws > 0
    args = [addr(1), addr(2), addr(3), addr(4), None, None, addr(5), addr(6), addr(7)]
    a = list(args)
    a[6] = None
    assert lib.la_backward_noncausal(*a, 2, 2, 100, 32, 32, 0, 0, addr(20), ws, None) == NULL
    a = list(args)
    a[7] = addr(1)  # dK on top of Q
    assert lib.la_backward_noncausal(*a, 2, 2, 100, 32, 32, 0, 0, addr(20), ws, None) == ALIAS
    assert lib.la_backward_noncausal(*args, 2, 2, 100, 32, 32, 0, 0, addr(20), ws - 1, None) == WORKSPACE
    assert lib.la_backward_noncausal(*args, 2, 2, 100, 48, 32, 0, 0, addr(20), ws, None) == UNSUPPORTED
    assert lib.la_backward_noncausal(*args, 2, 2, 0, 32, 32, 0, 0, None, 0, None) == OK
    a = list(args)
    a[4] = addr(8)  # S_tot without Z_tot
    assert lib.la_backward_noncausal(*a, 2, 2, 100, 32, 32, 0, 0, addr(20), ws, None) == ARG
    a[5] = addr(9)
    a[6] = addr(8)  # dQ on top of S_tot
    assert lib.la_backward_noncausal(*a, 2, 2, 100, 32, 32, 0, 0, addr(20), ws, None) == ALIAS
    assert lib.la_forward_noncausal(addr(1), addr(2), addr(3), addr(4), addr(5), None, 2, 2, 100, 32, 32, 0, 0,
                                    addr(20), 1 << 30, None) == ARG


def test_decode_validation(lib):
    assert lib.la_decode_step(addr(1), addr(2), addr(3), None, addr(4), addr(5), None, 2, 2, 64, 64, 1, 0, None) == NULL
    assert lib.la_decode_step(addr(1), addr(2), addr(3), None, addr(4), addr(4), addr(6), 2, 2, 64, 64, 1, 0, None) == ALIAS
    assert lib.la_decode_step(addr(1), addr(2), addr(3), addr(4), addr(4), addr(5), addr(6), 2, 2, 64, 64, 1, 0,
                              None) == ALIAS  # S on top of logA
    assert lib.la_decode_step(addr(1), addr(2), addr(3), None, addr(4), addr(5), addr(6), 2, 2, 16, 64, 1, 0,
                              None) == UNSUPPORTED
    assert lib.la_decode_step(addr(1), addr(2), addr(3), None, addr(4), addr(5), addr(6), 2, 0, 64, 64, 1, 0, None) == SHAPE


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
    assert lib.la_segment_length(B, H, N, D, M) == L
    sv = D * M + D
    assert lib.la_checkpoint_size(B, H, N, D, M) == B * H * (nseg + 1) * sv * 4
    # linear-memory bound: the checkpoint never exceeds B*H*N*max(D,M) floats by more than one state per head
    assert lib.la_checkpoint_size(B, H, N, D, M) <= 4 * B * H * (N * max(D, M) + 2 * sv)
    assert lib.la_workspace_size(3, B, H, N, D, M, 1) == 0
    # forward: segment aggregates, their prefix scan and the one-pass form's error word and per-segment flags
    # (32-bit words) when there is more than one segment
    agg, pref = _al(B * H * nseg * sv * 4), _al(B * H * (nseg + 1) * sv * 4)
    sync = _al((1 + B * H * nseg) * 4)
    assert lib.la_workspace_size(0, B, H, N, D, M, 0) == (0 if nseg == 1 else agg + pref + sync)
    _, nseg_nc = _plan(B, H, N, 512)
    agg_nc, pref_nc = _al(B * H * nseg_nc * sv * 4), _al(B * H * (nseg_nc + 1) * sv * 4)
    assert lib.la_workspace_size(1, B, H, N, D, M, 0) == agg_nc + pref_nc
    # backward: room to recompute the checkpoint, plus reverse aggregates
    bwd = _al(B * H * nseg * sv * 4) + _al(B * H * (nseg + 1) * sv * 4) + (0 if nseg == 1 else _al(B * H * nseg * sv * 4))
    assert lib.la_workspace_size(2, B, H, N, D, M, 0) == bwd
    # non-causal backward: key aggregates + scan, reverse aggregates + scan
    assert lib.la_workspace_size(4, B, H, N, D, M, 0) == 2 * (agg_nc + pref_nc)
    # decayed forward: aggregates, prefix states, per-segment log-decay sums (more than one segment);
    # decayed backward: those, reverse aggregates and (1/den, c) per token
    dl = _al(B * H * nseg_nc * 4)  # the decayed recurrence plans like the non-causal ops
    assert lib.la_workspace_size(5, B, H, N, D, M, 0) == (0 if nseg_nc == 1 else agg_nc + pref_nc + dl)
    assert lib.la_workspace_size(6, B, H, N, D, M, 1) == agg_nc + pref_nc + dl + agg_nc + _al(B * H * N * 8) + dl
    assert lib.la_workspace_size(9, B, H, N, D, M, 0) == 0


def _al(x):
    return (x + 255) // 256 * 256


def test_process_wide_switches(lib):
    """The segment-length override, the forward's form and the one-launch wait limit: valid values are taken and
    the previous one returned; invalid values are refused with -1 and change nothing."""
    assert lib.la_set_segment_chunks(-1) == -1
    prev = lib.la_set_segment_chunks(3)
    try:
        assert lib.la_set_segment_chunks(3) == 3
        assert lib.la_segment_length(2, 2, 1000, 32, 32) == 3 * 64
    finally:
        lib.la_set_segment_chunks(prev)
    for bad in (-1, 3):
        assert lib.la_set_forward_onepass(bad) == -1
    prev = lib.la_set_forward_onepass(2)
    try:
        assert lib.la_set_forward_onepass(0) == 2
    finally:
        lib.la_set_forward_onepass(prev)
    assert lib.la_set_wait_polls(-5) == -1
    prev = lib.la_set_wait_polls(7)
    try:
        assert lib.la_set_wait_polls(prev) == 7
    finally:
        lib.la_set_wait_polls(prev)
    with pytest.raises(ValueError):
        binding.set_forward_onepass(5)
    with pytest.raises(ValueError):
        binding.set_wait_polls(-1)
