"""la_forward_causal_noalloc (the causal forward on the library's static per-GPU scratch, for callers that cannot
allocate) against la_forward_causal with a caller workspace, through the C ABI: two calls in a row on the same
scratch, the second with a smaller input of another shape and form (the first call's aggregates and one-launch
flags are left behind in the scratch), each bit for bit equal to the workspace call and within the tolerance of
the float64 oracle; sizes beyond the scratch are refused before any launch."""
import numpy as np
import pytest
import torch

import oracle
from linear_rnn_layers_amd import binding, inputs
from tests.gpu_util import TOL, dev, host, rowerr

pytestmark = pytest.mark.gpu


def _call_pair(B, H, N, D, M, dtype, seed):
    q = inputs.gaussian((B, H, N, D), seed, 0.5, dtype)
    k = inputs.gaussian((B, H, N, D), seed + 1, 0.5, dtype)
    v = inputs.gaussian((B, H, N, M), seed + 2, 1.0, dtype)
    Q, K, V = dev(q, dtype), dev(k, dtype), dev(v, dtype)
    code = binding.dtype_code(Q.dtype)
    ck_n = binding.checkpoint_size(B, H, N, D, M) // 4
    outs = []
    for noalloc in (True, False):
        O = torch.full((B, H, N, M), float("nan"), dtype=Q.dtype, device="cuda")
        den = torch.full((B, H, N), float("nan"), device="cuda")
        S = torch.full((B, H, D, M), float("nan"), device="cuda")
        Z = torch.full((B, H, D), float("nan"), device="cuda")
        ck = torch.full((ck_n,), float("nan"), device="cuda")
        if noalloc:
            binding.la_forward_causal_noalloc(Q, K, V, O, den, S_out=S, Z_out=Z, ckpt=ck)
        else:
            ws = binding.alloc_workspace(binding.LA_OP_FWD_CAUSAL, B, H, N, D, M, code, "cuda")
            assert binding.workspace_size(binding.LA_OP_FWD_CAUSAL, B, H, N, D, M, code) > 0  # scratch in use
            binding.la_forward_causal(Q, K, V, O, den, S_out=S, Z_out=Z, ckpt=ck, ws=ws)
        torch.cuda.synchronize()
        outs.append([host(t) for t in (O, den, S, Z, ck)])
    a, b = outs
    for x, y in zip(a, b):
        assert np.array_equal(x, y)  # the same kernels on the same plan: identical
    o, d, s, z = oracle.forward_causal(q, k, v)
    assert rowerr(a[0], o) <= TOL[dtype] and rowerr(a[1], d, False) <= TOL[dtype]
    assert rowerr(a[2], s) <= TOL[dtype] and rowerr(a[3], z, False) <= TOL[dtype]


def test_noalloc_forward_matches_workspace_forward():
    binding.load()
    # first call: sixteen segments per head (two-launch form, aggregates summed by every workgroup)
    _call_pair(4, 8, 3072, 32, 32, inputs.BF16, 15000)
    # second call, smaller: D = 64, M = 32, the one-launch form, whose flags the first call did not clear
    _call_pair(2, 2, 700, 64, 32, inputs.F32, 15100)


def test_noalloc_refuses_sizes_beyond_the_scratch():
    import ctypes

    lib = binding.load()
    B, H, N, D, M = 1, 16, 65536, 64, 64
    opts = binding.Options(segment_chunks=1)  # 1024 segments per head: 272 MB of aggregates
    assert binding.workspace_size(binding.LA_OP_FWD_CAUSAL, B, H, N, D, M, binding.LA_BF16, opts) > (24 << 20)
    addr = lambda i: ctypes.c_void_p(0x7F0000000000 + i * (1 << 36))  # noqa: E731  (never dereferenced)
    st = lib.la_forward_causal_noalloc(addr(1), addr(2), addr(3), None, addr(4), None, None, None, None, None, None,
                                       B, H, N, D, M, binding.LA_BF16, 0, None, ctypes.byref(opts))
    assert st == 6, lib.la_last_error()  # LA_ERR_WORKSPACE before any launch
    assert b"static scratch" in lib.la_last_error()
