"""Benchmark of the causal linear attention library on one MI355X.

Headline (no --workload): the 2^16-token sequence of the pages' Figure 1 at
the widths of a 64-wide head, B=1 H=16 N=65536 D=M=64, bf16 storage (inputs
N(0, 1/8^2)), one step = causal forward (phi prologue, intra-chunk blocks,
state carry, epilogue) + causal backward.  The same run measures, as nested
records with their own roofline, the MNIST-shaped layer (B=16 H=8 N=784
D=M=32, float32: causal forward + backward + non-causal forward), the
CIFAR-shaped 16-layer stack (B=4 H=8 N=3072 D=M=32 bf16, sigma 0.5), and the
decode loop (4096 steps of B=256 H=16 D=M=64 after a 512-token prefill; HIP
graphs of 64 steps and one launch per step), a decode run whose state (537 MB)
exceeds the 256 MB last-level cache, the random-feature layer with C = 256
(mnist-rf256), one CIFAR-shaped layer with the degree-2 polynomial map
(cifar-poly2, C = 1088), the 2^16-token sequence with a data-dependent decay
(long-decay) and the 9-layer bidirectional speech encoder (non-causal).
--workload X measures X alone (also mnist-rf and small).

Prints one JSON line.  `value` is whole-job throughput with the inputs
resident in HBM; `roofline` is for the dominant kernel (the largest share of
the step in the committed kernel statistics), its duration taken from HIP
events that the library records on the launch stream around every launch of
that kernel inside the timed region (la_options::timed_kernel with
caller-created events), its bytes the algorithmic bytes of one launch, the
tensors that kernel must read or write over its token-heads (kernel_bytes);
`step_roofline` is the whole step's algorithmic bytes per token-head of each
pass (forward (2D+2M)s+4, backward (4D+4M)s+4, s bytes per element) over the
step time; `side_by_side` carries the HBM fraction, the executed-MFMA
fraction and MFMA-busy (rocprofv3 counters in profiles/, when they were taken
at the current kernel sources) and the useful-flop fraction.  `cpu_baseline`
is the float64 oracle on the host cores on a bounded sample of the headline
workload.  The per-kernel breakdown comes from the rocprofv3 kernel
statistics in profiles/ (per-launch events would inflate every kernel).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix, published
MFMA_FLOPS_PER_INST = 2 * 16 * 16 * 32  # v_mfma_f32_16x16x32_bf16, per wavefront instruction
CLOCK_GHZ = 2.4
SIMDS = 256 * 4
PROFILES = os.path.join(ROOT, "profiles")
HEADLINE = "long"
NESTED = ("mnist", "cifar", "decode", "decode-dram", "mnist-rf256", "cifar-poly2", "long-decay", "speech")
DECODE_GRAPH = 64  # decode steps per captured graph
THREADS = 16  # host threads for input generation (the GPU host's share of cores)

# The kernel with the largest share of a step's GPU time in the rocprofv3 kernel statistics in profiles/
# (dominant_kernel reads them; this table is what they showed, used when no statistics match the sources).
DOMINANT = {"long": "bwd_kv", "mnist": "bwd_kv", "cifar": "bwd_kv", "mnist-rf": "bwd_query",
            "mnist-rf256": "bwd_query", "cifar-poly2": "bwd_query",
            "long-decay": "dbq", "speech": "nc_qr", "decode": "decode", "decode-dram": "decode",
            "small": "fwd_causal"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default 50; decode: 4096)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed warm-up steps (default 10; decode: 256)")
    ap.add_argument("--workload", default=None,
                    choices=["mnist", "cifar", "long", "long-decay", "mnist-rf", "mnist-rf256", "cifar-poly2",
                             "speech", "decode", "decode-dram", "small"],
                    help="measure this workload alone (default: the headline plus the nested records)")
    ap.add_argument("--no-nested", action="store_true", help="headline only")
    ap.add_argument("--segment-chunks", type=int, default=0,
                    help="force the segment length of every call (64-token chunks; 0 = the library's plan)")
    ap.add_argument("--profile-run", action="store_true",
                    help="run exactly warm-up + timed steps of one workload and nothing else (for rocprofv3: "
                         "launches per step = calls / (warm-up + steps))")
    ap.add_argument("--steps-profiled", type=int, default=0,
                    help="--summarize-stats: the steps the profiled run executed (warm-up + timed)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true", help="skip the sampled parity check of the headline")
    ap.add_argument("--no-kernel-events", action="store_true", help="time without per-kernel events")
    ap.add_argument("--eager-decode", action="store_true",
                    help="decode: one host launch per step instead of replaying captured graphs of 64 steps")
    ap.add_argument("--seq-sweep", action="store_true",
                    help="causal forward + backward time and peak memory per sample for N = 2^9 .. 2^16 with the batch "
                         "scaled inversely (B*N = 65536; H=16, D=M=64, bf16), one JSON line")
    ap.add_argument("--copy-only", type=int, default=0, metavar="MiB",
                    help="only run a plain device copy of this size (traffic-counter calibration)")
    ap.add_argument("--summarize-stats", metavar="CSV", help="write profiles/<label>_kernels.md/.json from a "
                    "rocprofv3 --kernel-trace --stats kernel_stats.csv")
    ap.add_argument("--summarize-traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="write profiles/<label>_traffic.md and traffic_<kernel>_<label>.json from rocprofv3 --pmc CSVs")
    ap.add_argument("--summarize-mfma", nargs=2, metavar=("PMC_CSV", "STATS_CSV"),
                    help="write profiles/<label>_mfma.md/.json from a --pmc SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES ... "
                         "run and the kernel statistics of a --kernel-trace --stats run")
    ap.add_argument("--label", default=HEADLINE)
    ap.add_argument("--command", default="", help="the command that produced the CSVs (recorded in the summary)")
    return ap.parse_args()


def default_steps(wl):
    return {"decode": (4096, 256), "decode-dram": (256, 64), "cifar": (20, 5)}.get(wl, (50, 10))


# ------------------------------------------------------------------ inputs
def _parallel(fn, items, threads=THREADS):
    """Map fn over items on host threads (numpy's generators release the interpreter lock while drawing)."""
    from concurrent.futures import ThreadPoolExecutor

    with ThreadPoolExecutor(threads) as ex:
        return list(ex.map(fn, items))


def WORKLOADS(inputs):
    dram = inputs.Workload("decode-dram-b2048h16d64-256steps-bf16", 2048, 16, 64, 64, 64, inputs.BF16, 1.0,
                           (511, 512, 513, 514), steps=256)
    return {"mnist": inputs.MNIST, "cifar": inputs.CIFAR, "long": inputs.LONG, "speech": inputs.SPEECH,
            "long-decay": inputs.LONG_DECAY, "mnist-rf": inputs.MNIST_RF, "mnist-rf256": inputs.MNIST_RF256,
            "cifar-poly2": inputs.CIFAR_POLY2, "decode": inputs.DECODE,
            "decode-dram": dram, "small": inputs.SMALL}


class Step:
    """One workload: inputs resident in HBM, outputs and workspaces preallocated, one callable per step.  The
    options of every call carry a KernelTimer when the dominant kernel is being timed."""

    def __init__(self, wl, timed_kernel=None, pairs=8192, eager_decode=False, segment_chunks=0):
        import torch

        from linear_rnn_layers_amd import binding, inputs

        self.torch, self.b, self.inputs = torch, binding, inputs
        self.wl = wl
        self.w = w = WORKLOADS(inputs)[wl]
        self.dt = dt = torch.float32 if w.dtype == inputs.F32 else torch.bfloat16
        self.timer = binding.KernelTimer(timed_kernel, pairs) if timed_kernel else None
        self.opts = (binding.options(timer=self.timer, segment_chunks=segment_chunks)
                     if self.timer or segment_chunks else None)
        so = self.opts
        self.graphs = []
        if wl.startswith("decode"):
            self._init_decode(eager_decode)
            return
        B, H, N, D, M = w.B, w.H, w.N, w.D, w.M
        code = binding.dtype_code(dt)
        if wl in ("cifar", "speech"):
            specs = [("layer", i) for i in range(w.layers)]  # one independent input set per layer
        elif wl in ("mnist", "mnist-rf", "mnist-rf256"):
            specs = [("set", i) for i in range(6)]  # rotate batches so successive steps miss the 256 MB cache
        elif wl in ("long", "long-decay"):
            # 512 MB per set: one set already exceeds the cache, but the first chunks a step reads would still
            # be there from the end of the step before
            specs = [("set", i) for i in range(2)]
        else:
            specs = [("set", 0)]
        arrays = _parallel(lambda a: self._draw(*a), [(sp, t) for sp in specs for t in range(4)])
        self.sets = []
        for i in range(len(specs)):
            self.sets.append(tuple(self._dev(arrays[4 * i + t]) for t in range(4)))
        del arrays
        self.o = torch.empty((B, H, N, M), dtype=dt, device="cuda")
        self.onc = torch.empty((B, H, N, M), dtype=dt, device="cuda")
        self.den = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        self.dq = torch.empty((B, H, N, D), dtype=dt, device="cuda")
        self.dk = torch.empty((B, H, N, D), dtype=dt, device="cuda")
        self.dv = torch.empty((B, H, N, M), dtype=dt, device="cuda")
        Dk = w.features or D  # the attention's feature size
        self.ck = torch.empty(binding.checkpoint_size(B, H, N, Dk, M, so) // 4, dtype=torch.float32, device="cuda")
        fwd_op = binding.LA_OP_FWD_DECAY if wl == "long-decay" else binding.LA_OP_FWD_CAUSAL
        bwd_op = binding.LA_OP_BWD_DECAY if wl == "long-decay" else binding.LA_OP_BWD_CAUSAL
        self.ws_f = binding.alloc_workspace(fwd_op, B, H, N, Dk, M, code, "cuda", so)
        self.ws_b = binding.alloc_workspace(bwd_op, B, H, N, Dk, M, code, "cuda", so)
        self.ws_n = binding.alloc_workspace(binding.LA_OP_FWD_NONCAUSAL, B, H, N, D, M, code, "cuda", so)
        if wl == "speech":
            self.ws_nb = binding.alloc_workspace(binding.LA_OP_BWD_NONCAUSAL, B, H, N, D, M, code, "cuda", so)
            self.s_tot = torch.empty((B, H, D, M), dtype=torch.float32, device="cuda")
            self.z_tot = torch.empty((B, H, D), dtype=torch.float32, device="cuda")
        if w.features:  # the feature vectors of Q, K and their gradients (feature-sliced when C > 64)
            fs = binding.feature_shape(B, H, N, w.features)
            if w.fmap == "random":
                self.W = torch.from_numpy(w.projection()).to("cuda").contiguous()
            self.fq = torch.empty(fs, dtype=dt, device="cuda")
            self.fk = torch.empty(fs, dtype=dt, device="cuda")
            self.dfq = torch.empty(fs, dtype=dt, device="cuda")
            self.dfk = torch.empty(fs, dtype=dt, device="cuda")
        if wl == "long-decay":
            self.log_a = torch.from_numpy(w.log_a()).to("cuda").contiguous()
            self.dla = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        self.i = 0

    def _dev(self, a):
        import numpy as np

        t = self.torch.from_numpy(a)
        if a.dtype == np.uint16:
            return t.view(self.torch.bfloat16).to("cuda").contiguous()
        return t.to("cuda").to(self.dt).contiguous()

    def _draw(self, spec, t):
        """Array t (Q, K, V, dO) of an input set: layer i of a stack, or set i of a rotation (seed offset 100000 i;
        set 0 is the workload's own seeds)."""
        w, inputs = self.w, self.inputs
        kind, i = spec
        if kind == "layer":
            seed = w.layer_seeds(i)[t]
        else:
            seed = w.seeds[t] + 100_000 * i
        width = w.D if t < 2 else w.M
        sigma = w.sigma if t < 3 else 1.0
        shape = (w.B, w.H, w.N, width)
        if w.dtype == inputs.BF16:
            return inputs.gaussian_bf16_bits(shape, seed, sigma)
        return inputs.gaussian(shape, seed, sigma, w.dtype)

    def _init_decode(self, eager):
        import ctypes

        import numpy as np

        torch, b, w = self.torch, self.b, self.w
        B, H, D, M = w.B, w.H, w.D, w.M
        pool = w.steps
        dram = self.wl == "decode-dram"
        # prefill: a 512-token (64-token for the cache-exceeding run) causal forward, whose final state starts
        # the loop (seeded numpy recipe, the workload's seeds)
        q, k, v = (self._dev(inputs_bits) for inputs_bits in _parallel(
            lambda t: self.inputs.gaussian_bf16_bits((B, H, w.N, D if t < 2 else M), w.seeds[t], 1.0), range(3)))
        out = b.forward_causal(q, k, v, return_state=True, checkpoint=False)
        self.S, self.Z = out["s"], out["z"]
        del q, k, v, out
        # per-step q, k, v of every step: seeds base + 3 step + {0, 1, 2}, uploaded before timing
        base = 6_000_000 if dram else 5_000_000
        self.pool_q = torch.empty((pool, B, H, D), dtype=torch.bfloat16, device="cuda")
        self.pool_k = torch.empty((pool, B, H, D), dtype=torch.bfloat16, device="cuda")
        self.pool_v = torch.empty((pool, B, H, M), dtype=torch.bfloat16, device="cuda")
        chunk = 256
        for s0 in range(0, pool, chunk):
            steps = list(range(s0, min(pool, s0 + chunk)))
            trip = _parallel(lambda s: w.decode_step_bits(s, base), steps)
            for j, dst in enumerate((self.pool_q, self.pool_k, self.pool_v)):
                host = np.stack([t[j] for t in trip])
                dst[s0:s0 + len(steps)].copy_(torch.from_numpy(host).view(torch.bfloat16))
            del trip
        self.y = torch.empty((B, H, M), dtype=torch.bfloat16, device="cuda")
        lib = b.load()
        self._call = lib.la_decode_step
        code = b.dtype_code(torch.bfloat16)
        qs, ks, vs = self.pool_q.stride(0) * 2, self.pool_k.stride(0) * 2, self.pool_v.stride(0) * 2
        opt = b._opt(self.opts)
        self._args = [(ctypes.c_void_p(self.pool_q.data_ptr() + i * qs), ctypes.c_void_p(self.pool_k.data_ptr() + i * ks),
                       ctypes.c_void_p(self.pool_v.data_ptr() + i * vs), None, ctypes.c_void_p(self.S.data_ptr()),
                       ctypes.c_void_p(self.Z.data_ptr()), ctypes.c_void_p(self.y.data_ptr()), B, H, D, M, code, 0)
                      for i in range(pool)]
        self._opt = opt
        self.i = 0
        # A decode loop issues one small launch per step, so the host's launch cost shows between steps; a serving
        # loop captures its steps in HIP graphs.  Graph g replays steps 64 g .. 64 g + 63 of the pool (64 launches
        # back to back; the captured calls are the same C-ABI entry point on torch's capture stream).
        if not eager:
            for g0 in range(0, pool, DECODE_GRAPH):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    cs = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
                    for a in self._args[g0:g0 + DECODE_GRAPH]:
                        st = self._call(*a, cs, None)
                        if st != 0:
                            raise b.LAError(st, "la_decode_step")
                self.graphs.append(g)
            torch.cuda.synchronize()
        self.gi = 0

    def run(self, n, events=None):
        """n steps: whole graphs of DECODE_GRAPH decode steps where captured (events: a list that receives a
        (start, end) pair of timing events around every replay), the rest one launch at a time."""
        if self.graphs:
            torch = self.torch
            for _ in range(n // DECODE_GRAPH):
                g = self.graphs[self.gi % len(self.graphs)]
                self.gi += 1
                if events is not None:
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    g.replay()
                    e1.record()
                    events.append((e0, e1))
                else:
                    g.replay()
            n %= DECODE_GRAPH
        for _ in range(n):
            self()

    def __call__(self):
        wl, b, o = self.wl, self.b, self.opts
        if wl.startswith("decode"):
            a = self._args[self.i % len(self._args)]
            self.i += 1
            st = self._call(*a, b._stream(None), self._opt)
            if st != 0:
                raise b.LAError(st, "la_decode_step")
            return
        if wl == "cifar":
            for (q, k, v, do) in self.sets:
                self._fwd_bwd(q, k, v, do)
            return
        if wl == "speech":  # the forward's totals go to the backward, as a training step passes them
            for (q, k, v, do) in self.sets:
                b.la_forward_noncausal(q, k, v, self.onc, ws=self.ws_n, S_out=self.s_tot, Z_out=self.z_tot, opts=o)
                b.la_backward_noncausal(q, k, v, do, self.dq, self.dk, self.dv, ws=self.ws_nb, S_tot=self.s_tot,
                                        Z_tot=self.z_tot, opts=o)
            return
        if self.w.features:
            q, k, v, do = self.sets[self.i % len(self.sets)]
            self.i += 1
            self._features_step(q, k, v, do)
            return
        if wl == "long-decay":
            q, k, v, do = self.sets[self.i % len(self.sets)]
            self.i += 1
            b.la_forward_causal(q, k, v, self.o, self.den, ckpt=self.ck, ws=self.ws_f, logA=self.log_a, opts=o)
            b.la_backward_causal(q, k, v, self.o, self.den, do, self.dq, self.dk, self.dv, ckpt=self.ck,
                                 ws=self.ws_b, logA=self.log_a, dlogA=self.dla, opts=o)
            return
        q, k, v, do = self.sets[self.i % len(self.sets)]
        self.i += 1
        if wl == "small":
            b.la_forward_causal(q, k, v, self.o, self.den, ws=self.ws_f, opts=o)
            return
        self._fwd_bwd(q, k, v, do)
        if wl == "mnist":
            b.la_forward_noncausal(q, k, v, self.onc, ws=self.ws_n, opts=o)

    def _features_step(self, q, k, v, do):
        """The feature map of Q and K, the causal attention on the features (checkpointed forward, backward), the
        chain rule back through the map."""
        b, o, w = self.b, self.opts, self.w
        IDENT = b.LA_FEATURE_IDENTITY
        lib, st = b.load(), b._stream(None)
        B, H, N, D, C = w.B, w.H, w.N, w.D, w.features
        code = b.dtype_code(self.dt)
        for x, f in ((q, self.fq), (k, self.fk)):
            if w.fmap == "random":
                b._check(lib.la_feature_random(b._ptr(x), b._ptr(self.W), b._ptr(f), B, H, N, D, C, code, st),
                         "la_feature_random")
            else:
                b._check(lib.la_feature_poly2(b._ptr(x), b._ptr(f), B, H, N, D, C, code, st), "la_feature_poly2")
        b.la_forward_causal(self.fq, self.fk, v, self.o, self.den, ckpt=self.ck, ws=self.ws_f, feature=IDENT, opts=o)
        b.la_backward_causal(self.fq, self.fk, v, self.o, self.den, do, self.dfq, self.dfk, self.dv, ckpt=self.ck,
                             ws=self.ws_b, feature=IDENT, opts=o)
        for x, g, dx in ((q, self.dfq, self.dq), (k, self.dfk, self.dk)):
            if w.fmap == "random":
                b._check(lib.la_feature_random_vjp(b._ptr(x), b._ptr(self.W), b._ptr(g), b._ptr(dx), B, H, N, D, C,
                                                   code, st), "la_feature_random_vjp")
            else:
                b._check(lib.la_feature_poly2_vjp(b._ptr(x), b._ptr(g), b._ptr(dx), B, H, N, D, C, code, st),
                         "la_feature_poly2_vjp")

    def _fwd_bwd(self, q, k, v, do):
        b, o = self.b, self.opts
        b.la_forward_causal(q, k, v, self.o, self.den, ckpt=self.ck, ws=self.ws_f, opts=o)
        b.la_backward_causal(q, k, v, self.o, self.den, do, self.dq, self.dk, self.dv, ckpt=self.ck, ws=self.ws_b,
                             opts=o)


# ---------------------------------------------------- algorithmic figures
def pass_bytes(w, s):
    """Algorithmic bytes per token-head of each pass: forward (2D+2M)s+4 (read Q, K, V; write O,
    den), backward (4D+4M)s+4 (read Q, K, V, O, dO, den; write dQ, dK, dV), non-causal forward (2D+2M)s (read
    Q, K, V; write O).  With random features the attention sees C-wide feature vectors in place of D."""
    D, M = w.features or w.D, w.M
    return {"fwd": (2 * D + 2 * M) * s + 4, "bwd": (4 * D + 4 * M) * s + 4, "fwd_nc": (2 * D + 2 * M) * s}


def pass_flops(w):
    """Useful flops per token-head (recurrent form): forward 4DM+5D+M, backward 10DM+9D+3M."""
    D, M = w.features or w.D, w.M
    return {"fwd": 4 * D * M + 5 * D + M, "bwd": 10 * D * M + 9 * D + 3 * M, "fwd_nc": 4 * D * M + 5 * D + M}


def decode_step_bytes(w, s):
    """One decode step of all heads: read and write S and Z (float32), read q, k, v and write y."""
    D, M = w.D, w.M
    return w.B * w.H * (2 * D * M * 4 + 2 * D * 4 + (2 * D + 2 * M) * s)


def step_work(wl, w, s):
    """(algorithmic bytes, useful flops) of one step."""
    if wl.startswith("decode"):
        D, M = w.D, w.M
        return decode_step_bytes(w, s), w.B * w.H * (4 * D * M + 5 * D + M)
    th = w.B * w.H * w.N * max(1, w.layers)
    pb, pf = pass_bytes(w, s), pass_flops(w)
    passes = {"mnist": ("fwd", "bwd", "fwd_nc"), "small": ("fwd",), "speech": ("fwd_nc", "bwd")}.get(
        wl, ("fwd", "bwd"))
    byts = th * sum(pb[p] for p in passes)
    if w.features:  # the map of Q and K (read X, write Phi) and its chain rule (read X and dPhi, write dX)
        byts += th * 2 * ((w.D + w.features) + (2 * w.D + w.features)) * s
    if wl == "speech":  # non-causal backward reads Q, K, V, dO and writes dQ, dK, dV
        D, M = w.D, w.M
        byts = th * (pb["fwd_nc"] + (4 * D + 3 * M) * s)
    return byts, th * sum(pf[p] for p in passes)


def kernel_bytes(name, w, s):
    """Algorithmic HBM bytes per launch of a kernel: the bytes of the tensors it must read or write by its
    function (the split of the per-pass totals over the kernels that do the work).  Used for the traffic
    tables and, for the dominant kernel, the roofline (dominant_bytes)."""
    Din, M = w.D, w.M
    D = w.features or Din
    th = w.B * w.H * w.N
    per_th = {
        "fwd_causal": (2 * D + 2 * M) * s + 4,   # read Q, K, V; write O, den
        "seg_state": (D + M) * s,                # read K, V
        "fwd_noncausal": (2 * D + 2 * M) * s,    # read Q, K, V; write O
        "bwd_query": (3 * D + 2 * M) * s,        # read Q, K, V, dO; write dQ
        "bwd_kv": (3 * D + 3 * M) * s,           # read Q, K, V, dO; write dK, dV
        "nc_qr": (2 * D + M) * s,                # read Q, dO; write dQ
        "nc_kv": (2 * D + 2 * M) * s,            # read K, V; write dK, dV
        "dseg_state": (D + M) * s + 4,           # read K, V, logA
        "dfwd": (2 * D + 2 * M) * s + 8,         # read Q, K, V, logA; write O, den
        "dbq": (3 * D + 2 * M) * s + 4,          # read Q, K, V, dO, logA; write dQ
        "dbkv": (3 * D + 3 * M) * s + 8,         # read Q, K, V, dO, logA; write dK, dV, dlogA terms
        "dla_fix": 8,                            # read and write dlogA
        "feat_rf": (Din + D) * s,                # read X; write Phi
        "feat_rf_vjp": (2 * Din + D) * s,        # read X, dPhi; write dX
        "feat_rf_vjp_wide": (2 * Din + D) * s,   # read X, dPhi; write dX
        "feat_poly2": (Din + D) * s,             # read X; write Phi
        "feat_poly2_wide": (Din + D) * s,        # read X; write Phi
        "feat_poly2_vjp": (2 * Din + D) * s,     # read X, dPhi; write dX
        "feat_poly2_vjp_wide": (2 * Din + D) * s,  # read X, dPhi; write dX
    }
    ns = D // 64 if D > 64 else 1
    per_th.update({  # wide feature vectors: the sums over the ns slices (shares written by the slice kernels)
        "wide_combine": ns * (M + 1) * 4 + M * s + 4,  # read the shares; write O, den
        "bwd_query_shares": (2 * D + 2 * M) * s,  # read Q, K, V, dO (shares of num.dO, den: ns * 8 written)
        "wide_pairs": ns * 8 + 8,                # read the shares; write (1/den, O.dO)
        "wide_sum": ns * M * 4 + M * s,          # read dV shares; write dV
    })
    if name == "decode":
        return decode_step_bytes(w, s)
    if name in per_th:
        return th * per_th[name]
    return None


def dominant_bytes(wl, name, w, s):
    """Algorithmic bytes per launch for the roofline of the dominant kernel: the tensors it must read or write by
    its function (kernel_bytes); the per-token pair (1/den, O.dO), or (1/den, c) with a decay, that the backward's
    query pass hands to its key pass (8 bytes per token-head each way) is an intermediate of this implementation
    and is not counted."""
    return kernel_bytes(name, w, s)


def source_hash():
    h = hashlib.sha256()
    for f in ("la_device.h", "la_kernels.h", "la_decay.h", "la_feature.h", "la_bwd2.h", "la_wide.h", "la_api.hip"):
        with open(os.path.join(ROOT, "linear_rnn_layers_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _profile_json(name):
    path = os.path.join(PROFILES, name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    return rec if rec.get("source_hash") == source_hash() else None


def dominant_kernel(wl):
    """The kernel with the largest total time per step in the committed rocprofv3 statistics of this workload
    (profiles/<workload>_kernels.json, when taken at the current kernel sources), else the DOMINANT table."""
    ks = _profile_json(f"{wl}_kernels.json")
    if ks and ks.get("kernels"):
        return max(ks["kernels"], key=lambda k: ks["kernels"][k]["total_us"])
    return DOMINANT[wl]


def traffic_from_profiles(kernel, label):
    """HBM bytes per launch from committed counter summaries, if they were taken at the current kernels."""
    rec = _profile_json(f"traffic_{kernel}_{label}.json")
    return rec.get("bytes_per_launch") if rec else None


# ------------------------------------------------------ profile summaries
KERNEL_TAGS = (("k_bkv<", "bwd_kv"), ("k_bq<", "bwd_query"), ("k_seg_state<", "seg_state"),
               ("k_scan_states<", "scan_states"), ("k_scan_rev<", "scan_rev"), ("k_decode<", "decode"),
               ("k_nc_qr<", "nc_qr"), ("k_nc_kv<", "nc_kv"), ("k_dseg_state<", "dseg_state"),
               ("k_dscan_states<", "dscan_states"), ("k_dfwd<", "dfwd"), ("k_dbq<", "dbq"),
               ("k_dscan_rev<", "dscan_rev"), ("k_dbkv<", "dbkv"), ("k_dla_fix", "dla_fix"),
               ("k_feat_rf_vjp<", "feat_rf_vjp"), ("k_feat_rf<", "feat_rf"), ("k_state_copy<", "state_copy"),
               ("k_wide_combine<", "wide_combine"), ("k_wide_pairs", "wide_pairs"), ("k_wide_sum<", "wide_sum"),
               ("k_decode_wide<", "decode_wide"), ("k_feat_rf_vjp_wide<", "feat_rf_vjp_wide"),
               ("k_feat_poly2_vjp_wide<", "feat_poly2_vjp_wide"), ("k_feat_poly2_wide<", "feat_poly2_wide"),
               ("k_feat_poly2_vjp<", "feat_poly2_vjp"), ("k_feat_poly2<", "feat_poly2"))


def _template_args(full_name, kernel):
    """Template arguments of `kernel<...>` in a demangled name, as strings."""
    inner = full_name.split(kernel + "<", 1)[1].split(">", 1)[0]
    return [a.strip() for a in inner.split(",")]


def kernel_tag(full_name):
    """The library's launch name (la_kernel_names) of a demangled kernel name."""
    if "k_fwd_lb<" in full_name:  # the one-launch causal forward
        return "fwd_causal"
    if "k_sync_clear" in full_name:
        return "sync_clear"
    if "k_fwd<" in full_name:  # k_fwd<T, D, M, CAUSAL, PART>
        return "fwd_causal" if _template_args(full_name, "k_fwd")[3] == "true" else "fwd_noncausal"
    if "k_bq<" in full_name and _template_args(full_name, "k_bq")[3] == "2":  # kBqShares
        return "bwd_query_shares"
    if "k_nc_qr<" in full_name and _template_args(full_name, "k_nc_qr")[3] == "2":  # kNcShares
        return "nc_qr_shares"
    for key, tag in KERNEL_TAGS:
        if key in full_name:
            return tag
    return full_name.split("(")[0][:60]


def summarize_stats(args):
    """profiles/<label>_kernels.md (and .json: average duration and calls per kernel) from rocprofv3 kernel
    statistics."""
    import csv

    rows = list(csv.DictReader(open(args.summarize_stats)))
    os.makedirs(PROFILES, exist_ok=True)
    path = os.path.join(PROFILES, f"{args.label}_kernels.md")
    rec = {"workload": args.label, "source_hash": source_hash(), "command": args.command,
           "steps_profiled": args.steps_profiled or None, "kernels": {}}
    with open(path, "w") as f:
        f.write(f"# rocprofv3 kernel statistics: {args.label} workload\n\n")
        f.write(f"Command (run from the repository root on one MI355X):\n\n    {args.command}\n\n")
        f.write(f"Kernel sources: sha256[:16] = {source_hash()}\n\n")
        f.write("| kernel | template | calls | average us | min us | max us | share of GPU time |\n"
                "|---|---|---|---|---|---|---|\n")
        for r in rows:
            name = r["Name"]
            tmpl = name.split("(")[0].replace("void ", "")
            tag = kernel_tag(name)
            f.write(f"| {tag} | `{tmpl}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                    f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |\n")
            if "la::" in name:
                k = rec["kernels"].setdefault(tag, {"calls": 0, "total_us": 0.0})
                k["calls"] += int(r["Calls"])
                k["total_us"] += float(r["AverageNs"]) / 1e3 * int(r["Calls"])
    for k in rec["kernels"].values():
        k["average_us"] = k["total_us"] / k["calls"]
    with open(os.path.join(PROFILES, f"{args.label}_kernels.json"), "w") as f:
        json.dump(rec, f, indent=1)
    print(path)


def _counter_means(path, counter):
    import csv

    per = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in per.items()}, {k: len(v) for k, v in per.items()}


def summarize_traffic(args):
    fetch_csv, write_csv, cfetch_csv, cwrite_csv = args.summarize_traffic
    fetch, nf = _counter_means(fetch_csv, "FETCH_SIZE")
    write, _ = _counter_means(write_csv, "WRITE_SIZE")
    cf, _ = _counter_means(cfetch_csv, "FETCH_SIZE")
    cw, _ = _counter_means(cwrite_csv, "WRITE_SIZE")
    copy_key = [k for k in cf if "copyBuffer" in k][0]
    copy_bytes = 1024 * (1 << 20)  # bench.py --copy-only 1024: 1 GiB read and 1 GiB written per launch
    f_read = copy_bytes / (cf[copy_key] * 1024.0)
    f_write = copy_bytes / (cw[copy_key] * 1024.0)
    from linear_rnn_layers_amd import inputs

    w = WORKLOADS(inputs)[args.label]
    s = 4 if w.dtype == "f32" else 2
    os.makedirs(PROFILES, exist_ok=True)
    md = os.path.join(PROFILES, f"{args.label}_traffic.md")
    with open(md, "w") as f:
        f.write(f"# HBM traffic per launch from rocprofv3 counters: {args.label} workload\n\n")
        f.write(f"Commands (run from the repository root on one MI355X):\n\n    {args.command}\n\n")
        f.write(f"Kernel sources: sha256[:16] = {source_hash()}\n\n")
        f.write(f"Calibration with a plain 1 GiB device copy (bench.py --copy-only 1024): FETCH_SIZE reads "
                f"{cf[copy_key]:.0f} KiB and WRITE_SIZE {cw[copy_key]:.0f} KiB per copy, so bytes = "
                f"FETCH_SIZE x 1024 x {f_read:.4f} and WRITE_SIZE x 1024 x {f_write:.4f}.\n\n")
        f.write("| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes/launch (scaled) | algorithmic bytes "
                "(the kernel's own tensors) | ratio |\n")
        f.write("|---|---|---|---|---|---|---|\n")
        for k in sorted(fetch, key=lambda x: -fetch[x]):
            tag = kernel_tag(k)
            if "la::" not in k:
                continue
            byts = fetch[k] * 1024 * f_read + write.get(k, 0.0) * 1024 * f_write
            alg = kernel_bytes(tag, w, s)
            ratio = f"{byts / alg:.2f}" if alg else "-"
            f.write(f"| {tag} | {nf[k]} | {fetch[k]:.0f} | {write.get(k, 0.0):.0f} | {byts:.4g} | "
                    f"{alg if alg else '-'} | {ratio} |\n")
            rec = {"kernel": tag, "workload": args.label, "source_hash": source_hash(), "bytes_per_launch": byts,
                   "fetch_kib": fetch[k], "write_kib": write.get(k, 0.0), "read_scale": f_read,
                   "write_scale": f_write, "algorithmic_bytes": alg, "command": args.command}
            with open(os.path.join(PROFILES, f"traffic_{tag}_{args.label}.json"), "w") as fj:
                json.dump(rec, fj, indent=1)
    print(md)


def summarize_mfma(args):
    """Executed MFMA work per kernel (counters) against its duration (kernel statistics)."""
    import csv

    pmc_csv, stats_csv = args.summarize_mfma
    inst, n = _counter_means(pmc_csv, "SQ_INSTS_MFMA")
    busy, _ = _counter_means(pmc_csv, "SQ_VALU_MFMA_BUSY_CYCLES")
    valu, _ = _counter_means(pmc_csv, "SQ_INSTS_VALU")
    dur = {}
    for r in csv.DictReader(open(stats_csv)):
        dur[kernel_tag(r["Name"])] = float(r["AverageNs"]) * 1e-9
    md = os.path.join(PROFILES, f"{args.label}_mfma.md")
    rec = {"workload": args.label, "source_hash": source_hash(), "command": args.command, "kernels": {}}
    with open(md, "w") as f:
        f.write(f"# MFMA utilisation from rocprofv3 counters: {args.label} workload\n\n")
        f.write(f"Commands (run from the repository root on one MI355X):\n\n    {args.command}\n\n")
        f.write(f"Kernel sources: sha256[:16] = {source_hash()}\n\n")
        f.write("Executed MFMA flops = SQ_INSTS_MFMA x 16384 (every matrix instruction is v_mfma_f32_16x16x32_bf16, "
                "split-precision products included) over the kernel's average duration from the kernel statistics; "
                f"MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (duration x {CLOCK_GHZ} GHz x {SIMDS} SIMDs). "
                f"Peak: {MFMA_BF16_PEAK_TFLOPS:.0f} TFLOP/s dense bf16.\n\n")
        f.write("| kernel | dispatches | SQ_INSTS_MFMA | SQ_INSTS_VALU | VALU per MFMA | avg us | executed MFMA TFLOP/s "
                "| of bf16 peak | MFMA busy |\n|---|---|---|---|---|---|---|---|---|\n")
        for k in sorted(inst, key=lambda x: -inst[x]):
            tag = kernel_tag(k)
            if "la::" not in k or tag not in dur:
                continue
            t = dur[tag]
            ex = inst[k] * MFMA_FLOPS_PER_INST / t / 1e12
            b = busy.get(k, 0.0) / (t * CLOCK_GHZ * 1e9 * SIMDS)
            ratio = f"{valu.get(k, 0.0) / inst[k]:.1f}" if inst[k] else "-"
            f.write(f"| {tag} | {n[k]} | {inst[k]:.4g} | {valu.get(k, 0.0):.4g} | {ratio} | {t * 1e6:.1f} | "
                    f"{ex:.1f} | {ex / MFMA_BF16_PEAK_TFLOPS * 100:.1f}% | {b * 100:.1f}% |\n")
            rec["kernels"][tag] = {"mfma_insts_per_launch": inst[k], "valu_insts_per_launch": valu.get(k, 0.0),
                                   "mfma_busy_cycles_per_launch": busy.get(k, 0.0), "average_us": t * 1e6}
    with open(os.path.join(PROFILES, f"{args.label}_mfma.json"), "w") as f:
        json.dump(rec, f, indent=1)
    print(md)


def copy_bandwidth():
    """Achievable streaming bandwidth on this GPU: a plain 512 MiB device-to-device copy, GB/s of bytes
    read + written (best of 10)."""
    import torch

    n = (512 << 20) // 4
    a = torch.ones(n, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    best = None
    for _ in range(10):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        e1.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    del a, b
    return 2 * n * 4 / (best * 1e-3) / 1e9


def step_distribution(step, n=20):
    """p10/p50/p90 of one step's duration (us), from HIP events on the launch stream around each step, over n
    untimed steps: back to back as in the timed region ("warm": the step's data may still sit in the L2s and the
    256 MB last-level cache), and with a 512 MiB buffer read and written before each step ("cold").  Decode with
    graphs: one replay of DECODE_GRAPH steps per sample, divided by DECODE_GRAPH."""
    import numpy as np
    import torch

    scrub = torch.zeros(128 << 20, dtype=torch.float32, device="cuda")
    out = {"samples": n, "cold_scrub_bytes": scrub.numel() * 4}
    graphs = bool(step.graphs)
    for name, cold in (("warm", False), ("cold", True)):
        ev = []
        for _ in range(n):
            if cold:
                scrub.add_(1.0)
            if graphs:
                step.run(DECODE_GRAPH, ev)
            else:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                step()
                e1.record()
                ev.append((e0, e1))
        torch.cuda.synchronize()
        per = np.array([a.elapsed_time(b) * 1e3 / (DECODE_GRAPH if graphs else 1) for a, b in ev])
        out[name] = {f"p{q}": round(float(np.percentile(per, q)), 2) for q in (10, 50, 90)}
    del scrub
    return out


def memory_report(step):
    """Device memory the library needs beside the I/O tensors (checkpoint of segment states and workspaces), what
    storing the state S_i of every token would take instead (B*H*N*D*M float32), and the peak allocation."""
    import torch

    w = step.w
    out = {"peak_device_bytes": int(torch.cuda.max_memory_allocated())}
    if step.wl.startswith("decode"):
        return out
    lib = 0
    for name in ("ck", "ws_f", "ws_b", "ws_n", "ws_nb"):
        t = getattr(step, name, None)
        if t is not None:
            lib += t.numel() * t.element_size()
    d = getattr(w, "features", None) or w.D
    out.update({"checkpoint_and_workspace_bytes": int(lib), "stored_states_bytes": w.B * w.H * w.N * d * w.M * 4})
    return out


def seq_sweep(args):
    """The pages' sequence-length experiment ("Transformers are RNNs -- part 2/3", section 4.1.2, Figure 1): the
    attention and its gradients on synthetic input for N = 2^9 .. 2^16, the batch scaled inversely with N, time and
    peak allocated memory per sample.  Heads and widths follow the 2^16-token workload (H=16, D=M=64, bf16, inputs
    N(0, 1/8^2)); B = 65536 / N.  The inputs of every N are the same 2^16 x 16 x 64 seeded draws (seeds 401-404)
    cut into B sequences.  Per N: 3 warm-up steps, then `steps` (default 20) steps timed with events."""
    import torch

    from linear_rnn_layers_amd import binding, inputs

    w = inputs.LONG
    H, D, M, total = w.H, w.D, w.M, w.N
    full = [torch.from_numpy(a).to("cuda").to(torch.bfloat16) for a in (*w.qkv(), w.grad_out())]
    code = binding.dtype_code(torch.bfloat16)
    steps = args.steps or 20
    rows = []
    for lg in range(9, 17):
        N = 1 << lg
        B = total // N
        q, k, v, do = (x.reshape(H, B, N, x.shape[-1]).permute(1, 0, 2, 3).contiguous() for x in full)
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        o = torch.empty((B, H, N, M), dtype=torch.bfloat16, device="cuda")
        den = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        ck = torch.empty(binding.checkpoint_size(B, H, N, D, M) // 4, dtype=torch.float32, device="cuda")
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws_f = binding.alloc_workspace(binding.LA_OP_FWD_CAUSAL, B, H, N, D, M, code, "cuda")
        ws_b = binding.alloc_workspace(binding.LA_OP_BWD_CAUSAL, B, H, N, D, M, code, "cuda")

        def one():
            binding.la_forward_causal(q, k, v, o, den, ckpt=ck, ws=ws_f)
            binding.la_backward_causal(q, k, v, o, den, do, dq, dk, dv, ckpt=ck, ws=ws_b)

        for _ in range(3):
            one()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            one()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        peak = torch.cuda.max_memory_allocated() - base  # outputs, checkpoint and workspaces of this N
        lib = sum(t.numel() * t.element_size() for t in (ck, ws_f, ws_b))
        io = sum(t.numel() * t.element_size() for t in (q, k, v, do))
        rows.append({"N": N, "B": B, "us_per_step": round(us, 2), "us_per_sample": round(us / B, 3),
                     "tokens_per_s": B * N / (us * 1e-6),
                     "inputs_bytes_per_sample": io // B, "peak_bytes_per_sample": (io + peak) // B,
                     "checkpoint_and_workspace_bytes_per_sample": lib // B,
                     "stored_states_bytes_per_sample": H * N * D * M * 4})
        del q, k, v, do, o, den, ck, dq, dk, dv, ws_f, ws_b
    print(json.dumps({"metric": "causal linear-attn fwd+bwd time and peak memory per sample vs N (batch x N = 65536)",
                      "unit": "us/sample", "n_gpus": 1, "steps": steps, "dtype": "bf16 storage, split-bf16 MFMA with f32 accumulate",
                      "data": "synthetic",
                      "config": {"workload": "sequence-length sweep", "H": H, "D": D, "M": M, "tokens": total},
                      "rows": rows}))


# ------------------------------------------------------------ cpu baseline
def cpu_baseline(wl, w):
    """The float64 oracle (oracle/, OpenMP over heads) on the host cores, on a bounded sample of the workload,
    repeated for at least 10 s, scaled to the workload's unit."""
    import numpy as np

    import oracle

    oracle.build()
    if wl.startswith("decode"):
        nheads, steps = 64, 512  # 64 of the heads, 512 steps each
        s = np.zeros((1, nheads, w.D, w.M))
        z = np.zeros((1, nheads, w.D))
        rng = np.random.Generator(np.random.PCG64(5))
        qs = rng.standard_normal((steps, 1, nheads, w.D))
        ks = rng.standard_normal((steps, 1, nheads, w.D))
        vs = rng.standard_normal((steps, 1, nheads, w.M))
        t = time.perf_counter()
        for i in range(steps):
            _, s, z = oracle.decode_step(qs[i], ks[i], vs[i], s, z)
        el = time.perf_counter() - t
        return {"value": steps / el * nheads / (w.B * w.H), "unit": "decode steps/s (all B*H heads)",
                "cores": oracle.num_threads(), "kind": "oracle",
                "sample": f"{steps} steps on {nheads} of {w.B * w.H} heads, scaled to all heads"}
    B, H, N = w.B, w.H, w.N
    nb = {"mnist": 4, "cifar": 1, "long": 1, "long-decay": 1, "mnist-rf": 4, "mnist-rf256": 2, "cifar-poly2": 1,
          "speech": 4, "small": 1}[wl]
    nh = {"mnist": H, "cifar": 8, "long": 2, "long-decay": 2, "mnist-rf": H, "mnist-rf256": H, "cifar-poly2": 2,
          "speech": H, "small": 1}[wl]
    n = {"long": 16384, "long-decay": 8192}.get(wl, N)
    q, k, v = (a[:nb, :nh, :n] for a in w.qkv(n=n))
    do = w.grad_out(n=n)[:nb, :nh, :n]
    la = w.log_a(n=n)[:nb, :nh, :n] if wl == "long-decay" else None
    wp = w.projection() if w.features and w.fmap == "random" else None
    reps = 0
    t = time.perf_counter()
    while True:
        if w.features and w.fmap == "random":
            fq, fk = oracle.feature_performer(q, wp[:nh]), oracle.feature_performer(k, wp[:nh])
            oracle.forward_causal(fq, fk, v, feature=1)
            dfq, dfk, _ = oracle.backward_causal(fq, fk, v, do, feature=1)
            oracle.feature_performer_vjp(q, wp[:nh], dfq)
            oracle.feature_performer_vjp(k, wp[:nh], dfk)
        elif w.features:
            fq, fk = oracle.feature_poly2(q, w.features), oracle.feature_poly2(k, w.features)
            oracle.forward_causal(fq, fk, v, feature=1)
            dfq, dfk, _ = oracle.backward_causal(fq, fk, v, do, feature=1)
            oracle.feature_poly2_vjp(q, dfq)
            oracle.feature_poly2_vjp(k, dfk)
        elif wl == "long-decay":
            oracle.forward_decay(q, k, v, la)
            oracle.backward_decay(q, k, v, la, do)
        elif wl == "speech":
            oracle.forward_noncausal(q, k, v)
            oracle.backward_noncausal(q, k, v, do)
        else:
            oracle.forward_causal(q, k, v)
            if wl != "small":
                oracle.backward_causal(q, k, v, do)
            if wl == "mnist":
                oracle.forward_noncausal(q, k, v)
        reps += 1
        el = time.perf_counter() - t
        if el >= 10.0 or reps >= 1000:
            break
    layers = w.layers if wl in ("cifar", "speech") else 1
    value = reps * nb * nh * n / el / (H * layers)  # model tokens/s: every token goes through H heads (x layers)
    return {"value": value, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{reps} x one step's passes on {nb}x{nh} of {B}x{H} sequences, {n} of {N} tokens"
                      f"{f', scaled to {layers} layers' if layers > 1 else ''}"}


def _rowerr(x, y, scalar_rows=False):
    """max over rows of |x_r - y_r|_inf / max(|y_r|_inf, 1e-3 max over the head's rows) (float64)."""
    import numpy as np

    x, y = np.asarray(x, np.float64), np.asarray(y, np.float64)
    if scalar_rows:
        x, y = x[..., None], y[..., None]
    d = np.abs(x - y).max(-1)
    yn = np.abs(y).max(-1)
    fl = 1e-3 * yn.reshape(yn.shape[0], yn.shape[1], -1).max(-1)
    den = np.maximum(yn, fl.reshape(fl.shape + (1,) * (yn.ndim - 2)))
    return float(np.max(np.where(den > 0, d / np.where(den > 0, den, 1), d)))


def headline_parity(step, heads=(0, 15)):
    """The timed step's outputs against the oracle (float64) on sampled heads at the full sequence: O, den, dQ,
    dK, dV per row (the dQ rows floored at 1e-2 of their cancelled eq. 13 term, as in the parity tests)."""
    import numpy as np
    import torch

    import oracle

    w = step.w
    q, k, v, do = step.sets[0]
    step.b.la_forward_causal(q, k, v, step.o, step.den, ckpt=step.ck, ws=step.ws_f)
    step.b.la_backward_causal(q, k, v, step.o, step.den, do, step.dq, step.dk, step.dv, ckpt=step.ck, ws=step.ws_b)
    torch.cuda.synchronize()
    host = lambda t, h: t[:, h:h + 1].float().cpu().numpy().astype(np.float64)  # noqa: E731
    out = {}
    for h in heads:
        qh, kh, vh, dh = (host(t, h) for t in (q, k, v, do))
        o, den, _, _ = oracle.forward_causal(qh, kh, vh)
        dq, dk, dv = oracle.backward_causal(qh, kh, vh, dh)
        # the eq. 13 term S_i g_i of dQ (numerator-only backward with g = dO / den), through phi'
        p = np.where(qh > 0, qh + 1, np.exp(qh))
        kf = np.where(kh > 0, kh + 1, np.exp(kh))
        g = dh / den[..., None]
        sq = oracle.numerator_backward(p[0, 0], kf[0, 0], vh[0, 0], g[0, 0])[0][None, None]
        floor = 1e-2 * np.abs(sq * np.minimum(p, 1.0)).max(-1)
        errs = {"O": _rowerr(host(step.o, h), o), "den": _rowerr(host(step.den, h), den, True),
                "dK": _rowerr(host(step.dk, h), dk), "dV": _rowerr(host(step.dv, h), dv)}
        x, y = host(step.dq, h), dq
        d = np.abs(x - y).max(-1)
        yn = np.maximum(np.abs(y).max(-1), 1e-3 * np.abs(y).max())
        errs["dQ"] = float((d / np.maximum(yn, floor)).max())
        for key, val in errs.items():
            out[key] = max(out.get(key, 0.0), val)
    return {"heads": list(heads), "tokens": w.N, "measure": "rowerr (max over rows of the row's inf-norm error over "
            "its inf-norm, floored at 1e-3 of the head's largest row)", "tolerance": 2e-2 if w.dtype == "bf16" else 1e-4,
            **{k: round(v, 6) for k, v in out.items()}}


def feature_parity(step, heads=(0,)):
    """A feature-map step against the oracle on sampled heads of the first batch entry, each stage at its own
    inputs: the map of the stored inputs, the attention (O, the feature gradients, dV) on the features the library
    produced, the chain rule on the feature gradients it produced.  The query-side feature gradient is floored at
    1e-2 of its numerator term |S_i g_i|, as in the parity tests."""
    import numpy as np
    import torch

    import oracle

    w, b = step.w, step.b
    q, k, v, do = step.sets[0]
    step._features_step(q, k, v, do)
    torch.cuda.synchronize()
    C = w.features

    def host(t, h):
        x = t[:1, h:h + 1].float().cpu().numpy().astype(np.float64)
        if x.ndim == 5:  # feature-sliced [1, 1, ns, N, 64] -> [1, 1, N, C]
            x = x.transpose(0, 1, 3, 2, 4).reshape(1, 1, x.shape[3], -1)
        return x

    out = {}
    for h in heads:
        qh, kh, vh, dh = (host(t, h) for t in (q, k, v, do))
        if w.fmap == "random":
            wp = step.W[h:h + 1].cpu().numpy().astype(np.float64)
            fmap = lambda x: oracle.feature_performer(x, wp)  # noqa: E731
            fvjp = lambda x, g: oracle.feature_performer_vjp(x, wp, g)  # noqa: E731
        else:
            fmap = lambda x: oracle.feature_poly2(x, C)  # noqa: E731
            fvjp = oracle.feature_poly2_vjp
        fq, fk, dfq, dfk = (host(t, h) for t in (step.fq, step.fk, step.dfq, step.dfk))
        o, den, _, _ = oracle.forward_causal(fq, fk, vh, feature=1)
        rq, rk, rv = oracle.backward_causal(fq, fk, vh, dh, feature=1)
        sq = oracle.numerator_backward(fq[0, 0], fk[0, 0], vh[0, 0], dh[0, 0] / den[0, 0][:, None])[0][None, None]
        floor = 1e-2 * np.abs(sq).max(-1)
        errs = {"Phi": max(_rowerr(fq, fmap(qh)), _rowerr(fk, fmap(kh))), "O": _rowerr(host(step.o, h), o),
                "den": _rowerr(host(step.den, h), den, True), "dPhiK": _rowerr(dfk, rk),
                "dV": _rowerr(host(step.dv, h), rv),
                "dQ": _rowerr(host(step.dq, h), fvjp(qh, dfq)), "dK": _rowerr(host(step.dk, h), fvjp(kh, dfk))}
        d = np.abs(dfq - rq).max(-1)
        yn = np.maximum(np.abs(rq).max(-1), 1e-3 * np.abs(rq).max())
        errs["dPhiQ"] = float((d / np.maximum(yn, floor)).max())
        for key, val in errs.items():
            out[key] = max(out.get(key, 0.0), val)
    return {"heads": list(heads), "batch_entries": [0], "tokens": w.N, "features": C,
            "measure": "rowerr, each stage at its own inputs (the library's features into the attention, its "
                       "feature gradients into the chain rule)", "tolerance": 2e-2 if w.dtype == "bf16" else 1e-4,
            **{k: round(v, 6) for k, v in out.items()}}


# -------------------------------------------------------------- measuring
def dtype_label(wl, s):
    """Storage type and arithmetic: the attention passes multiply bf16 planes of their operands on MFMA with
    float32 accumulation (one plane for bf16 inputs, split planes for computed and float32 operands); the decode
    step is float32 vector arithmetic on a float32 state."""
    store = "f32" if s == 4 else "bf16"
    if wl.startswith("decode"):
        return f"{store} storage, f32 state and arithmetic"
    return f"{store} storage, split-bf16 MFMA with f32 accumulate"


def measure(wl, steps, warmup, args, headline=False, copy_gbs=None):
    """One record: exactly `steps` timed steps after `warmup` untimed ones, the dominant kernel's launches
    bracketed by HIP events inside the timed region."""
    import torch

    dominant = dominant_kernel(wl)
    eager = wl.startswith("decode") and args.eager_decode
    per_step = {"cifar": 16, "speech": 9}.get(wl, 1)  # launches of the dominant kernel per step
    graphs_planned = wl.startswith("decode") and not eager  # replays are timed with events around each graph
    timed = None if args.no_kernel_events or graphs_planned else dominant
    step = Step(wl, timed, pairs=per_step * (steps + warmup) + 8, eager_decode=eager,
                segment_chunks=args.segment_chunks)
    w = step.w
    s = 4 if w.dtype == "f32" else 2
    graphs = bool(step.graphs)
    if graphs:
        step.run(warmup)
    else:
        for _ in range(warmup):
            step()
    torch.cuda.synchronize()
    if step.timer:
        step.timer.reset()
    gev = [] if graphs and not args.no_kernel_events else None
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graphs:
        step.run(steps, gev)
    else:
        for _ in range(steps):
            step()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    kms, kn = step.timer.collect() if step.timer else (0.0, 0)
    if gev:
        kms, kn = sum(e0.elapsed_time(e1) for e0, e1 in gev), len(gev) * DECODE_GRAPH
    ms_per_step = el * 1e3 / steps
    if wl.startswith("decode"):
        metric, unit, value = "decode steps/s", "steps/s", steps / el
    else:
        metric = {"speech": "non-causal linear-attn fwd+bwd tokens/s",
                  "mnist-rf": "random-feature causal linear-attn fwd+bwd tokens/s",
                  "mnist-rf256": "random-feature causal linear-attn fwd+bwd tokens/s",
                  "cifar-poly2": "degree-2 polynomial-feature causal linear-attn fwd+bwd tokens/s",
                  "long-decay": "decayed causal linear-attn fwd+bwd tokens/s",
                  "small": "causal linear-attn fwd tokens/s"}.get(wl, "causal linear-attn fwd+bwd tokens/s")
        unit, value = "tokens/s", w.B * w.N * steps / el
    step_bytes, step_flops = step_work(wl, w, s)
    copy_gbs = copy_gbs or copy_bandwidth()
    roof = None
    if kn:
        avg_s = kms / kn / 1e3
        byts = dominant_bytes(wl, dominant, w, s)
        achieved = byts / avg_s / 1e9
        traffic = traffic_from_profiles(dominant, wl)
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": traffic, "kernel": dominant,
                "algorithmic_bytes_per_launch": byts, "avg_launch_us": avg_s * 1e6, "launches": kn,
                "copy_gbs": copy_gbs, "frac_of_copy": achieved / copy_gbs}
        if gev:
            roof["timing"] = (f"events around each replay of a graph of {DECODE_GRAPH} launches, divided by "
                              f"{DECODE_GRAPH} (back-to-back launches, gaps included)")
    step_time = ms_per_step * 1e-3
    step_roof = {"bound": "hbm", "algorithmic_bytes": step_bytes, "achieved": step_bytes / step_time / 1e9,
                 "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": step_bytes / step_time / 1e9 / HBM_PEAK_GBS,
                 "frac_of_copy": step_bytes / step_time / 1e9 / copy_gbs}
    mf = _profile_json(f"{wl}_mfma.json")
    ks = _profile_json(f"{wl}_kernels.json")
    side = {"hbm_frac": step_roof["frac"],
            "useful_flop_frac": step_flops / step_time / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "executed_mfma_frac": None, "mfma_busy": None,
            "source": "executed MFMA and MFMA-busy from rocprofv3 counters in profiles/ taken at the current kernel "
                      "sources (null when the sources have changed since)"}
    if mf and ks and ks.get("steps_profiled"):
        launches = {k: v["calls"] / ks["steps_profiled"] for k, v in ks["kernels"].items()}
        ex = sum(v["mfma_insts_per_launch"] * launches.get(k, 0.0) for k, v in mf["kernels"].items())
        side["executed_mfma_frac"] = ex * MFMA_FLOPS_PER_INST / step_time / 1e12 / MFMA_BF16_PEAK_TFLOPS
    if mf:
        if dominant in mf["kernels"]:
            d = mf["kernels"][dominant]
            side["mfma_busy"] = d["mfma_busy_cycles_per_launch"] / (d["average_us"] * 1e-6 * CLOCK_GHZ * 1e9 * SIMDS)
            side["dominant_executed_mfma_frac"] = (d["mfma_insts_per_launch"] * MFMA_FLOPS_PER_INST /
                                                   (d["average_us"] * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS)
    breakdown = None
    if ks:
        tot = ks.get("steps_profiled")
        breakdown = {k: {"average_us": round(v["average_us"], 2),
                         "launches_per_step": (v["calls"] / tot) if tot else None}
                     for k, v in ks["kernels"].items()}
    cfg = {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "D": w.D, "M": w.M}
    if w.features:
        cfg["C"] = w.features
    cfg["step"] = {"mnist": "causal forward + causal backward + non-causal forward",
                   "cifar": "16 layers x (causal forward + backward)", "long": "causal forward + backward",
                   "long-decay": "decayed causal forward + backward (dQ, dK, dV, dlogA)",
                   "mnist-rf": "random features of Q, K (C = 64) + causal forward and backward on them + chain rule",
                   "mnist-rf256": "random features of Q, K (C = 256, feature-sliced) + causal forward and backward on "
                                  "them + chain rule",
                   "cifar-poly2": "degree-2 polynomial features of Q, K (Din = 32, C = 1088, feature-sliced) + causal "
                                  "forward and backward on them + chain rule",
                   "speech": "9 layers x (non-causal forward + backward)",
                   "small": "causal forward"}.get(wl, "one decode step of all B*H heads after the prefill")
    if args.segment_chunks:
        cfg["segment_tokens"] = 64 * args.segment_chunks  # forced, not the library's plan
    if wl.startswith("decode"):
        cfg["prefill_tokens"] = w.N
        cfg["launch"] = f"HIP graphs of {DECODE_GRAPH} steps" if graphs else "one host launch per step"
        cfg["state_bytes"] = w.B * w.H * (w.D * w.M + w.D) * 4
    rec = {"metric": metric, "value": value, "unit": unit, "steps": steps, "warmup": warmup,
           "ms_per_step": ms_per_step, "dtype": dtype_label(wl, s),
           "config": cfg, "roofline": roof, "step_roofline": step_roof, "side_by_side": side,
           "kernels_from_rocprof": breakdown}
    if headline:
        rec["step_us"] = step_distribution(step)
        rec["memory"] = memory_report(step)
    if not args.no_parity and wl in ("long", "mnist", "cifar"):
        rec["parity"] = headline_parity(step, (0, w.H - 1) if wl == "long" else (0,))
    if not args.no_parity and w.features:
        rec["parity"] = feature_parity(step)
    if wl == "decode" and not eager and not args.no_kernel_events:
        # the same steps launched one at a time from the host (the decode kernel timed per launch)
        del step
        torch.cuda.empty_cache()
        e_steps = steps
        st2 = Step(wl, dominant, pairs=e_steps + 8, eager_decode=True)
        for _ in range(warmup):
            st2()
        torch.cuda.synchronize()
        st2.timer.reset()
        t0 = time.perf_counter()
        for _ in range(e_steps):
            st2()
        torch.cuda.synchronize()
        el2 = time.perf_counter() - t0
        kms2, kn2 = st2.timer.collect()
        rec["eager"] = {"value": e_steps / el2, "unit": "steps/s", "ms_per_step": el2 * 1e3 / e_steps,
                        "decode_kernel_us": kms2 / kn2 * 1e3 if kn2 else None,
                        "frac": (decode_step_bytes(w, s) / (kms2 / kn2 * 1e-3) / 1e9 / HBM_PEAK_GBS) if kn2 else None}
        del st2
    else:
        del step
    torch.cuda.empty_cache()
    return rec


# -------------------------------------------------------------------- main
def main():
    args = parse()
    if args.summarize_stats:
        summarize_stats(args)
        return
    if args.summarize_traffic:
        summarize_traffic(args)
        return
    if args.summarize_mfma:
        summarize_mfma(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: every head is independent, so more GPUs "
                                   "would shard B*H with no communication inside the method; no multi-GPU figure is "
                                   "measured here", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    torch.cuda.set_device(0)
    if args.copy_only:
        n = args.copy_only * (1 << 20) // 4
        a = torch.ones(n, device="cuda")
        bb = torch.empty_like(a)
        for _ in range(max(1, args.steps or 1)):
            bb.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "launches": max(1, args.steps or 1)}))
        return
    if args.seq_sweep:
        seq_sweep(args)
        return

    wl = args.workload or HEADLINE
    ds, dw = default_steps(wl)
    steps = args.steps if args.steps is not None else ds
    warmup = args.warmup if args.warmup is not None else dw
    if args.profile_run:
        step = Step(wl, None, eager_decode=args.eager_decode, segment_chunks=args.segment_chunks)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        if step.graphs:
            step.run(warmup + steps)
        else:
            for _ in range(warmup + steps):
                step()
        torch.cuda.synchronize()
        print(json.dumps({"profile_run": wl, "steps_executed": warmup + steps,
                          "ms_per_step": (time.perf_counter() - t0) * 1e3 / (warmup + steps),
                          "source_hash": source_hash()}))
        return
    from linear_rnn_layers_amd import build as _build

    lib_stale = _build.stale()
    if lib_stale:
        print("bench: WARNING the HIP library is older than its sources; the figures are for the older build",
              file=sys.stderr, flush=True)
    copy = copy_bandwidth()
    print(f"bench: {wl} ({steps} steps, {warmup} warm-up)", file=sys.stderr, flush=True)
    rec = measure(wl, steps, warmup, args, headline=True, copy_gbs=copy)
    nested = {}
    if args.workload is None and not args.no_nested:
        for nw in NESTED:
            ns, nwu = default_steps(nw)
            print(f"bench: nested {nw} ({ns} steps, {nwu} warm-up)", file=sys.stderr, flush=True)
            nested[nw] = measure(nw, ns, nwu, args, copy_gbs=copy)
    cpu = None
    if not args.no_cpu_baseline:
        print("bench: cpu baseline", file=sys.stderr, flush=True)
    from linear_rnn_layers_amd import inputs as _inputs

    w = WORKLOADS(_inputs)[wl]
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, w)
    roof = rec["roofline"]
    out = {"metric": rec["metric"], "value": rec["value"], "unit": rec["unit"], "n_gpus": 1, "steps": steps,
           "warmup": warmup, "ms_per_step": rec["ms_per_step"], "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": rec["dtype"], "data": "synthetic (seeded Gaussian inputs of the workload's "
           "shape; no dataset)", "config": rec["config"], "roofline": roof, "cpu_baseline": cpu,
           "step_roofline": rec["step_roofline"], "side_by_side": rec["side_by_side"],
           "kernels_from_rocprof": rec["kernels_from_rocprof"], "parity": rec.get("parity"),
           "step_us": rec.get("step_us"), "memory": rec.get("memory"), "nested": nested or None,
           "copy_gbs": copy, "gpu": torch.cuda.get_device_name(0), "rocm": torch.version.hip,
           "seeds": list(w.seeds), "source_hash": source_hash(), "library_older_than_sources": lib_stale,
           "kernel_events_in_timed_region": not args.no_kernel_events}
    if cpu and rec["unit"] == cpu["unit"]:
        out["gpu_over_cpu"] = rec["value"] / cpu["value"]
    print(json.dumps(out))


if __name__ == "__main__":
    main()
