"""Benchmark of the causal linear attention library on one MI355X.

Default workload (the one the headline metric is quoted on): an MNIST-shaped
attention layer, B=16 H=8 N=784 D=M=32, float32 storage.  One step is the
whole hot path over one batch: causal forward (phi prologue, intra-chunk
blocks, state carry, epilogue), causal backward, and the non-causal forward
at the same shape.  Other workloads (--workload): cifar (16 independent layers
of B=4 H=8 N=3072 D=M=32, bf16, sigma 0.5, forward + backward each), long
(B=1 H=16 N=65536 D=M=64, bf16, sigma 1/8, forward + backward), speech (9
independent non-causal layers of B=16 H=6 N=800 D=M=32, float32, non-causal
forward + backward each), long-decay (the long shape with a per-token,
per-head decay on the state: decayed forward + backward including the
gradient of the log-decay), mnist-rf (the mnist shape with 64 positive random
features in place of elu + 1: feature maps, causal forward and backward in
feature mode, chain rule through the features), decode (one
step = one la_decode_step on B=256 H=16 D=M=64 after a 512-token prefill),
small (B=1 H=1 N=64 D=M=32 float32 causal forward).

Prints one JSON line: throughput, the roofline of the dominant kernel (its
duration measured with HIP events recorded by the library around every
launch of that kernel inside the timed region), and the float64 oracle timed
on the host cores on a bounded sample of the same workload.  After the timed
region, untimed steps give the p10/p50/p90 of one step's duration with the
caches as the timed loop leaves them and after a 512 MiB scrub ("step_us").
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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default 50; decode: 4096)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed warm-up steps (default 10; decode: 256)")
    ap.add_argument("--workload", default="mnist", choices=["mnist", "cifar", "long", "long-decay", "mnist-rf", "speech", "decode",
                                                            "small"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-events", action="store_true", help="time without per-kernel events")
    ap.add_argument("--eager-decode", action="store_true",
                    help="decode: one host launch per step instead of replaying captured graphs of 64 steps")
    ap.add_argument("--seq-sweep", action="store_true",
                    help="causal forward + backward time and peak memory per sample for N = 2^9 .. 2^16 with the batch "
                         "scaled inversely (B*N = 65536; H=16, D=M=64, bf16), one JSON line")
    ap.add_argument("--copy-only", type=int, default=0, metavar="MiB",
                    help="only run a plain device copy of this size (traffic-counter calibration)")
    ap.add_argument("--summarize-stats", metavar="CSV", help="write profiles/<label>_kernels.md from a "
                    "rocprofv3 --kernel-trace --stats kernel_stats.csv")
    ap.add_argument("--summarize-traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="write profiles/traffic_<kernel>_<label>.json/.md from rocprofv3 --pmc counter CSVs")
    ap.add_argument("--summarize-mfma", nargs=2, metavar=("PMC_CSV", "STATS_CSV"),
                    help="write profiles/<label>_mfma.md from a --pmc SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES ... run "
                         "and the kernel statistics of a --kernel-trace --stats run")
    ap.add_argument("--label", default="mnist")
    ap.add_argument("--command", default="", help="the command that produced the CSVs (recorded in the summary)")
    a = ap.parse_args()
    if a.steps is None:
        a.steps = 4096 if a.workload == "decode" else 50
    if a.warmup is None:
        a.warmup = 256 if a.workload == "decode" else 10
    return a


# ------------------------------------------------------------------ steps
class Step:
    """Inputs resident in HBM, outputs preallocated, one callable per step."""

    def __init__(self, args):
        import torch

        from linear_rnn_layers_amd import binding, inputs

        self.torch, self.b, self.inputs = torch, binding, inputs
        self.args = args
        wl = args.workload
        self.w = WORKLOADS(inputs)[wl]
        w = self.w
        dt = torch.float32 if w.dtype == inputs.F32 else torch.bfloat16
        self.dt = dt
        dev = lambda x: torch.from_numpy(x).to("cuda").to(dt).contiguous()  # noqa: E731
        B, H, N, D, M = w.B, w.H, w.N, w.D, w.M
        code = binding.dtype_code(dt)
        self.sets = []
        if wl == "decode":
            self._init_decode(dev)
            return
        if wl in ("cifar", "speech"):
            nsets = w.layers  # one independent input set per layer
        elif wl in ("mnist", "mnist-rf"):
            nsets = 6  # rotate batches so successive steps do not hit the 256 MB last-level cache
        else:
            nsets = 1
        for i in range(nsets):
            if wl in ("cifar", "speech"):
                q, k, v = w.qkv(layer=i)
                do = w.grad_out(layer=i)
            elif i == 0:
                q, k, v = w.qkv()
                do = w.grad_out()
            else:
                q, k, v, do = self._extra_set(i)
            self.sets.append(tuple(dev(a) for a in (q, k, v, do)))
        self.o = torch.empty((B, H, N, M), dtype=dt, device="cuda")
        self.onc = torch.empty((B, H, N, M), dtype=dt, device="cuda")
        self.den = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        self.ck = torch.empty(binding.checkpoint_size(B, H, N, D, M) // 4, dtype=torch.float32, device="cuda")
        self.dq = torch.empty((B, H, N, D), dtype=dt, device="cuda")
        self.dk = torch.empty((B, H, N, D), dtype=dt, device="cuda")
        self.dv = torch.empty((B, H, N, M), dtype=dt, device="cuda")
        self.ws_f = binding.alloc_workspace(binding.LA_OP_FWD_CAUSAL, B, H, N, D, M, code, "cuda")
        self.ws_b = binding.alloc_workspace(binding.LA_OP_BWD_CAUSAL, B, H, N, D, M, code, "cuda")
        self.ws_n = binding.alloc_workspace(binding.LA_OP_FWD_NONCAUSAL, B, H, N, D, M, code, "cuda")
        if wl == "speech":
            self.ws_nb = binding.alloc_workspace(binding.LA_OP_BWD_NONCAUSAL, B, H, N, D, M, code, "cuda")
            self.s_tot = torch.empty((B, H, D, M), dtype=torch.float32, device="cuda")
            self.z_tot = torch.empty((B, H, D), dtype=torch.float32, device="cuda")
        if wl == "mnist-rf":
            C = w.features
            self.W = torch.from_numpy(w.projection()).to("cuda").contiguous()
            self.fq = torch.empty((B, H, N, C), dtype=dt, device="cuda")
            self.fk = torch.empty((B, H, N, C), dtype=dt, device="cuda")
            self.dfq = torch.empty((B, H, N, C), dtype=dt, device="cuda")
            self.dfk = torch.empty((B, H, N, C), dtype=dt, device="cuda")
            self.ck = torch.empty(binding.checkpoint_size(B, H, N, C, M) // 4, dtype=torch.float32, device="cuda")
            self.ws_f = binding.alloc_workspace(binding.LA_OP_FWD_CAUSAL, B, H, N, C, M, code, "cuda")
            self.ws_b = binding.alloc_workspace(binding.LA_OP_BWD_CAUSAL, B, H, N, C, M, code, "cuda")
        if wl == "long-decay":
            self.log_a = torch.from_numpy(w.log_a()).to("cuda").contiguous()
            self.dla = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
            self.ws_f = binding.alloc_workspace(binding.LA_OP_FWD_DECAY, B, H, N, D, M, code, "cuda")
            self.ws_b = binding.alloc_workspace(binding.LA_OP_BWD_DECAY, B, H, N, D, M, code, "cuda")
        self.i = 0

    def _extra_set(self, i):
        w, inputs = self.w, self.inputs
        base = 100_000 * i
        sh = (w.B, w.H, w.N)
        return (inputs.gaussian(sh + (w.D,), w.seeds[0] + base, w.sigma, w.dtype),
                inputs.gaussian(sh + (w.D,), w.seeds[1] + base, w.sigma, w.dtype),
                inputs.gaussian(sh + (w.M,), w.seeds[2] + base, w.sigma, w.dtype),
                inputs.gaussian(sh + (w.M,), w.seeds[3] + base, 1.0, w.dtype))

    def _init_decode(self, dev):
        torch, b, w = self.torch, self.b, self.w
        B, H, D, M = w.B, w.H, w.D, w.M
        q, k, v = w.qkv()  # 512-token prefill (seeded numpy recipe)
        out = b.forward_causal(dev(q), dev(k), dev(v), return_state=True, checkpoint=False)
        self.S, self.Z = out["s"], out["z"]
        pool = 4096  # distinct per-step inputs, drawn on the GPU (Philox, seed 5000000), N(0,1) in bf16
        gen = torch.Generator(device="cuda")
        gen.manual_seed(5_000_000)
        self.pool_q = torch.randn((pool, B, H, D), generator=gen, device="cuda").to(self.dt)
        self.pool_k = torch.randn((pool, B, H, D), generator=gen, device="cuda").to(self.dt)
        self.pool_v = torch.randn((pool, B, H, M), generator=gen, device="cuda").to(self.dt)
        self.y = torch.empty((B, H, M), dtype=self.dt, device="cuda")
        import ctypes

        lib = b.load()
        self._call = lib.la_decode_step
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        code = b.dtype_code(self.dt)
        qs, ks, vs = self.pool_q.stride(0) * 2, self.pool_k.stride(0) * 2, self.pool_v.stride(0) * 2
        self._args = [(ctypes.c_void_p(self.pool_q.data_ptr() + i * qs), ctypes.c_void_p(self.pool_k.data_ptr() + i * ks),
                       ctypes.c_void_p(self.pool_v.data_ptr() + i * vs), None, ctypes.c_void_p(self.S.data_ptr()),
                       ctypes.c_void_p(self.Z.data_ptr()), ctypes.c_void_p(self.y.data_ptr()), B, H, D, M, code, 0,
                       stream)
                      for i in range(pool)]
        self.i = 0
        # A decode loop issues one small launch per step, so the host's launch cost shows between steps; a
        # serving loop captures its steps in HIP graphs.  Graph g replays steps 64 g .. 64 g + 63 of the pool
        # (64 launches back to back; the captured calls are the same C-ABI entry point on torch's capture
        # stream).
        self.graphs = []
        if not getattr(self.args, "eager_decode", False):
            for g0 in range(0, pool, DECODE_GRAPH):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    cs = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
                    for a in self._args[g0:g0 + DECODE_GRAPH]:
                        st = self._call(*(a[:-1] + (cs,)))
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
        wl, b = self.args.workload, self.b
        if wl == "decode":
            a = self._args[self.i % len(self._args)]
            self.i += 1
            st = self._call(*a)
            if st != 0:
                raise b.LAError(st, "la_decode_step")
            return
        if wl == "cifar":
            for (q, k, v, do) in self.sets:
                self._fwd_bwd(q, k, v, do)
            return
        if wl == "speech":  # the forward's totals go to the backward, as a training step passes them
            for (q, k, v, do) in self.sets:
                b.la_forward_noncausal(q, k, v, self.onc, ws=self.ws_n, S_out=self.s_tot, Z_out=self.z_tot)
                b.la_backward_noncausal(q, k, v, do, self.dq, self.dk, self.dv, ws=self.ws_nb, S_tot=self.s_tot,
                                        Z_tot=self.z_tot)
            return
        if wl == "mnist-rf":
            q, k, v, do = self.sets[self.i % len(self.sets)]
            self.i += 1
            lib, st = b.load(), b._stream(None)
            B, H, N, D, M, C = self.w.B, self.w.H, self.w.N, self.w.D, self.w.M, self.w.features
            IDENT = b.LA_FEATURE_IDENTITY
            for x, f in ((q, self.fq), (k, self.fk)):
                b._check(lib.la_feature_random(b._ptr(x), b._ptr(self.W), b._ptr(f), B, H, N, D, C, 0, st), "rf")
            b.la_forward_causal(self.fq, self.fk, v, self.o, self.den, ckpt=self.ck, ws=self.ws_f, feature=IDENT)
            b.la_backward_causal(self.fq, self.fk, v, self.o, self.den, do, self.dfq, self.dfk, self.dv, ckpt=self.ck,
                                 ws=self.ws_b, feature=IDENT)
            for x, g, dx in ((q, self.dfq, self.dq), (k, self.dfk, self.dk)):
                b._check(lib.la_feature_random_vjp(b._ptr(x), b._ptr(self.W), b._ptr(g), b._ptr(dx), B, H, N, D, C, 0,
                                                   st), "rf_vjp")
            return
        if wl == "long-decay":
            q, k, v, do = self.sets[0]
            b.la_forward_causal(q, k, v, self.o, self.den, ckpt=self.ck, ws=self.ws_f, logA=self.log_a)
            b.la_backward_causal(q, k, v, self.o, self.den, do, self.dq, self.dk, self.dv, ckpt=self.ck,
                                 ws=self.ws_b, logA=self.log_a, dlogA=self.dla)
            return
        q, k, v, do = self.sets[self.i % len(self.sets)]
        self.i += 1
        if wl == "small":
            b.la_forward_causal(q, k, v, self.o, self.den, ws=self.ws_f)
            return
        self._fwd_bwd(q, k, v, do)
        if wl == "mnist":
            b.la_forward_noncausal(q, k, v, self.onc, ws=self.ws_n)

    def _fwd_bwd(self, q, k, v, do):
        b = self.b
        b.la_forward_causal(q, k, v, self.o, self.den, ckpt=self.ck, ws=self.ws_f)
        b.la_backward_causal(q, k, v, self.o, self.den, do, self.dq, self.dk, self.dv, ckpt=self.ck, ws=self.ws_b)


DECODE_GRAPH = 64  # decode steps per captured graph


def WORKLOADS(inputs):
    return {"mnist": inputs.MNIST, "cifar": inputs.CIFAR, "long": inputs.LONG, "speech": inputs.SPEECH,
            "long-decay": inputs.LONG_DECAY, "mnist-rf": inputs.MNIST_RF, "decode": inputs.DECODE,
            "small": inputs.SMALL}


# ---------------------------------------------------- algorithmic figures
def kernel_bytes(name, w, s):
    """Algorithmic HBM bytes per launch: the tensors the kernel must read or write by its function.  Per
    token-head the method moves (2D+2M)s+4 bytes forward (read Q, K, V; write O, den) and (4D+4M)s+4 backward
    (read Q, K, V, O, dO, den; write dQ, dK, dV), s the bytes per element; these totals are split over the
    kernels that do the work.  With random features the attention kernels see feature vectors of size C in
    place of D."""
    Din, M = w.D, w.M
    D = w.features or Din
    th = w.B * w.H * w.N
    per_th = {
        "fwd_causal": (2 * D + 2 * M) * s + 4,   # read Q, K, V; write O, den
        "seg_state": (D + M) * s,                # read K, V
        "fwd_noncausal": (D + M) * s,            # read Q; write O
        "seg_rstate": (D + 2 * M) * s + 4,       # read Q, O, dO, den
        "bwd_causal": (4 * D + 3 * M) * s,       # read Q, K, V, dO; write dQ, dK, dV
        "nc_qr": (2 * D + M) * s,                # read Q, dO; write dQ
        "nc_kv": (2 * D + 2 * M) * s,            # read K, V; write dK, dV
        "dseg_state": (D + M) * s + 4,           # read K, V, logA
        "dfwd": (2 * D + 2 * M) * s + 8,         # read Q, K, V, logA; write O, den
        "dbq": (3 * D + 2 * M) * s + 12,         # read Q, K, V, dO, logA; write dQ, (1/den, c)
        "dbkv": (3 * D + 3 * M) * s + 16,        # read Q, K, V, dO, logA, (1/den, c); write dK, dV, dlogA terms
        "dla_fix": 8,                            # read and write dlogA
        "feat_rf": (Din + D) * s,                # read X; write Phi
        "feat_rf_vjp": (2 * Din + D) * s,        # read X, dPhi; write dX
    }
    if name == "decode":
        return w.B * w.H * (2 * D * M * 4 + 2 * D * 4 + (2 * D + 2 * M) * s)
    if name in per_th:
        return th * per_th[name]
    return None


def kernel_flops(name, w):
    D, M = w.features or w.D, w.M
    th = w.B * w.H * w.N
    if name == "fwd_causal":
        return th * (4 * D * M + 5 * D + M)
    if name == "bwd_causal":
        return th * (10 * D * M + 9 * D + 3 * M)
    if name == "decode":
        return w.B * w.H * (4 * D * M + 5 * D + M)
    return None


def source_hash():
    h = hashlib.sha256()
    for f in ("la_device.h", "la_kernels.h", "la_decay.h", "la_feature.h", "la_api.hip"):
        with open(os.path.join(ROOT, "linear_rnn_layers_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel, workload):
    """HBM bytes per launch from committed counter summaries, if they match the current kernels."""
    path = os.path.join(PROFILES, f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != source_hash():
        return None
    return rec.get("bytes_per_launch")


# ------------------------------------------------------ profile summaries
KERNEL_TAGS = (("k_bwd<", "bwd_causal"), ("k_seg_rstate<", "seg_rstate"), ("k_seg_state<", "seg_state"),
               ("k_scan_states<", "scan_states"), ("k_scan_rev<", "scan_rev"), ("k_decode<", "decode"),
               ("k_nc_qr<", "nc_qr"), ("k_nc_kv<", "nc_kv"), ("k_dseg_state<", "dseg_state"),
               ("k_dscan_states<", "dscan_states"), ("k_dfwd<", "dfwd"), ("k_dbq<", "dbq"),
               ("k_dscan_rev<", "dscan_rev"), ("k_dbkv<", "dbkv"), ("k_dla_fix", "dla_fix"),
               ("k_feat_rf_vjp<", "feat_rf_vjp"), ("k_feat_rf<", "feat_rf"))


def kernel_tag(full_name):
    if "k_fwd_lb<" in full_name:  # the one-launch causal forward
        return "fwd_causal"
    if "k_sync_clear" in full_name:
        return "sync_clear"
    if "k_fwd<" in full_name:
        return "fwd_noncausal" if "false>" in full_name else "fwd_causal"
    for key, tag in KERNEL_TAGS:
        if key in full_name:
            return tag
    return full_name.split("(")[0][:60]


def step_distribution(step, graphs, n=20):
    """p10/p50/p90 of one step's duration (us), from HIP events on the launch stream around each step, over n
    untimed steps: back to back as in the timed region ("warm": the step's data may still sit in the L2s and the
    256 MB last-level cache), and with a 512 MiB buffer read and written before each step ("cold").  Decode with
    graphs: one replay of DECODE_GRAPH steps per sample, divided by DECODE_GRAPH."""
    import numpy as np
    import torch

    scrub = torch.zeros(128 << 20, dtype=torch.float32, device="cuda")
    out = {"samples": n, "cold_scrub_bytes": scrub.numel() * 4}
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


def seq_sweep(args):
    """The pages' sequence-length experiment ("Transformers are RNNs -- part 2/3", section 4.1.2, Figure 1): the
    attention and its gradients on synthetic input for N = 2^9 .. 2^16, the batch scaled inversely with N, time and
    peak allocated memory per sample.  Heads and widths follow the 2^16-token workload (H=16, D=M=64, bf16, inputs
    N(0, 1/8^2)); B = 65536 / N.  The inputs of every N are the same 2^16 x 16 x 64 seeded draws (seeds 401-404)
    cut into B sequences.  Per N: 3 warm-up steps, then `steps` (default 20) steps timed with events."""
    import numpy as np
    import torch

    from linear_rnn_layers_amd import binding, inputs

    w = inputs.LONG
    H, D, M, total = w.H, w.D, w.M, w.N
    full = [torch.from_numpy(a).to("cuda").to(torch.bfloat16) for a in (*w.qkv(), w.grad_out())]
    code = binding.dtype_code(torch.bfloat16)
    steps = args.steps if args.steps != 50 else 20
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

        def step():
            binding.la_forward_causal(q, k, v, o, den, ckpt=ck, ws=ws_f)
            binding.la_backward_causal(q, k, v, o, den, do, dq, dk, dv, ckpt=ck, ws=ws_b)

        for _ in range(3):
            step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            step()
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
                      "unit": "us/sample", "n_gpus": 1, "steps": steps, "dtype": "bf16", "data": "synthetic",
                      "config": {"workload": "sequence-length sweep", "H": H, "D": D, "M": M, "tokens": total},
                      "rows": rows}))


def memory_report(step):
    """Device memory the library needs beside the I/O tensors (checkpoint of segment states and workspaces), what
    storing the state S_i of every token would take instead (B*H*N*D*M float32), and the run's peak allocation."""
    import torch

    w = step.w
    out = {"peak_device_bytes": int(torch.cuda.max_memory_allocated())}
    if step.args.workload == "decode":
        return out
    lib = 0
    for name in ("ck", "ws_f", "ws_b", "ws_n", "ws_nb"):
        t = getattr(step, name, None)
        if t is not None:
            lib += t.numel() * t.element_size()
    d = getattr(w, "features", None) or w.D
    out.update({"checkpoint_and_workspace_bytes": int(lib), "stored_states_bytes": w.B * w.H * w.N * d * w.M * 4})
    return out


def summarize_stats(args):
    import csv

    rows = list(csv.DictReader(open(args.summarize_stats)))
    os.makedirs(PROFILES, exist_ok=True)
    path = os.path.join(PROFILES, f"{args.label}_kernels.md")
    with open(path, "w") as f:
        f.write(f"# rocprofv3 kernel statistics: {args.label} workload\n\n")
        f.write(f"Command (run from the repository root on one MI355X):\n\n    {args.command}\n\n")
        f.write(f"Kernel sources: sha256[:16] = {source_hash()}\n\n")
        f.write("| kernel | template | calls | average us | min us | max us | share of GPU time |\n|---|---|---|---|---|---|---|\n")
        for r in rows:
            name = r["Name"]
            tmpl = name.split("(")[0].replace("void ", "")
            f.write(f"| {kernel_tag(name)} | `{tmpl}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                    f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |\n")
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
        f.write("| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes/launch (scaled) | algorithmic bytes | ratio |\n")
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
    from linear_rnn_layers_amd import inputs

    w = WORKLOADS(inputs)[args.label]
    md = os.path.join(PROFILES, f"{args.label}_mfma.md")
    with open(md, "w") as f:
        f.write(f"# MFMA utilisation from rocprofv3 counters: {args.label} workload\n\n")
        f.write(f"Commands (run from the repository root on one MI355X):\n\n    {args.command}\n\n")
        f.write(f"Kernel sources: sha256[:16] = {source_hash()}\n\n")
        f.write("Executed MFMA flops = SQ_INSTS_MFMA x 16384 (every matrix instruction is v_mfma_f32_16x16x32_bf16, "
                "split-precision products included) over the kernel's average duration from the kernel statistics; "
                f"MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (duration x {CLOCK_GHZ} GHz x {SIMDS} SIMDs); useful "
                "flops are the method's own per token-head counts (forward 4DM+5D+M, backward 10DM+9D+3M). "
                f"Peak: {MFMA_BF16_PEAK_TFLOPS:.0f} TFLOP/s dense bf16.\n\n")
        f.write("| kernel | dispatches | SQ_INSTS_MFMA | SQ_INSTS_VALU | avg us | executed MFMA TFLOP/s | of bf16 peak "
                "| MFMA busy | useful TFLOP/s |\n|---|---|---|---|---|---|---|---|---|\n")
        for k in sorted(inst, key=lambda x: -inst[x]):
            tag = kernel_tag(k)
            if "la::" not in k or tag not in dur:
                continue
            t = dur[tag]
            ex = inst[k] * MFMA_FLOPS_PER_INST / t / 1e12
            b = busy.get(k, 0.0) / (t * CLOCK_GHZ * 1e9 * SIMDS)
            fl = kernel_flops(tag, w)
            useful = f"{fl / t / 1e12:.1f}" if fl else "-"
            f.write(f"| {tag} | {n[k]} | {inst[k]:.4g} | {valu.get(k, 0.0):.4g} | {t * 1e6:.1f} | {ex:.1f} | "
                    f"{ex / MFMA_BF16_PEAK_TFLOPS * 100:.1f}% | {b * 100:.1f}% | {useful} |\n")
    print(md)


def copy_bandwidth():
    """Achievable streaming bandwidth on this GPU: a plain 512 MiB device-to-device copy, GB/s of bytes
    read + written."""
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


# ------------------------------------------------------------ cpu baseline
def cpu_baseline(args, w):
    import numpy as np

    import oracle

    oracle.build()
    wl = args.workload
    if wl == "decode":
        nheads = 64  # bounded sample: 64 of the 4096 heads, 512 steps each
        steps = 512
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
        value = steps / el * nheads / (w.B * w.H)
        return {"value": value, "unit": "decode steps/s (all B*H heads)", "cores": oracle.num_threads(),
                "kind": "oracle", "sample": f"{steps} steps on {nheads} of {w.B * w.H} heads, scaled to all heads"}
    # token workloads: run the oracle's passes of one step on a subset of heads until >= 10 s
    B, H, N = w.B, w.H, w.N
    nb = {"mnist": 4, "cifar": 1, "long": 1, "long-decay": 1, "mnist-rf": 4, "speech": 4, "small": 1}[wl]
    nh = {"mnist": H, "cifar": 8, "long": 2, "long-decay": 2, "mnist-rf": H, "speech": H, "small": 1}[wl]
    n = {"mnist": N, "cifar": N, "long": 16384, "long-decay": 8192, "mnist-rf": N, "speech": N, "small": N}[wl]
    q, k, v = (a[:nb, :nh, :n] for a in w.qkv(n=n))
    do = w.grad_out(n=n)[:nb, :nh, :n]
    reps = 0
    t = time.perf_counter()
    la = w.log_a(n=n)[:nb, :nh, :n] if wl == "long-decay" else None
    wp = w.projection() if wl == "mnist-rf" else None
    while True:
        if wl == "mnist-rf":
            fq, fk = oracle.feature_performer(q, wp[:nh]), oracle.feature_performer(k, wp[:nh])
            oracle.forward_causal(fq, fk, v, feature=1)
            dfq, dfk, _ = oracle.backward_causal(fq, fk, v, do, feature=1)
            oracle.feature_performer_vjp(q, wp[:nh], dfq)
            oracle.feature_performer_vjp(k, wp[:nh], dfk)
            reps += 1
            el = time.perf_counter() - t
            if el >= 10.0 or reps >= 1000:
                break
            continue
        if wl == "long-decay":
            oracle.forward_decay(q, k, v, la)
            oracle.backward_decay(q, k, v, la, do)
            reps += 1
            el = time.perf_counter() - t
            if el >= 10.0 or reps >= 1000:
                break
            continue
        if wl == "speech":
            oracle.forward_noncausal(q, k, v)
            oracle.backward_noncausal(q, k, v, do)
            reps += 1
            el = time.perf_counter() - t
            if el >= 10.0 or reps >= 1000:
                break
            continue
        o_ref, den_ref, _, _ = oracle.forward_causal(q, k, v)
        ref = {"O": o_ref, "den": den_ref}
        if wl != "small":
            ref["dQ"], ref["dK"], ref["dV"] = oracle.backward_causal(q, k, v, do)
        if wl == "mnist":
            ref["O_noncausal"] = oracle.forward_noncausal(q, k, v)
        reps += 1
        el = time.perf_counter() - t
        if el >= 10.0 or reps >= 1000:
            break
    head_tokens_per_s = reps * nb * nh * n / el
    layers = w.layers if wl in ("cifar", "speech") else 1
    value = head_tokens_per_s / (H * layers)  # model tokens/s: every token goes through H heads (x layers)
    out = {"value": value, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
           "sample": f"{reps} x one step's passes on {nb}x{nh} of {B}x{H} sequences, {n} of {N} tokens"
                     f"{f', scaled to {layers} layers' if layers > 1 else ''}"}
    if wl in ("mnist", "cifar", "small") and n == N:
        out["_ref"] = (ref, nb, nh)  # whole sequences of the first input set: the GPU step can be compared
    return out


def sample_parity(step, ref, nb, nh):
    """The GPU path on the first input set (one untimed step) against the oracle outputs of the CPU-baseline
    sample: per tensor, the largest over the sampled heads of max|gpu - oracle| / max|oracle|."""
    import numpy as np
    import torch

    b = step.b
    q, k, v, do = step.sets[0]
    b.la_forward_causal(q, k, v, step.o, step.den, ckpt=step.ck, ws=step.ws_f)
    got = {}
    if "dQ" in ref:
        b.la_backward_causal(q, k, v, step.o, step.den, do, step.dq, step.dk, step.dv, ckpt=step.ck, ws=step.ws_b)
        got.update(dQ=step.dq, dK=step.dk, dV=step.dv)
    if "O_noncausal" in ref:
        b.la_forward_noncausal(q, k, v, step.onc, ws=step.ws_n)
        got["O_noncausal"] = step.onc
    got.update(O=step.o, den=step.den)
    torch.cuda.synchronize()
    res = {}
    for name, y in ref.items():
        x = got[name][:nb, :nh].float().cpu().numpy().astype(np.float64)
        y = np.asarray(y, dtype=np.float64)
        ax = tuple(range(2, y.ndim))
        res[name] = float((np.abs(x - y).max(axis=ax) / np.abs(y).max(axis=ax)).max())
    return res


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
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; heads are independent, so more GPUs "
                                   "shard B*H with no communication (see DESIGN.md)", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    torch.cuda.set_device(0)
    if args.copy_only:
        n = args.copy_only * (1 << 20) // 4
        a = torch.ones(n, device="cuda")
        bb = torch.empty_like(a)
        for _ in range(max(1, args.steps)):
            bb.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "launches": max(1, args.steps)}))
        return

    if args.seq_sweep:
        seq_sweep(args)
        return

    from linear_rnn_layers_amd import binding

    step = Step(args)
    w = step.w
    s = 4 if w.dtype == "f32" else 2
    names = binding.kernel_names()
    graphs = args.workload == "decode" and bool(step.graphs)
    if graphs:
        step.run(args.warmup)
    else:
        for _ in range(args.warmup):
            step()
    torch.cuda.synchronize()

    # per-kernel durations over a few untimed steps, to find the dominant kernel
    probe = {}
    nprobe = 5 if args.workload != "decode" else 50
    for name in names:
        binding.prof_select(name)
        for _ in range(nprobe):
            step()
        torch.cuda.synchronize()
        ms, n, _ = binding.prof_collect()
        if n:
            probe[name] = {"ms_per_step": ms / nprobe, "launches_per_step": n / nprobe}
    binding.prof_select(None)
    dominant = max(probe, key=lambda k: probe[k]["ms_per_step"])

    # timed region: exactly `steps` steps between synchronisations; the library records a pair of
    # HIP events on the launch stream around every launch of the dominant kernel
    # (decode with graphs: a pair of events around every graph replay instead; the per-launch duration is then
    # the replay time over its 64 back-to-back launches, gaps included)
    gev = [] if graphs and not args.no_kernel_events else None
    if not args.no_kernel_events and not graphs:
        binding.prof_select(dominant)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graphs:
        step.run(args.steps, gev)
    else:
        for _ in range(args.steps):
            step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kms, kn, dropped = binding.prof_collect()
    binding.prof_select(None)
    if gev:
        kms, kn = sum(e0.elapsed_time(e1) for e0, e1 in gev), len(gev) * DECODE_GRAPH
    el = t1 - t0
    ms_per_step = el * 1e3 / args.steps

    if args.workload == "decode":
        metric, unit = "decode steps/s", "steps/s"
        value = args.steps / el
    elif args.workload == "speech":
        metric, unit = "non-causal linear-attn fwd+bwd tokens/s", "tokens/s"
        value = w.B * w.N * args.steps / el
    elif args.workload == "mnist-rf":
        metric, unit = "random-feature causal linear-attn fwd+bwd tokens/s", "tokens/s"
        value = w.B * w.N * args.steps / el
    elif args.workload == "long-decay":
        metric, unit = "decayed causal linear-attn fwd+bwd tokens/s", "tokens/s"
        value = w.B * w.N * args.steps / el
    else:
        metric, unit = "causal linear-attn fwd+bwd tokens/s", "tokens/s"
        value = w.B * w.N * args.steps / el

    roof = None
    if kn:
        avg_s = kms / kn / 1e3
        byts = kernel_bytes(dominant, w, s)
        achieved = byts / avg_s / 1e9 if byts else None
        traffic = traffic_from_profiles(dominant, args.workload)
        roof = {"kernel": dominant, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS if achieved else None, "traffic": traffic,
                "algorithmic_bytes_per_launch": byts, "avg_launch_us": avg_s * 1e6, "launches": kn}
        if gev:
            roof["timing"] = f"events around each replay of a graph of {DECODE_GRAPH} launches, divided by {DECODE_GRAPH}"
        fl = kernel_flops(dominant, w)
        if fl:
            roof["useful_tflops"] = fl / avg_s / 1e12
        copy = copy_bandwidth()
        roof["copy_gbs"] = copy
        roof["frac_of_copy"] = achieved / copy if achieved else None

    dist = step_distribution(step, graphs)
    mem = memory_report(step)
    breakdown = {k: {"us_per_step": round(v["ms_per_step"] * 1e3, 2),
                     "launches_per_step": v["launches_per_step"]} for k, v in probe.items()}
    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args, w)
        if "_ref" in cpu:
            ref, nb, nh = cpu.pop("_ref")
            parity = {"sample": f"first input set, {nb}x{nh} sequences of {w.B}x{w.H}, one untimed step",
                      "measure": "max over sampled heads of max|gpu - oracle| / max|oracle| per tensor",
                      "tolerance": 1e-4 if s == 4 else 2e-2, **sample_parity(step, ref, nb, nh)}

    cfg = {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "D": w.D, "M": w.M, "gpus": 1}
    if args.workload == "mnist":
        cfg["step"] = "causal forward + causal backward + non-causal forward"
    elif args.workload == "cifar":
        cfg["step"] = "16 layers x (causal forward + backward)"
        cfg["layers"] = 16
    elif args.workload == "long":
        cfg["step"] = "causal forward + backward"
    elif args.workload == "long-decay":
        cfg["step"] = "decayed causal forward + backward (dQ, dK, dV, dlogA)"
    elif args.workload == "mnist-rf":
        cfg["step"] = "random features of Q, K (C = 64) + causal forward and backward on them + chain rule to Q, K"
        cfg["features"] = w.features
    elif args.workload == "speech":
        cfg["step"] = "9 layers x (non-causal forward + backward)"
        cfg["layers"] = 9
    elif args.workload == "decode":
        cfg["step"] = "one decode step of all B*H heads after a 512-token prefill"
        cfg["launch"] = f"HIP graphs of {DECODE_GRAPH} steps" if graphs else "one host launch per step"
    else:
        cfg["step"] = "causal forward"
    out = {"metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f32" if s == 4 else "bf16", "data": "synthetic", "config": cfg,
           "roofline": roof, "cpu_baseline": cpu, "parity": parity, "step_us": dist, "memory": mem,
           "gpu": torch.cuda.get_device_name(0), "rocm": torch.version.hip, "seeds": list(w.seeds),
           "kernels_us_per_step": breakdown,
           "kernel_events_in_timed_region": not args.no_kernel_events, "events_dropped": dropped}
    print(json.dumps(out))


if __name__ == "__main__":
    main()
