#!/usr/bin/env python3
"""Throughput of the HyFlash drafter-layer hot path on one MI355X.

Headline step: batched serving on one GPU, the largest single-GPU workload.  The Qwen3-4B-shaped
drafter layer (bf16, d_model 2560, 32 heads x 80, d_state 128, chunk 64, window 512, block 7 +
anchor) serves 64 requests with per-request states and rings.  A step resets the 64 states,
commits their prefixes (U{2048..16384} features each, one hyf_memory_commit call), then runs 128
verification rounds; in each round every request commits its 1-8 accepted features and drafts its
block, all 64 in one hyf_draft_block call.  `value` = draft blocks/s over whole steps (prefill
included), summed over the requests.  Inputs are seeded synthetic arrays (NumPy PCG64 streams,
seed 3), resident in HBM before the timed region.

`roofline` is the round's dominant kernel at this shape, the round kernel with one workgroup per
(request, head) (k_round_pair): algorithmic bytes per launch (ring windows, H read and written,
the append, the projection columns it reads, its output) over its average duration, measured with HIP events as a graph of the 128 rounds minus a graph
of the same rounds' two projections (the same kernels and launch shapes, run through hyf_linear).
`round` is the whole round against its algorithmic bytes.

Sub-objects: the batch-1 Qwen3-4B-shaped episode (8192-feature prefix, 256 rounds; eight
requests' episodes interleaved and seven weight copies rotated so the figures are HBM figures),
the Phi-4-shaped two-layer drafter (32768-feature prefix, 512 rounds), the long-context
Phi-4-shaped layer (131072-feature prefix, chunk 256, 128 rounds; Mamba-2 and the gated delta
rule), kernel loops (commit scan, prefill GEMM, round projections, 4-bit projections), and the
CPU oracle's rate on a bounded sample of the headline workload.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "committed feats/s (SSD commit scan) + draft blocks/s per layer; % roofline"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
W_COPIES = 7                 # 7 x 54 MB of Qwen-shaped weights > 256 MB last-level cache
SCAN_COPIES = 6              # 6 x 46 MB of scan inputs
EPISODES = 8                 # interleaved batch-1 episodes (8 states of 6.6 MB)
HEADLINE = "qwen3_4b_batched64"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--kernel-reps", type=int, default=60)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    p.add_argument("--profile", action="store_true", help="short run for a profiler (few steps and reps)")
    p.add_argument("--pmc-probe", action="store_true",
                   help="only the measured kernels (plus a copy of known size), for rocprofv3 --pmc runs")
    p.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                   help="turn two rocprofv3 --pmc databases (FETCH_SIZE, WRITE_SIZE) of --pmc-probe runs "
                        "into profiles/pmc_traffic.json and .md")
    p.add_argument("--stats-summary", metavar="DIR",
                   help="turn the csv output of a rocprofv3 --kernel-trace --stats run of --profile (output "
                        "prefix 'bench') into profiles/bench_kernel_stats.md")
    return p.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# ---- inputs --------------------------------------------------------------------------------------


def device_rows(torch, rng, n, d, scale, chunk=65536):
    """n x d rows ~ N(0, 1) * scale drawn on the host from `rng` (float32, in chunks), cast to bf16
    (round to nearest even) and placed on the device."""
    import numpy as np

    out = torch.empty((max(n, 1), d), dtype=torch.bfloat16, device="cuda")
    for i in range(0, n, chunk):
        m = min(chunk, n - i)
        a = rng.standard_normal((m, d), dtype=np.float32) * np.float32(scale)
        out[i:i + m].copy_(torch.from_numpy(a).to(torch.bfloat16))
    return out


class Calls:
    """Prebuilt C-ABI arguments (ctypes) so that a step's host side is a loop of library calls."""

    def __init__(self, hf, cfg, weights):
        self.L = hf.lib()
        self.cfg = cfg
        self.cfg_ref = ctypes.byref(cfg)
        self.w = weights if isinstance(weights, list) else [weights]
        self.w_ref = [ctypes.byref(x) for x in self.w]

    @staticmethod
    def i64(vals):
        return (ctypes.c_int64 * len(vals))(*[int(v) for v in vals])


def weights_struct(hf, w_in, w_out, a_log, dt_bias, d_skip):
    return hf.HyfWeights(w_in.data_ptr(), w_out.data_ptr(), a_log.data_ptr(), dt_bias.data_ptr(), d_skip.data_ptr())


def layer_weights(torch, hf, I, shape, rng, copies=1):
    """Device weights of one layer (`copies` copies of the projection weights) and their C structs.
    With 4-bit weights (shape.weights == "w4") the projections get random codes and scales: the
    timing does not depend on their values."""
    w = I.make_weights(shape, rng)
    vec = [hf.to_device(w[k], shape, storage=False) for k in ("a_log", "dt_bias", "d_skip")]
    if shape.weights == "w4":
        q = []
        for _ in range(copies):
            qi, si = I.random_w4(rng, shape.n_in, shape.d_model)
            qo, so = I.random_w4(rng, shape.d_model, shape.dq)
            q.append([torch.from_numpy(a).cuda() for a in (qi, si, qo, so)])
        structs = [hf.HyfWeights(None, None, *[v.data_ptr() for v in vec], *[a.data_ptr() for a in q[i]])
                   for i in range(copies)]
        return w, dict(w_in=None, w_out=None, q=q, vec=vec, structs=structs)
    w_in = [hf.to_device(w["w_in"], shape) for _ in range(copies)]
    w_out = [hf.to_device(w["w_out"], shape) for _ in range(copies)]
    structs = [weights_struct(hf, w_in[i], w_out[i], *vec) for i in range(copies)]
    return w, dict(w_in=w_in, w_out=w_out, vec=vec, structs=structs)


# ---- algorithmic bytes ---------------------------------------------------------------------------


def kround_bytes(sh, R, rows, windows):
    """Bytes the round kernel must move once: each request's ring window (K and V of `windows[i]`
    slots) read, H read and written, the committed rows' k and v appended to the ring, the fp32
    projection columns it consumes (q, C, k, v of the block rows; k, v, B, step of the committed
    rows) and its bf16 output (the output projection's input)."""
    es = 2
    nh, P, N = sh.n_heads, sh.head_dim, sh.d_state
    ring = sum(windows) * nh * P * 2 * es
    h = 2 * R * nh * P * N * 4
    append = rows * nh * P * 2 * es
    proj = (8 * R * (3 * sh.dq + sh.gn) + rows * (2 * sh.dq + sh.gn + sh.n_heads)) * 4
    out = 8 * R * sh.dq * es
    return ring + h + append + proj + out


def round_bytes(sh, R, rows, windows):
    """Bytes a whole round must move once: w_in and w_out, the committed and block rows in, the
    block rows out, the ring windows read, the append, H read and written."""
    es = 2
    nh, P, N, d = sh.n_heads, sh.head_dim, sh.d_state, sh.d_model
    weights = (sh.n_in + sh.dq) * d * es
    rows_io = (rows + 8 * R + 8 * R) * d * es
    ring = sum(windows) * nh * P * 2 * es
    return weights + rows_io + ring + rows * nh * P * 2 * es + 2 * R * nh * P * N * 4


def scan_bytes(sh, T):
    return T * (sh.n_heads * sh.head_dim * 2 + sh.gn * 2 + sh.n_heads * 4) + 2 * sh.n_heads * sh.head_dim * sh.d_state * 4


# ---- timing --------------------------------------------------------------------------------------


def time_graph(torch, fn, reps, replays=3, stream=None):
    """Mean microseconds per call of `reps` calls captured in one HIP graph, replayed `replays`
    times between HIP events recorded on the replay stream."""
    g = torch.cuda.CUDAGraph()
    s = stream or torch.cuda.Stream()
    with torch.cuda.stream(s):
        fn(0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        for i in range(reps):
            fn(i)
    with torch.cuda.stream(s):
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(replays):
            g.replay()
        e1.record(s)
    torch.cuda.synchronize()
    del g
    return 1e3 * e0.elapsed_time(e1) / (replays * reps)


def time_calls(torch, fn, reps):
    """Mean microseconds per call: HIP events on the current stream around `reps` back-to-back calls."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(reps):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return 1e3 * e0.elapsed_time(e1) / reps


def run_steps(torch, step, steps, warmup):
    """Eager steps on torch's current stream; events around the prefill and the rounds of each."""
    stream = torch.cuda.current_stream().cuda_stream
    for _ in range(warmup):
        step(stream)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for k in range(steps):
        step(stream, evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    step_ms = [e[0].elapsed_time(e[2]) for e in evs]
    pre_ms = [e[0].elapsed_time(e[1]) for e in evs]
    rnd_ms = [e[1].elapsed_time(e[2]) for e in evs]
    mean = lambda v: sum(v) / len(v)
    return dict(step_ms=mean(step_ms), prefill_ms=mean(pre_ms), rounds_ms=mean(rnd_ms), wall_s=wall)


def hbm(bytes_, us):
    gbs = bytes_ / (us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS}


# ---- workloads -----------------------------------------------------------------------------------


class Batched:
    """Batched serving: 64 Qwen3-4B-shaped requests, prefixes U{2048..16384}, 128 rounds."""

    def __init__(self, torch, hf, I, name=HEADLINE):
        import numpy as np

        wl = I.WORKLOADS[name]
        self.shape = sh = wl["shape"]
        self.R = R = wl["requests"]
        self.rounds = wl["rounds"]
        d = sh.d_model
        rng = I.rng_streams(wl["seed"])
        self.host_w, self.wd = layer_weights(torch, hf, I, sh, rng[0])
        lo, hi = wl["prefix_range"]
        self.lens = rng[4].integers(lo, hi + 1, size=R)
        self.acc = rng[4].integers(1, 9, size=(self.rounds, R))
        self.T = int(self.lens.sum())
        log(f"batched: drawing {self.T} prefix rows")
        self.prefix = device_rows(torch, rng[1], self.T, d, wl["feat_scale"])
        self.commits = device_rows(torch, rng[2], int(self.acc.sum()), d, wl["feat_scale"])
        self.blocks = device_rows(torch, rng[3], self.rounds * R * 8, d, wl["block_scale"])
        self.out = torch.empty((R * 8, d), dtype=torch.bfloat16, device="cuda")
        self.cfg = hf.make_config(sh)
        self.c = Calls(hf, self.cfg, self.wd["structs"])
        self.state_bytes = hf.hyf_state_bytes(self.cfg)
        self.pool = torch.zeros(R * self.state_bytes, dtype=torch.uint8, device="cuda")
        self.ws_bytes = hf.hyf_workspace_bytes(self.cfg, R, self.T)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device="cuda")
        self.cu_pre = Calls.i64(np.concatenate([[0], np.cumsum(self.lens)]))
        self.cu = [Calls.i64(np.concatenate([[0], np.cumsum(a)])) for a in self.acc]
        offs = np.concatenate([[0], np.cumsum(self.acc.sum(axis=1))])
        es = 2
        self.c_ptr = [ctypes.c_void_p(self.commits.data_ptr() + int(offs[i]) * d * es) for i in range(self.rounds)]
        self.b_ptr = [ctypes.c_void_p(self.blocks.data_ptr() + i * R * 8 * d * es) for i in range(self.rounds)]
        self.pool_p, self.ws_p = ctypes.c_void_p(self.pool.data_ptr()), ctypes.c_void_p(self.ws.data_ptr())
        self.pre_p, self.out_p = ctypes.c_void_p(self.prefix.data_ptr()), ctypes.c_void_p(self.out.data_ptr())
        self.windows = [min(int(n), sh.window) for n in self.lens]

    def reset_and_prefill(self, s):
        L, c = self.c.L, self.c
        st = L.hyf_state_reset(c.cfg_ref, self.pool_p, self.R, None, self.R, s)
        st |= L.hyf_memory_commit(c.cfg_ref, c.w_ref[0], self.pool_p, self.R, None, self.R, self.pre_p, self.cu_pre,
                                  None, self.ws_p, self.ws_bytes, s)
        return st

    def round(self, i, s):
        c = self.c
        return c.L.hyf_draft_block(c.cfg_ref, c.w_ref[0], self.pool_p, self.R, None, self.R, self.c_ptr[i], self.cu[i],
                                   self.b_ptr[i], self.out_p, self.ws_p, self.ws_bytes, s)

    def step(self, stream, ev=None):
        s = ctypes.c_void_p(stream)
        if ev:
            ev[0].record()
        st = self.reset_and_prefill(s)
        if ev:
            ev[1].record()
        for i in range(self.rounds):
            st |= self.round(i, s)
        if ev:
            ev[2].record()
        if st:
            raise RuntimeError(f"libhyflash call failed (status bits {st})")

    def round_kernel(self, torch, hf, nr=None):
        """Per-round microseconds of the rounds (graph) and of their two projections alone (graph of
        hyf_linear calls with the same shapes), and the round kernel's share (the difference)."""
        import numpy as np

        nr = nr or self.rounds
        sh, R, d = self.shape, self.R, self.shape.d_model
        st = [0]
        stream = torch.cuda.Stream()

        def rounds(i):
            st[0] |= self.round(i % self.rounds, ctypes.c_void_p(stream.cuda_stream))

        t_round = time_graph(torch, rounds, nr, stream=stream)
        M = [int(self.acc[i % self.rounds].sum()) + 8 * R for i in range(nr)]
        y = torch.empty((max(M), sh.n_in), dtype=torch.float32, device="cuda")
        xo = torch.empty((8 * R, sh.dq), dtype=torch.bfloat16, device="cuda").normal_()
        xin = torch.empty((max(M), d), dtype=torch.bfloat16, device="cuda").normal_()
        # In a round the round kernel streams its 531 MB between two rounds' projections, so their
        # weights come from HBM; the projection-only graph rotates W_COPIES weight copies (more than
        # the last-level cache holds) to price them the same way.
        w_in = [torch.empty_like(self.wd["w_in"][0]).normal_() for _ in range(W_COPIES)]
        w_out = [torch.empty_like(self.wd["w_out"][0]).normal_() for _ in range(W_COPIES)]

        def projs(i):
            s = stream.cuda_stream
            st[0] |= hf.hyf_linear(self.cfg, xin, M[i], d, w_in[i % W_COPIES], sh.n_in, y, 1, s)
            st[0] |= hf.hyf_linear(self.cfg, xo, 8 * R, sh.dq, w_out[i % W_COPIES], d, self.out, 0, s)

        t_proj = time_graph(torch, projs, nr, stream=stream)
        if st[0]:
            raise RuntimeError(f"round kernel timing failed (status bits {st[0]})")
        rows = float(np.mean(self.acc[:nr].sum(axis=1)))
        return t_round, t_proj, rows


class EpisodesB1:
    """The batch-1 Qwen3-4B-shaped episode (8192-feature prefix commit, 256 rounds), EPISODES
    requests' episodes interleaved (each call is batch 1, on its own state) with W_COPIES weight
    copies rotated call by call, so weights and states come from HBM."""

    def __init__(self, torch, hf, I, name="qwen3_4b_bf16", memory="mamba2", weights="dense"):
        import numpy as np

        wl = I.WORKLOADS[name]
        self.shape = sh = wl["shape"].replace(memory=memory, weights=weights)
        self.T, self.rounds = wl["prefix"], wl["rounds"]
        d = sh.d_model
        rng = I.rng_streams(wl["seed"])
        self.host_w, self.wd = layer_weights(torch, hf, I, sh, rng[0], copies=W_COPIES)
        self.prefix = device_rows(torch, rng[1], self.T, d, wl["feat_scale"])
        self.acc = rng[4].integers(1, 9, size=self.rounds)
        self.commits = device_rows(torch, rng[2], int(self.acc.sum()), d, wl["feat_scale"])
        self.blocks = device_rows(torch, rng[3], self.rounds * 8, d, wl["block_scale"])
        self.out = torch.empty((8, d), dtype=torch.bfloat16, device="cuda")
        self.cfg = hf.make_config(sh)
        self.c = Calls(hf, self.cfg, self.wd["structs"])
        self.state_bytes = hf.hyf_state_bytes(self.cfg)
        self.pool = torch.zeros(EPISODES * self.state_bytes, dtype=torch.uint8, device="cuda")
        self.ws_bytes = hf.hyf_workspace_bytes(self.cfg, 1, self.T)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device="cuda")
        self.cu_pre = Calls.i64([0, self.T])
        self.cu = [Calls.i64([0, a]) for a in self.acc]
        offs = np.concatenate([[0], np.cumsum(self.acc)])
        es = 2
        self.c_ptr = [ctypes.c_void_p(self.commits.data_ptr() + int(offs[i]) * d * es) for i in range(self.rounds)]
        self.b_ptr = [ctypes.c_void_p(self.blocks.data_ptr() + i * 8 * d * es) for i in range(self.rounds)]
        self.slots = [(ctypes.c_int32 * 1)(e) for e in range(EPISODES)]
        self.pool_p, self.ws_p = ctypes.c_void_p(self.pool.data_ptr()), ctypes.c_void_p(self.ws.data_ptr())
        self.pre_p, self.out_p = ctypes.c_void_p(self.prefix.data_ptr()), ctypes.c_void_p(self.out.data_ptr())
        self.k = 0

    def round(self, e, i, s):
        c = self.c
        self.k = (self.k + 1) % W_COPIES
        return c.L.hyf_draft_block(c.cfg_ref, c.w_ref[self.k], self.pool_p, EPISODES, self.slots[e], 1, self.c_ptr[i],
                                   self.cu[i], self.b_ptr[i], self.out_p, self.ws_p, self.ws_bytes, s)

    def step(self, stream, ev=None):
        L, c = self.c.L, self.c
        s = ctypes.c_void_p(stream)
        if ev:
            ev[0].record()
        st = L.hyf_state_reset(c.cfg_ref, self.pool_p, EPISODES, None, EPISODES, s)
        for e in range(EPISODES):
            self.k = (self.k + 1) % W_COPIES
            st |= L.hyf_memory_commit(c.cfg_ref, c.w_ref[self.k], self.pool_p, EPISODES, self.slots[e], 1, self.pre_p,
                                      self.cu_pre, None, self.ws_p, self.ws_bytes, s)
        if ev:
            ev[1].record()
        for i in range(self.rounds):
            for e in range(EPISODES):
                st |= self.round(e, i, s)
        if ev:
            ev[2].record()
        if st:
            raise RuntimeError(f"libhyflash call failed (status bits {st})")

    def round_graph(self, torch, nr=64):
        """Microseconds per round of `nr` rounds captured in one HIP graph (interleaved states)."""
        st = [0]
        stream = torch.cuda.Stream()

        def rounds(i):
            st[0] |= self.round(i % EPISODES, (i // EPISODES) % self.rounds, ctypes.c_void_p(stream.cuda_stream))

        t = time_graph(torch, rounds, nr, stream=stream)
        if st[0]:
            raise RuntimeError("round graph failed")
        return t

    def round_kernel(self, torch, hf, nr=64):
        """As Batched.round_kernel, for batch-1 rounds over the interleaved states."""
        sh, d = self.shape, self.shape.d_model
        st = [0]
        stream = torch.cuda.Stream()

        def rounds(i):
            st[0] |= self.round(i % EPISODES, (i // EPISODES) % self.rounds, ctypes.c_void_p(stream.cuda_stream))

        t_round = time_graph(torch, rounds, nr, stream=stream)
        M = [int(self.acc[(i // EPISODES) % self.rounds]) + 8 for i in range(nr)]
        y = torch.empty((16, sh.n_in), dtype=torch.float32, device="cuda")
        xo = torch.empty((8, sh.dq), dtype=torch.bfloat16, device="cuda").normal_()
        xin = torch.empty((16, d), dtype=torch.bfloat16, device="cuda").normal_()
        kk = [0]

        def projs(i):
            s = stream.cuda_stream
            kk[0] = (kk[0] + 1) % W_COPIES
            if sh.weights == "w4":
                qi, si, qo, so = self.wd["q"][kk[0]]
                st[0] |= hf.hyf_linear_w4(self.cfg, xin, M[i], d, qi, si, sh.n_in, y, 1, s)
                st[0] |= hf.hyf_linear_w4(self.cfg, xo, 8, sh.dq, qo, so, d, self.out, 0, s)
            else:
                st[0] |= hf.hyf_linear(self.cfg, xin, M[i], d, self.wd["w_in"][kk[0]], sh.n_in, y, 1, s)
                st[0] |= hf.hyf_linear(self.cfg, xo, 8, sh.dq, self.wd["w_out"][kk[0]], d, self.out, 0, s)

        t_proj = time_graph(torch, projs, nr, stream=stream)
        if st[0]:
            raise RuntimeError(f"round kernel timing failed (status bits {st[0]})")
        rows = sum(M) / len(M) - 8
        return t_round, t_proj, rows


class EpisodesBlockB1(EpisodesB1):
    """The batch-1 episode of the full drafter block around the Qwen3-4B-shaped layer (pre-norms,
    residuals, SwiGLU MLP of width 3 d_model): prefix commit through hyf_block_commit, rounds through
    hyf_block_draft; layer and MLP weights rotated over W_COPIES copies."""

    def __init__(self, torch, hf, I):
        import numpy as np

        super().__init__(torch, hf, I)
        sh = self.shape
        bw = I.make_block_weights(sh, I.rng_streams(77)[0])
        self.F = bw["w_gate"].shape[0]
        self.norms = [torch.from_numpy(bw[k]).cuda() for k in ("norm1", "norm2")]
        gu = np.concatenate([bw["w_gate"], bw["w_up"]], axis=0)
        self.mlp = [(hf.to_device(gu, sh), hf.to_device(bw["w_down"], sh)) for _ in range(W_COPIES)]
        self.bws = [hf.HyfBlockWeights(self.norms[0].data_ptr(), self.norms[1].data_ptr(), g.data_ptr(),
                                       dn.data_ptr(), self.F, float(bw["eps"])) for g, dn in self.mlp]
        self.bw_ref = [ctypes.byref(b) for b in self.bws]
        self.ws_bytes = hf.hyf_block_workspace_bytes(self.cfg, self.bws[0], 1, self.T)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device="cuda")
        self.ws_p = ctypes.c_void_p(self.ws.data_ptr())

    def round(self, e, i, s):
        c = self.c
        self.k = (self.k + 1) % W_COPIES
        return c.L.hyf_block_draft(c.cfg_ref, c.w_ref[self.k], self.bw_ref[self.k], self.pool_p, EPISODES,
                                   self.slots[e], 1, self.c_ptr[i], self.cu[i], self.b_ptr[i], self.out_p, self.ws_p,
                                   self.ws_bytes, s)

    def step(self, stream, ev=None):
        L, c = self.c.L, self.c
        s = ctypes.c_void_p(stream)
        if ev:
            ev[0].record()
        st = L.hyf_state_reset(c.cfg_ref, self.pool_p, EPISODES, None, EPISODES, s)
        for e in range(EPISODES):
            self.k = (self.k + 1) % W_COPIES
            st |= L.hyf_block_commit(c.cfg_ref, c.w_ref[self.k], self.bw_ref[self.k], self.pool_p, EPISODES,
                                     self.slots[e], 1, self.pre_p, self.cu_pre, self.ws_p, self.ws_bytes, s)
        if ev:
            ev[1].record()
        for i in range(self.rounds):
            for e in range(EPISODES):
                st |= self.round(e, i, s)
        if ev:
            ev[2].record()
        if st:
            raise RuntimeError(f"libhyflash call failed (status bits {st})")


class TwoLayerPhi4:
    """The Phi-4-shaped two-layer drafter: both layers commit the 32768-feature prefix, then 512
    rounds; in each, both layers commit the round's accepted features, layer 1 drafts the block and
    layer 2 drafts from block_in + layer 1's output (the residual add between the two calls is the
    caller's, in torch: the layer ends at its output projection)."""

    def __init__(self, torch, hf, I, name="phi4_bf16_2layer"):
        import numpy as np

        wl = I.WORKLOADS[name]
        self.shape = sh = wl["shape"]
        self.T, self.rounds = wl["prefix"], wl["rounds"]
        d = sh.d_model
        rng = I.rng_streams(wl["seed"])
        self.layers = [layer_weights(torch, hf, I, sh, rng[0])[1], layer_weights(torch, hf, I, sh, rng[5])[1]]
        self.prefix = device_rows(torch, rng[1], self.T, d, wl["feat_scale"])
        self.acc = rng[4].integers(1, 9, size=self.rounds)
        self.commits = device_rows(torch, rng[2], int(self.acc.sum()), d, wl["feat_scale"])
        self.blocks = device_rows(torch, rng[3], self.rounds * 8, d, wl["block_scale"])
        self.o1 = torch.empty((8, d), dtype=torch.bfloat16, device="cuda")
        self.x2 = torch.empty((8, d), dtype=torch.bfloat16, device="cuda")
        self.o2 = torch.empty((8, d), dtype=torch.bfloat16, device="cuda")
        self.cfg = hf.make_config(sh)
        self.c = Calls(hf, self.cfg, [x["structs"][0] for x in self.layers])
        self.state_bytes = hf.hyf_state_bytes(self.cfg)
        self.pool = torch.zeros(2 * self.state_bytes, dtype=torch.uint8, device="cuda")
        self.ws_bytes = hf.hyf_workspace_bytes(self.cfg, 1, self.T)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device="cuda")
        self.cu_pre = Calls.i64([0, self.T])
        self.cu = [Calls.i64([0, a]) for a in self.acc]
        offs = np.concatenate([[0], np.cumsum(self.acc)])
        es = 2
        self.c_ptr = [ctypes.c_void_p(self.commits.data_ptr() + int(offs[i]) * d * es) for i in range(self.rounds)]
        self.b = [self.blocks[8 * i: 8 * i + 8] for i in range(self.rounds)]
        self.slots = [(ctypes.c_int32 * 1)(e) for e in range(2)]
        self.pool_p, self.ws_p = ctypes.c_void_p(self.pool.data_ptr()), ctypes.c_void_p(self.ws.data_ptr())
        self.pre_p = ctypes.c_void_p(self.prefix.data_ptr())
        self.p = [ctypes.c_void_p(t.data_ptr()) for t in (self.o1, self.x2, self.o2)]

    def step(self, stream, ev=None):
        L, c = self.c.L, self.c
        s = ctypes.c_void_p(stream)
        if ev:
            ev[0].record()
        st = L.hyf_state_reset(c.cfg_ref, self.pool_p, 2, None, 2, s)
        for li in range(2):
            st |= L.hyf_memory_commit(c.cfg_ref, c.w_ref[li], self.pool_p, 2, self.slots[li], 1, self.pre_p,
                                      self.cu_pre, None, self.ws_p, self.ws_bytes, s)
        if ev:
            ev[1].record()
        for i in range(self.rounds):
            bp = ctypes.c_void_p(self.b[i].data_ptr())
            st |= L.hyf_draft_block(c.cfg_ref, c.w_ref[0], self.pool_p, 2, self.slots[0], 1, self.c_ptr[i], self.cu[i],
                                    bp, self.p[0], self.ws_p, self.ws_bytes, s)
            self.x2.copy_(self.b[i])
            self.x2.add_(self.o1)
            st |= L.hyf_draft_block(c.cfg_ref, c.w_ref[1], self.pool_p, 2, self.slots[1], 1, self.c_ptr[i], self.cu[i],
                                    self.p[1], self.p[2], self.ws_p, self.ws_bytes, s)
        if ev:
            ev[2].record()
        if st:
            raise RuntimeError(f"libhyflash call failed (status bits {st})")


class LongPhi4:
    """The long-context Phi-4-shaped layer: chunk 256, a 131072-feature prefix commit, 128 rounds."""

    def __init__(self, torch, hf, I, memory="mamba2", name="phi4_long131k", prefix_dev=None):
        import numpy as np

        wl = I.WORKLOADS[name]
        self.shape = sh = wl["shape"].replace(memory=memory)
        self.T, self.rounds = wl["prefix"], wl["rounds"]
        d = sh.d_model
        rng = I.rng_streams(wl["seed"])
        self.host_w, self.wd = layer_weights(torch, hf, I, sh, rng[0])
        self.prefix = prefix_dev if prefix_dev is not None else device_rows(torch, rng[1], self.T, d, wl["feat_scale"])
        self.acc = rng[4].integers(1, 9, size=self.rounds)
        self.commits = device_rows(torch, rng[2], int(self.acc.sum()), d, wl["feat_scale"])
        self.blocks = device_rows(torch, rng[3], self.rounds * 8, d, wl["block_scale"])
        self.out = torch.empty((8, d), dtype=torch.bfloat16, device="cuda")
        self.cfg = hf.make_config(sh)
        self.c = Calls(hf, self.cfg, self.wd["structs"])
        self.state_bytes = hf.hyf_state_bytes(self.cfg)
        self.pool = torch.zeros(self.state_bytes, dtype=torch.uint8, device="cuda")
        self.ws_bytes = hf.hyf_workspace_bytes(self.cfg, 1, self.T)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device="cuda")
        self.cu_pre = Calls.i64([0, self.T])
        self.cu = [Calls.i64([0, a]) for a in self.acc]
        offs = np.concatenate([[0], np.cumsum(self.acc)])
        es = 2
        self.c_ptr = [ctypes.c_void_p(self.commits.data_ptr() + int(offs[i]) * d * es) for i in range(self.rounds)]
        self.b_ptr = [ctypes.c_void_p(self.blocks.data_ptr() + i * 8 * d * es) for i in range(self.rounds)]
        self.pool_p, self.ws_p = ctypes.c_void_p(self.pool.data_ptr()), ctypes.c_void_p(self.ws.data_ptr())
        self.pre_p, self.out_p = ctypes.c_void_p(self.prefix.data_ptr()), ctypes.c_void_p(self.out.data_ptr())

    def step(self, stream, ev=None):
        L, c = self.c.L, self.c
        s = ctypes.c_void_p(stream)
        if ev:
            ev[0].record()
        st = L.hyf_state_reset(c.cfg_ref, self.pool_p, 1, None, 1, s)
        st |= L.hyf_memory_commit(c.cfg_ref, c.w_ref[0], self.pool_p, 1, None, 1, self.pre_p, self.cu_pre, None,
                                  self.ws_p, self.ws_bytes, s)
        if ev:
            ev[1].record()
        for i in range(self.rounds):
            st |= c.L.hyf_draft_block(c.cfg_ref, c.w_ref[0], self.pool_p, 1, None, 1, self.c_ptr[i], self.cu[i],
                                      self.b_ptr[i], self.out_p, self.ws_p, self.ws_bytes, s)
        if ev:
            ev[2].record()
        if st:
            raise RuntimeError(f"libhyflash call failed (status bits {st})")


# ---- kernel loops --------------------------------------------------------------------------------


def scan_loop(torch, hf, I, shape, T, copies, reps, seed):
    """hyf_ssd_scan (state only) on pre-projected, time-blocked inputs x, B, dt_raw ~ N(0, 1),
    `copies` copies rotated; returns mean microseconds per call and the algorithmic bytes."""
    nh, P, N = shape.n_heads, shape.head_dim, shape.d_state
    cfg = hf.make_config(shape)
    nb = (T + 127) // 128
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    cp = [dict(x=torch.randn(nb * nh * P * 128, generator=gen, device="cuda").to(torch.bfloat16),
               B=torch.randn(nb * shape.gn * 128, generator=gen, device="cuda").to(torch.bfloat16),
               dt=torch.randn(nb * nh * 128, generator=gen, device="cuda"),
               H=torch.zeros((nh, P, N), device="cuda")) for _ in range(copies)]
    a_log = torch.rand(nh, generator=gen, device="cuda") * math.log(16.0)
    dt_bias = torch.full((nh,), -2.0, device="cuda")
    d_skip = torch.ones(nh, device="cuda")
    wsb = hf.hyf_ssd_scan_workspace_bytes(cfg, T)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    st = [0]

    def scan(i):
        c = cp[i % copies]
        st[0] |= hf.hyf_ssd_scan(cfg, c["x"], c["B"], None, c["dt"], a_log, dt_bias, d_skip, c["H"], None, T, ws, wsb)

    scan(0)
    us = time_graph(torch, scan, copies * max(1, reps // copies))
    if st[0]:
        raise RuntimeError("scan loop failed")
    del cp, ws
    torch.cuda.empty_cache()
    return us, scan_bytes(shape, T)


def scan_y_loop(torch, hf, I, shape, T, reps):
    """hyf_ssd_scan with per-token outputs (C in, y out)."""
    nh, P, N = shape.n_heads, shape.head_dim, shape.d_state
    cfg = hf.make_config(shape)
    sc = I.make_scan_inputs(shape, T, I.rng_streams(101)[0], with_c=True, h0_scale=0.0)
    eb = hf.elem_bytes(shape)
    x = hf.to_device(hf.time_tiled(sc["x"], T, eb), shape)
    B = hf.to_device(hf.time_tiled(sc["B"], T, eb), shape)
    C = hf.to_device(hf.time_tiled(sc["C"], T, eb), shape)
    dt = torch.from_numpy(hf.time_blocked(sc["dt_raw"], T)).cuda()
    v = [torch.from_numpy(sc[k]).cuda() for k in ("a_log", "dt_bias", "d_skip")]
    H = torch.zeros((nh, P, N), device="cuda")
    y = torch.empty((T, nh, P), dtype=torch.bfloat16, device="cuda")
    wsb = hf.hyf_ssd_scan_workspace_bytes(cfg, T, 1)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    st = [0]

    def scan(i):
        st[0] |= hf.hyf_ssd_scan(cfg, x, B, C, dt, *v, H, y, T, ws, wsb)

    scan(0)
    us = time_calls(torch, scan, reps)
    if st[0]:
        raise RuntimeError("y-mode scan loop failed")
    return us, scan_bytes(shape, T) + T * (shape.gn * 2 + nh * P * 2)


def gemm_loop(torch, hf, shape, M, reps, copies=2):
    """The prefill projection GEMM of v | B | dt over M rows (hyf_linear, tiled time-blocked output
    is not needed here: plain bf16 output), `copies` weight copies rotated."""
    d = shape.d_model
    nout = shape.dq + shape.gn + shape.n_heads
    cfg = hf.make_config(shape)
    X = torch.empty((M, d), dtype=torch.bfloat16, device="cuda").normal_()
    W = [torch.empty((nout, d), dtype=torch.bfloat16, device="cuda").normal_() for _ in range(copies)]
    out = torch.empty((M, nout), dtype=torch.bfloat16, device="cuda")
    st = [0]

    def gemm(i):
        st[0] |= hf.hyf_linear(cfg, X, M, d, W[i % copies], nout, out, 0)

    gemm(0)
    us = time_calls(torch, gemm, reps)
    if st[0]:
        raise RuntimeError("gemm loop failed")
    flops = 2.0 * M * d * nout
    tf = flops / (us * 1e-6) / 1e12
    res = {"M": M, "K": d, "N": nout, "avg_us": us, "tflops": tf,
           "roofline": {"bound": "mfma", "achieved": tf, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": tf / BF16_PEAK_TFLOPS}}
    res["vendor_blas"] = vendor_gemm(torch, X, W, M, d, nout, reps)
    return res


def vendor_gemm(torch, X, W, M, K, N, reps):
    """The same product through torch.matmul (ROCm's vendor BLAS), for context only."""
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    Wt = [w.t() for w in W]
    torch.matmul(X, Wt[0], out=out)
    us = time_calls(torch, lambda i: torch.matmul(X, Wt[i % len(Wt)], out=out), reps)
    tf = 2.0 * M * K * N / (us * 1e-6) / 1e12
    return {"what": "torch.matmul on the same operands (vendor BLAS), context only", "avg_us": us,
            "tflops": tf, "frac": tf / BF16_PEAK_TFLOPS}


def round_gemm_loop(torch, hf, shape, M, K, N, reps):
    """A batched round's projection through the tiled GEMM (bf16 in, fp32 out as the round takes it),
    W_COPIES weight copies rotated, and the vendor BLAS on the same shape for context."""
    cfg = hf.make_config(shape)
    X = torch.empty((M, K), dtype=torch.bfloat16, device="cuda").normal_()
    W = [torch.empty((N, K), dtype=torch.bfloat16, device="cuda").normal_() for _ in range(W_COPIES)]
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    st = [0]

    def proj(i):
        st[0] |= hf.hyf_linear(cfg, X, M, K, W[i % W_COPIES], N, y, 1)

    proj(0)
    us = time_calls(torch, proj, reps)
    if st[0]:
        raise RuntimeError("round GEMM loop failed")
    tf = 2.0 * M * K * N / (us * 1e-6) / 1e12
    return {"M": M, "K": K, "N": N, "avg_us": us, "tflops": tf,
            "roofline": {"bound": "mfma", "achieved": tf, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": tf / BF16_PEAK_TFLOPS},
            "vendor_blas": vendor_gemm(torch, X, W, M, K, N, reps)}


def proj_loop(torch, hf, shape, M, K, N, reps):
    """A round projection (M rows, hyf_linear, fp32 output) with W_COPIES weight copies rotated."""
    cfg = hf.make_config(shape)
    X = torch.empty((M, K), dtype=torch.bfloat16, device="cuda").normal_()
    W = [torch.empty((N, K), dtype=torch.bfloat16, device="cuda").normal_() for _ in range(W_COPIES)]
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    st = [0]

    def proj(i):
        st[0] |= hf.hyf_linear(cfg, X, M, K, W[i % W_COPIES], N, y, 1)

    proj(0)
    us = time_graph(torch, proj, W_COPIES * max(1, reps // W_COPIES))
    if st[0]:
        raise RuntimeError("projection loop failed")
    b = N * K * 2 + M * K * 2 + M * N * 4
    return {"rows": M, "K": K, "N": N, "avg_us": us, "bytes_per_launch": b, **hbm(b, us)}


def w4_projections(torch, hf, shape, reps=96):
    """The round's two projections (12 rows x w_in, 8 rows x w_out) with 4-bit weights
    (hyf_linear_w4) beside the bf16 ones, each graph-timed over rotated weight copies."""
    cfg = hf.make_config(shape)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4)
    st = [0]
    res = {}
    for name, M, K, N in (("w_in", 12, shape.d_model, shape.n_in), ("w_out", 8, shape.dq, shape.d_model)):
        X = torch.randn((M, K), device="cuda", generator=gen).to(torch.bfloat16)
        y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        w4b = N * K // 2 + N * (K // 128) * 4
        n4 = max(2, math.ceil(320e6 / w4b))
        codes = [torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device="cuda", generator=gen) for _ in range(n4)]
        scales = [torch.rand((N, K // 128), device="cuda", generator=gen) / (7.0 * math.sqrt(K)) for _ in range(n4)]

        def w4(i):
            st[0] |= hf.hyf_linear_w4(cfg, X, M, K, codes[i % n4], scales[i % n4], N, y, 1)

        us4 = time_graph(torch, w4, n4 * max(1, reps // n4))
        del codes, scales
        byt = w4b + M * K * 2 + M * N * 4
        res[name] = {"rows": M, "K": K, "N": N, "w4_us": us4, "bytes_per_launch": byt, **hbm(byt, us4)}
    if st[0]:
        raise RuntimeError(f"projection call failed: status {st[0]}")
    torch.cuda.empty_cache()
    return res


# ---- HBM traffic from hardware counters -------------------------------------------------------
# rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of a --pmc-probe run are scaled by
# what the same counters read for a plain device copy of COPY_BYTES (read COPY_BYTES, write
# COPY_BYTES).  The figures stay valid only for the kernel sources they were taken from.
COPY_BYTES = 256 << 20
PMC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.json")
PMC_KERNELS = {  # key -> (kernel name substring, source file, launch shape the probe runs)
    "round": ("k_round", "hybrid_ssm_local_amd/csrc/hyf_round.hip", "64 Qwen3-4B-shaped requests, full windows"),
    "scan_seg": ("k_ssd_seg", "hybrid_ssm_local_amd/csrc/hyf_scan.hip", "8192 tokens, Qwen3-4B shape"),
    "scan_combine": ("k_ssd_combine", "hybrid_ssm_local_amd/csrc/hyf_scan.hip", "8192 tokens, Qwen3-4B shape"),
    "gemm": ("k_gemm_bf16_tile", "hybrid_ssm_local_amd/csrc/hyf_gemm.hip", "8192 x 2560 x 2720"),
    "proj": ("k_proj_stream<8, 1>", "hybrid_ssm_local_amd/csrc/hyf_proj.hip", "12 rows x w_in (2560 x 7968)"),
    "w4": ("k_linear_w4", "hybrid_ssm_local_amd/csrc/hyf_w4.hip", "12 rows x 4-bit w_in"),
}


def source_digest(rel):
    import hashlib

    with open(os.path.join(ROOT, rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


PMC_REPS = 4  # launches of each measured shape at the end of its section of the PMC probe


def pmc_probe(torch, hf, I, reps=PMC_REPS):
    """The measured kernels in a fixed order, each at one launch shape: a copy of known size; the
    round kernel at the batched shape (64 requests, windows filled by earlier rounds); the 8192-token
    scan; the 8192 x 2560 x 2720 GEMM; the 12-row w_in projection (bf16, then 4-bit)."""
    import numpy as np

    src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda").normal_()
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    sh = I.QWEN
    R, d = 64, sh.d_model
    rng = I.rng_streams(3)
    _, wd = layer_weights(torch, hf, I, sh, rng[0])
    cfg = hf.make_config(sh)
    pool = torch.zeros(R * hf.hyf_state_bytes(cfg), dtype=torch.uint8, device="cuda")
    wsb = hf.hyf_workspace_bytes(cfg, R, 8 * R)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    rows = (torch.randn((8 * R, d), device="cuda") / math.sqrt(d)).to(torch.bfloat16)
    out = torch.empty_like(rows)
    cu = np.arange(0, 8 * R + 1, 8, dtype=np.int64)
    st = hf.hyf_state_reset(cfg, pool, R, None, R)
    for _ in range(sh.window // 8 + reps):  # 64 rounds fill the windows, then `reps` more
        st |= hf.hyf_draft_block(cfg, wd["structs"][0], pool, R, None, R, rows, cu, rows, out, ws, wsb)
    torch.cuda.synchronize()
    del pool, ws
    scan_loop(torch, hf, I, sh, 8192, 2, reps, 100)
    gemm_loop(torch, hf, sh, 8192, reps)
    proj_loop(torch, hf, sh, 12, d, sh.n_in, W_COPIES)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4)
    M, K, N = 12, d, sh.n_in
    X = torch.randn((M, K), device="cuda", generator=gen).to(torch.bfloat16)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    for _ in range(reps):
        codes = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device="cuda", generator=gen)
        scales = torch.rand((N, K // 128), device="cuda", generator=gen) / (7.0 * math.sqrt(K))
        st |= hf.hyf_linear_w4(cfg, X, M, K, codes, scales, N, y, 1)
    torch.cuda.synchronize()
    if st:
        raise RuntimeError(f"pmc probe call failed: status {st}")


def pmc_summary(fetch_db, write_db):
    import sqlite3

    def dispatches(db, counter):
        con = sqlite3.connect(db)
        rows = con.execute("select dispatch_id, kernel_name, grid_size, sum(value) from counters_collection "
                           "where counter_name = ? group by dispatch_id order by dispatch_id", (counter,)).fetchall()
        return [(k, g, v) for _, k, g, v in rows]

    fd, wd = dispatches(fetch_db, "FETCH_SIZE"), dispatches(write_db, "WRITE_SIZE")
    copy_f = max(v for k, g, v in fd if "copyBuffer" in k)
    copy_w = max(v for k, g, v in wd if "copyBuffer" in k)
    scale_f, scale_w = COPY_BYTES / (copy_f * 1024), COPY_BYTES / (copy_w * 1024)
    out = {"copy_bytes": COPY_BYTES, "copy_fetch_kib": copy_f, "copy_write_kib": copy_w,
           "fetch_scale": scale_f, "write_scale": scale_w, "kernels": {}}

    def pick(rows, sub):
        # the kernel's last PMC_REPS dispatches: each section of the probe ends with PMC_REPS launches
        # of its measured shape (the round kernel after the windows have filled, the GEMM after the
        # rounds' own projection GEMMs)
        m = [(k, g, v) for k, g, v in rows if sub in k][-PMC_REPS:]
        if not m:
            return None, None, None
        return m[-1][0], m[-1][1], sum(v for _, _, v in m) / len(m)

    for key, (sub, src, what) in PMC_KERNELS.items():
        name, g, f_kib = pick(fd, sub)
        if g is None:
            continue
        _, _, w_kib = pick(wd, sub)
        out["kernels"][key] = {"kernel": name, "grid": g, "shape": what, "source": src,
                               "source_sha256": source_digest(src), "fetch_kib": f_kib, "write_kib": w_kib or 0.0,
                               "traffic_bytes": f_kib * 1024 * scale_f + (w_kib or 0.0) * 1024 * scale_w}
    with open(PMC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    lines = ["# HBM traffic of the measured kernels (rocprofv3 counters)", "",
             "Commands (repository root, one MI355X; each counter in a run of its own):", "", "```",
             "rocprofv3 --pmc FETCH_SIZE -d out/pmc/f -o f -- python3 bench.py --pmc-probe",
             "rocprofv3 --pmc WRITE_SIZE -d out/pmc/w -o w -- python3 bench.py --pmc-probe",
             "python3 bench.py --pmc-summary out/pmc/f/f_results.db out/pmc/w/w_results.db", "```", "",
             f"Calibration: a device copy of {COPY_BYTES >> 20} MiB reads FETCH_SIZE {copy_f:.0f} KiB and "
             f"WRITE_SIZE {copy_w:.0f} KiB, so measured KiB are scaled by {scale_f:.3f} (fetch) and "
             f"{scale_w:.3f} (write).", "",
             "| key | kernel | launch shape | grid (threads) | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes per launch |",
             "|---|---|---|---:|---:|---:|---:|"]
    for key, k in out["kernels"].items():
        lines.append(f"| {key} | `{k['kernel'][:60]}` | {k['shape']} | {k['grid']} | {k['fetch_kib']:.0f} | "
                     f"{k['write_kib']:.0f} | {k['traffic_bytes']:.0f} |")
    with open(PMC_FILE.replace(".json", ".md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps(out, indent=1))


def pmc_traffic(key):
    """Measured HBM bytes per launch of a kernel, or None if absent or taken from other sources."""
    try:
        with open(PMC_FILE) as f:
            k = json.load(f)["kernels"][key]
    except (OSError, KeyError, ValueError):
        return None
    return k["traffic_bytes"] if k["source_sha256"] == source_digest(k["source"]) else None


def scan_traffic():
    """HBM bytes of one state-only scan call: the segment kernel plus the fold."""
    seg, comb = pmc_traffic("scan_seg"), pmc_traffic("scan_combine")
    return None if seg is None or comb is None else seg + comb


def stats_summary(d):
    """Kernel statistics of a profiled --profile run: per kernel, and per (kernel, launch shape) in
    the order the shapes first ran, so each workload's launches can be read off separately."""
    import csv

    stats = list(csv.DictReader(open(os.path.join(d, "bench_kernel_stats.csv"))))
    trace = list(csv.DictReader(open(os.path.join(d, "bench_kernel_trace.csv"))))
    trace.sort(key=lambda r: int(r["Start_Timestamp"]))
    dur = lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    short = lambda n: n if len(n) <= 100 else n[:97] + "..."
    lines = ["# bench.py --profile: kernel statistics", "",
             "Command (from the repository root, on one MI355X):", "", "```",
             "rocprofv3 --kernel-trace --stats --output-format csv -d out/prof_bench -o bench -- "
             "python3 bench.py --profile",
             "python3 bench.py --stats-summary out/prof_bench", "```", "",
             "The run holds, in order: the batched 64-request serving steps (headline) and their round-kernel "
             "graphs, the batch-1 Qwen3-4B-shaped episodes, the Phi-4-shaped two-layer steps, the long-context "
             "Phi-4-shaped steps (Mamba-2, then the gated delta rule), then bench.py's kernel loops.", "",
             "rocprofv3 kernel statistics (durations in microseconds):", "",
             "| kernel | calls | total us | average us | % |", "|---|---:|---:|---:|---:|"]
    for r in stats:
        lines.append(f"| `{short(r['Name'])}` | {r['Calls']} | {float(r['TotalDurationNs']) / 1e3:.1f} | "
                     f"{float(r['AverageNs']) / 1e3:.3f} | {float(r['Percentage']):.2f} |")
    shapes, order = {}, []
    for r in trace:
        key = (r["Kernel_Name"], int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]),
               int(r["Workgroup_Size_X"]))
        if key not in shapes:
            shapes[key] = []
            order.append(key)
        shapes[key].append(dur(r))
    lines += ["", "By launch shape, in order of first launch (grid = threads in all dimensions; microseconds).  "
              "Launches of one shape whose durations differ by more than 3x (the same grid over different "
              "work, e.g. the 8192- and 131072-token scans) are listed as separate duration classes:", "",
              "| kernel | grid | workgroup | calls | average us | min us |", "|---|---:|---:|---:|---:|---:|"]
    for key in order:
        k, g, w = key
        if "hyf" not in k:
            continue
        v = sorted(shapes[key])
        classes, cur = [], [v[0]]
        for x in v[1:]:
            if x > 3.0 * cur[-1] and x > cur[-1] + 5.0:
                classes.append(cur)
                cur = []
            cur.append(x)
        classes.append(cur)
        for c in classes:
            lines.append(f"| `{short(k)}` | {g} | {w} | {len(c)} | {sum(c) / len(c):.3f} | {min(c):.3f} |")
    out = os.path.join(ROOT, "profiles", "bench_kernel_stats.md")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out)


# ---- CPU baseline --------------------------------------------------------------------------------


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(I, host_w, wl_name=HEADLINE, min_seconds=12.0):
    """The float64 oracle on the host cores, on a bounded sample of the headline workload: whole
    request episodes (the request's prefix commit, then all of its rounds, each committing 1-8
    accepted features and drafting a block), request after request with prefix lengths drawn like
    the workload's, until at least min_seconds of work.  The rate is draft blocks/s over those
    episodes; requests are independent, so 64 of them take 64 times as long.  cores = process CPU
    time / wall time of the timed work (the per-token loops are single-threaded Python; only the
    projections use BLAS threads)."""
    import numpy as np

    from oracle import hyflash_oracle as O

    try:
        from threadpoolctl import threadpool_info

        allowed = max([x["num_threads"] for x in threadpool_info()] + [1])
    except Exception:
        allowed = 1
    wl = I.WORKLOADS[wl_name]
    sh = wl["shape"]
    rng = I.rng_streams(wl["seed"] + 1000)
    lo, hi = wl["prefix_range"]
    w = {k: np.asarray(v, np.float64) for k, v in host_w.items()}
    t_commit = t_rounds = cpu = 0.0
    feats = blocks = 0
    lens = []
    while t_commit + t_rounds < min_seconds:
        n_pre = int(rng[4].integers(lo, hi + 1))
        lens.append(n_pre)
        pre = I.make_rows(rng[1], n_pre, sh.d_model, wl["feat_scale"], sh.dtype)
        acc = I.acceptance_lengths(rng[4], wl["rounds"])
        commits = [I.make_rows(rng[2], int(a), sh.d_model, wl["feat_scale"], sh.dtype) for a in acc]
        blks = [I.make_rows(rng[3], 8, sh.d_model, wl["block_scale"], sh.dtype) for _ in acc]
        c0, t0 = time.process_time(), time.perf_counter()
        st, _ = O.commit(sh, w, O.new_state(sh), pre)
        t1 = time.perf_counter()
        for cf, blk in zip(commits, blks):
            st, _ = O.round_step(sh, w, st, cf, blk)
        t2 = time.perf_counter()
        cpu += time.process_time() - c0
        t_commit += t1 - t0
        t_rounds += t2 - t1
        feats += n_pre
        blocks += len(acc)
    wall = t_commit + t_rounds
    return {"value": blocks / wall, "unit": "draft blocks/s (headline workload)",
            "cores": max(1, round(cpu / wall)), "kind": "oracle",
            "sample": f"float64 NumPy oracle: {len(lens)} whole request episodes of the batched workload (prefixes "
                      f"{lens} features, then {wl['rounds']} rounds each); requests are independent, so the rate is "
                      f"the workload's",
            "cpu_model": cpu_model(), "threads_allowed": allowed, "seconds": wall,
            "commit_feats_per_s": feats / t_commit, "round_ms": 1e3 * t_rounds / blocks}


# ---- main ----------------------------------------------------------------------------------------


def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary)
        return
    if args.stats_summary:
        stats_summary(args.stats_summary)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)
    sub_steps = 3
    if args.profile:
        args.steps, args.warmup, args.kernel_reps, args.no_cpu = 2, 1, 8, True
        sub_steps = 1

    import torch

    from hybrid_ssm_local_amd import hyflash as hf
    from hybrid_ssm_local_amd import inputs as I

    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    if args.pmc_probe:
        pmc_probe(torch, hf, I)
        return

    # ---- headline: batched serving, 64 requests, whole steps
    log("headline: building the batched workload")
    bt = Batched(torch, hf, I)
    log("headline: eager steps", args.warmup, "+", args.steps)
    head = run_steps(torch, bt.step, args.steps, args.warmup)
    log("headline: round-kernel graphs")
    t_round, t_proj, rows = bt.round_kernel(torch, hf)
    sh, R = bt.shape, bt.R
    kb = kround_bytes(sh, R, rows, bt.windows)
    rb = round_bytes(sh, R, rows, bt.windows)
    t_k = t_round - t_proj
    blocks = R * bt.rounds
    head_obj = {"host_w": bt.host_w, "T": bt.T}
    del bt
    torch.cuda.empty_cache()

    # ---- batch-1 Qwen3-4B-shaped episodes
    log("batch-1 episodes")
    ep = EpisodesB1(torch, hf, I)
    b1 = run_steps(torch, ep.step, sub_steps, 1)
    b1_round, b1_proj, b1_rows = ep.round_kernel(torch, hf)
    b1_win = [ep.shape.window]
    b1_kb = kround_bytes(ep.shape, 1, b1_rows, b1_win)
    b1_rb = round_bytes(ep.shape, 1, b1_rows, b1_win)
    b1_blocks = EPISODES * ep.rounds
    qwen_b1 = {
        "workload": "Qwen3-4B-shaped layer, batch 1: 8192-feature prefix commit, then 256 rounds (1-8 accepted "
                    f"features each); {EPISODES} requests' episodes interleaved call by call, {W_COPIES} weight copies "
                    "rotated",
        "value": b1_blocks / (b1["step_ms"] * 1e-3), "unit": "draft blocks/s per layer (batch 1)",
        "ms_per_step": b1["step_ms"], "prefill_commit_us": 1e3 * b1["prefill_ms"] / EPISODES,
        "round_us": 1e3 * b1["rounds_ms"] / b1_blocks,
        "round_graph_us": b1_round, "round": {"bytes_per_round": b1_rb, **hbm(b1_rb, b1_round)},
        "round_kernel": {"kernel": "k_round (1 request x 32 heads)", "avg_us": b1_round - b1_proj,
                         "bytes_per_launch": b1_kb, **hbm(b1_kb, b1_round - b1_proj),
                         "projections_graph_us": b1_proj},
    }
    del ep
    torch.cuda.empty_cache()
    log("batch-1 episodes, 4-bit weights")
    ep4 = EpisodesB1(torch, hf, I, weights="w4")
    b4 = run_steps(torch, ep4.step, sub_steps, 1)
    b4_round, b4_proj, b4_rows = ep4.round_kernel(torch, hf)
    w4b = (ep4.shape.n_in * ep4.shape.d_model + ep4.shape.d_model * ep4.shape.dq) // 2 + \
        (ep4.shape.n_in * ep4.shape.d_model + ep4.shape.d_model * ep4.shape.dq) // 128 * 4
    b4_rb = b1_rb - (ep4.shape.n_in + ep4.shape.dq) * ep4.shape.d_model * 2 + w4b
    qwen_b1_w4 = {
        "workload": "as qwen3_4b_batch1, with the projections' weights as 4-bit codes (random) and fp32 scales",
        "value": b1_blocks / (b4["step_ms"] * 1e-3), "unit": "draft blocks/s per layer (batch 1)",
        "ms_per_step": b4["step_ms"], "prefill_commit_us": 1e3 * b4["prefill_ms"] / EPISODES,
        "round_us": 1e3 * b4["rounds_ms"] / b1_blocks, "round_graph_us": b4_round,
        "round": {"bytes_per_round": b4_rb, **hbm(b4_rb, b4_round)}, "projections_graph_us": b4_proj,
        "speedup_vs_bf16_round": b1_round / b4_round,
    }
    del ep4
    torch.cuda.empty_cache()
    log("batch-1 episodes, last-W memory")
    epw = EpisodesB1(torch, hf, I, memory="lastw")
    bw = run_steps(torch, epw.step, sub_steps, 1)
    qwen_b1_lastw = {
        "workload": "as qwen3_4b_batch1, with the memory restricted to the last W = 512 committed rows (each commit "
                    "rescans the window into H; a round commits, then drafts)",
        "value": b1_blocks / (bw["step_ms"] * 1e-3), "unit": "draft blocks/s per layer (batch 1)",
        "ms_per_step": bw["step_ms"], "prefill_commit_us": 1e3 * bw["prefill_ms"] / EPISODES,
        "round_us": 1e3 * bw["rounds_ms"] / b1_blocks,
    }
    del epw
    torch.cuda.empty_cache()
    log("batch-1 episodes, full drafter block")
    epb = EpisodesBlockB1(torch, hf, I)
    bb = run_steps(torch, epb.step, sub_steps, 1)
    bb_round = epb.round_graph(torch)
    sh_b = epb.shape
    mlp_b = 3 * epb.F * sh_b.d_model * 2
    bb_rb = b1_rb + mlp_b  # the layer's round bytes plus the MLP's weights (the norms' rows are a few KB)
    qwen_b1_block = {
        "workload": "the full drafter block around the Qwen3-4B-shaped layer (pre-norm, layer, residual, pre-norm, "
                    f"SwiGLU MLP of width {epb.F}, residual), batch 1, episodes as qwen3_4b_batch1",
        "value": b1_blocks / (bb["step_ms"] * 1e-3), "unit": "draft blocks/s per block (batch 1)",
        "ms_per_step": bb["step_ms"], "prefill_commit_us": 1e3 * bb["prefill_ms"] / EPISODES,
        "round_us": 1e3 * bb["rounds_ms"] / b1_blocks, "round_graph_us": bb_round,
        "round": {"bytes_per_round": bb_rb, **hbm(bb_rb, bb_round)},
    }
    del epb
    torch.cuda.empty_cache()

    # ---- Phi-4-shaped two-layer drafter
    log("phi-4 two-layer")
    tl = TwoLayerPhi4(torch, hf, I)
    p3 = run_steps(torch, tl.step, sub_steps, 1)
    phi4_2l = {"workload": "Phi-4-shaped two-layer drafter: both layers commit a 32768-feature prefix, then 512 rounds "
                           "(each: both layers commit 1-8 accepted features; layer 2 drafts from block_in + layer 1's "
                           "output)",
               "value": tl.rounds / (p3["step_ms"] * 1e-3), "unit": "two-layer draft rounds/s (batch 1)",
               "ms_per_step": p3["step_ms"], "prefill_commit_us": 1e3 * p3["prefill_ms"] / 2,
               "round_us": 1e3 * p3["rounds_ms"] / tl.rounds,
               "per_layer_blocks_per_s": 2 * tl.rounds / (p3["rounds_ms"] * 1e-3)}
    del tl
    torch.cuda.empty_cache()

    # ---- long-context Phi-4-shaped layer, both memories
    long5 = {}
    prefix = None
    for memory in ("mamba2", "gdn"):
        log("phi-4 long context", memory)
        lp = LongPhi4(torch, hf, I, memory=memory, prefix_dev=prefix)
        prefix = lp.prefix
        p5 = run_steps(torch, lp.step, sub_steps, 1)
        long5[memory] = {"value": lp.rounds / (p5["step_ms"] * 1e-3), "unit": "draft blocks/s per layer (batch 1)",
                         "ms_per_step": p5["step_ms"], "prefill_commit_us": 1e3 * p5["prefill_ms"],
                         "commit_feats_per_s": lp.T / (p5["prefill_ms"] * 1e-3),
                         "round_us": 1e3 * p5["rounds_ms"] / lp.rounds}
        del lp
        torch.cuda.empty_cache()
    long5["workload"] = ("Phi-4-shaped layer, chunk 256: 131072-feature prefix commit, then 128 rounds; Mamba-2 and "
                         "the gated delta rule")
    del prefix
    torch.cuda.empty_cache()

    # ---- kernel loops
    log("kernel loops")
    reps = args.kernel_reps
    s_us, s_b = scan_loop(torch, hf, I, I.QWEN, 8192, SCAN_COPIES, reps, 100)
    sl_us, sl_b = scan_loop(torch, hf, I, I.PHI4_LONG, 131072, 2, max(4, reps // 6), 131072)
    sq_us, sq_b = scan_loop(torch, hf, I, I.QWEN, 131072, 2, max(4, reps // 6), 131073)
    sy_us, sy_b = scan_y_loop(torch, hf, I, I.QWEN, 8192, max(4, reps // 6))
    g2 = gemm_loop(torch, hf, I.QWEN, 8192, max(4, reps // 6))
    g3 = gemm_loop(torch, hf, I.PHI4, 32768, max(4, reps // 12))
    gr_in = round_gemm_loop(torch, hf, I.QWEN, 800, I.QWEN.d_model, I.QWEN.n_in, reps)
    gr_out = round_gemm_loop(torch, hf, I.QWEN, 512, I.QWEN.dq, I.QWEN.d_model, reps)
    pj = proj_loop(torch, hf, I.QWEN, 12, I.QWEN.d_model, I.QWEN.n_in, reps)
    w4 = w4_projections(torch, hf, I.QWEN)
    g2["traffic"] = pmc_traffic("gemm")
    pj["traffic"] = pmc_traffic("proj")
    cpu = None if args.no_cpu else cpu_baseline(I, head_obj["host_w"])

    res = {
        "metric": METRIC,
        "value": blocks / (head["step_ms"] * 1e-3),
        "unit": "draft blocks/s (64 requests, one layer)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["step_ms"],
        "wall_s": head["wall_s"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded NumPy PCG64: N(0,1)/sqrt(d) features and block rows, Xavier-normal weights)",
        "config": {"workload": "batched serving on one GPU: Qwen3-4B-shaped HyFlash drafter layer, 64 requests with "
                               "prefixes U{2048..16384} committed in one call, then 128 rounds of commit (1-8 "
                               "accepted per request) + draft block for all 64",
                   "d_model": sh.d_model, "n_heads": sh.n_heads, "head_dim": sh.head_dim, "d_state": sh.d_state,
                   "chunk": sh.chunk, "window": sh.window, "block": sh.block, "requests": R, "rounds": 128,
                   "prefix_rows": head_obj["T"], "parallelism": "single GPU"},
        "breakdown": {"prefill_commit_us": 1e3 * head["prefill_ms"], "rounds_us": 1e3 * head["rounds_ms"],
                      "round_us": 1e3 * head["rounds_ms"] / 128, "round_graph_us": t_round,
                      "projections_graph_us": t_proj},
        "roofline": {**hbm(kb, t_k), "traffic": pmc_traffic("round"),
                     "kernel": "k_round_pair<bf16>: commit, readout and attention of 64 requests x 32 heads, one "
                               "workgroup per (request, head)",
                     "bytes_per_launch": kb, "avg_us": t_k,
                     "method": "graph of the 128 rounds minus a graph of their two projections (same kernels and "
                               "shapes through hyf_linear), per round"},
        "round": {"bytes_per_round": rb, "avg_us": t_round, **hbm(rb, t_round)},
        "qwen3_4b_batch1": qwen_b1,
        "qwen3_4b_batch1_w4": qwen_b1_w4,
        "qwen3_4b_batch1_lastw": qwen_b1_lastw,
        "qwen3_4b_full_block_batch1": qwen_b1_block,
        "phi4_two_layer": phi4_2l,
        "phi4_long131k": long5,
        "commit_scan": {"value": 8192 / (s_us * 1e-6), "unit": "committed feats/s", "T": 8192, "shape": "Qwen3-4B",
                        "avg_us": s_us, "roofline": {**hbm(s_b, s_us), "traffic": scan_traffic(),
                                                     "bytes_per_launch": s_b}},
        "commit_scan_phi4_131k": {"value": 131072 / (sl_us * 1e-6), "unit": "committed feats/s", "T": 131072,
                                  "shape": "Phi-4, chunk 256", "avg_us": sl_us,
                                  "roofline": {**hbm(sl_b, sl_us), "traffic": None, "bytes_per_launch": sl_b}},
        "commit_scan_qwen_131k": {"value": 131072 / (sq_us * 1e-6), "unit": "committed feats/s", "T": 131072,
                                  "shape": "Qwen3-4B", "avg_us": sq_us,
                                  "roofline": {**hbm(sq_b, sq_us), "traffic": None, "bytes_per_launch": sq_b}},
        "commit_scan_y": {"value": 8192 / (sy_us * 1e-6), "unit": "committed feats/s", "T": 8192, "avg_us": sy_us,
                          "roofline": {**hbm(sy_b, sy_us), "traffic": None, "bytes_per_launch": sy_b}},
        "gemm_qwen_8192": g2,
        "gemm_phi4_32768": g3,
        "gemm_batched_round_w_in": gr_in,
        "gemm_batched_round_w_out": gr_out,
        "round_projection_w_in": pj,
        "w4a16_round_projections": w4,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
