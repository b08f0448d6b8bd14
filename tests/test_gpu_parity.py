"""Parity of the HIP path (through the C ABI) with the CPU oracle, and the layer's invariants.

Tolerance (max-norm relative, per output tensor): fp32 1e-4; bf16 2e-2 with max abs error 5e-2.
Each GPU step prints its case before it runs.
"""

import itertools

import numpy as np
import pytest
import torch

from hybrid_ssm_local_amd import hyflash as hf
from hybrid_ssm_local_amd import inputs as I
from oracle import hyflash_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print("[case]", *a, flush=True)


def assert_close(got, ref, dtype, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), what
    err = np.max(np.abs(got - ref)) if got.size else 0.0
    scale = max(np.max(np.abs(ref)) if ref.size else 0.0, 1e-30)
    rel = err / scale
    if dtype == "f32":
        assert rel <= 1e-4, f"{what}: rel {rel:.3e} (abs {err:.3e})"
    else:
        assert rel <= 2e-2 and err <= 5e-2, f"{what}: rel {rel:.3e} abs {err:.3e}"
    return rel


def small_shape(dtype, **kw):
    base = dict(d_model=256, n_heads=4, head_dim=64, d_state=64, window=128, chunk=64, dtype=dtype)
    base.update(kw)
    return I.LayerShape(**base)


# ---------------------------------------------------------------- scan level


def run_scan(shape, sc, T, with_y=False):
    # Tokens past T in the last time block hold NaN: none may reach the state or y.
    cfg = hf.make_config(shape)
    eb = hf.elem_bytes(shape)
    x = hf.to_device(hf.time_tiled(sc["x"], T, eb, np.nan), shape)
    B = hf.to_device(hf.time_tiled(sc["B"], T, eb, np.nan), shape)
    C = hf.to_device(hf.time_tiled(sc["C"], T, eb, np.nan), shape) if with_y else None
    dt = torch.from_numpy(hf.time_blocked(sc["dt_raw"], T, np.nan)).to(DEV)
    a_log = torch.from_numpy(sc["a_log"]).to(DEV)
    dt_bias = torch.from_numpy(sc["dt_bias"]).to(DEV)
    d_skip = torch.from_numpy(sc["d_skip"]).to(DEV)
    H = torch.from_numpy(sc["H0"]).to(DEV).contiguous()
    y = torch.full((T, shape.n_heads, shape.head_dim), float("nan"), dtype=hf.torch_dtype(shape), device=DEV) \
        if with_y else None
    wsb = hf.hyf_ssd_scan_workspace_bytes(cfg, T, with_y)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=DEV)
    hf.check(hf.hyf_ssd_scan(cfg, x, B, C, dt, a_log, dt_bias, d_skip, H, y, T, ws, wsb), "hyf_ssd_scan")
    torch.cuda.synchronize()
    if with_y:
        return H.cpu().numpy(), y.float().cpu().numpy()
    return H.cpu().numpy()


SCAN_CASES = [
    ("tiny_fp32", I.TINY, [1, 63, 64, 65, 300, 1024]),
    ("qwen_bf16", I.QWEN, [7, 64, 129, 1000]),
    ("phi4_bf16_L256", I.PHI4_LONG, [255, 700]),
    ("odd_bf16", small_shape("bf16", n_heads=3, head_dim=48, d_state=80, n_groups=3, chunk=32), [1, 100]),
    ("odd_fp32", small_shape("f32", n_heads=6, head_dim=32, d_state=48, n_groups=2, chunk=32), [37, 200]),
]


@pytest.mark.parametrize("name,shape,Ts", SCAN_CASES, ids=[c[0] for c in SCAN_CASES])
def test_scan_state_matches_the_sequential_recurrence(name, shape, Ts):
    for T in Ts:
        rng = I.rng_streams(T)[0]
        sc = I.make_scan_inputs(shape, T, rng, with_c=False, h0_scale=0.5)
        say("hyf_ssd_scan", name, "T", T)
        H = run_scan(shape, sc, T)
        ref, _ = O.ssd_sequential(sc["x"], sc["B"], None, sc["dt_raw"], sc["a_log"], sc["dt_bias"], sc["d_skip"],
                                  sc["H0"], shape.n_groups)
        assert_close(H, ref, shape.dtype, f"{name} T={T}")


Y_CASES = [
    ("tiny_fp32", I.TINY, [1, 127, 128, 129, 300]),
    ("qwen_bf16", I.QWEN, [7, 200]),
    ("phi4_bf16_L256", I.PHI4_LONG, [255, 300]),
    ("odd_bf16", small_shape("bf16", n_heads=3, head_dim=48, d_state=80, n_groups=3, chunk=32), [1, 100]),
    ("odd_fp32", small_shape("f32", n_heads=6, head_dim=32, d_state=48, n_groups=2, chunk=32), [37, 260]),
    # one 16-dimension tile per head with 256 state columns (16 feature groups, the largest LDS
    # staging of the bf16 kernel), lengths on and past 16-token tile edges and a whole block
    ("wide_state_bf16", small_shape("bf16", n_heads=2, head_dim=16, d_state=256, n_groups=1, chunk=32),
     [16, 17, 128, 129]),
    # seven dimension tiles (the state read per feature group, not one ahead)
    ("p112_bf16", small_shape("bf16", n_heads=2, head_dim=112, d_state=32, n_groups=2, chunk=32), [33]),
    # 128 dimensions with 256 state columns: only the matrix-core kernel's LDS (B and C) fits
    ("p128_n256_bf16", small_shape("bf16", n_heads=2, head_dim=128, d_state=256, n_groups=1, chunk=32), [130]),
]


@pytest.mark.parametrize("name,shape,Ts", Y_CASES, ids=[c[0] for c in Y_CASES])
def test_scan_per_token_outputs_match_the_sequential_recurrence(name, shape, Ts):
    for T in Ts:
        rng = I.rng_streams(1000 + T)[0]
        sc = I.make_scan_inputs(shape, T, rng, with_c=True, h0_scale=0.5)
        # C scaled by a power of two near 1/sqrt(N) (exact in the storage dtype), so that y is of
        # order one like the layer's outputs, where the absolute bound means something
        sc["C"] = sc["C"] * np.float32(2.0 ** -round(np.log2(np.sqrt(shape.d_state))))
        say("hyf_ssd_scan y", name, "T", T)
        H, y = run_scan(shape, sc, T, with_y=True)
        refH, refy = O.ssd_sequential(sc["x"], sc["B"], sc["C"], sc["dt_raw"], sc["a_log"], sc["dt_bias"],
                                      sc["d_skip"], sc["H0"], shape.n_groups)
        assert_close(H, refH, shape.dtype, f"{name} T={T} H")
        assert_close(y, refy, shape.dtype, f"{name} T={T} y")
        # the y-mode state equals the state-only scan's
        assert_close(H, run_scan(shape, sc, T), shape.dtype, f"{name} T={T} H vs state-only")


def test_scan_full_size_qwen_prefix_sampled_heads():
    # The 8192-token Qwen-shaped prefix as the benchmark runs it; the oracle checks 4 of 32 heads.
    shape, T = I.QWEN, 8192
    sc = I.make_scan_inputs(shape, T, I.rng_streams(11)[0], with_c=False, h0_scale=0.5)
    say("hyf_ssd_scan qwen T", T)
    H = run_scan(shape, sc, T)
    for h in (0, 9, 22, 31):
        sl = slice(h, h + 1)
        ref, _ = O.ssd_sequential(sc["x"][:, sl], sc["B"], None, sc["dt_raw"][:, sl], sc["a_log"][sl],
                                  sc["dt_bias"][sl], sc["d_skip"][sl], sc["H0"][sl])
        assert_close(H[sl], ref, "bf16", f"head {h}")


def test_scan_full_size_qwen_prefix_per_token_outputs_sampled_heads():
    # The 8192-token Qwen-shaped prefix with per-token outputs, at the size the benchmark runs the
    # y-mode kernels (64 blocks x 32 heads); the oracle checks the final state and y on 3 of 32 heads.
    shape, T = I.QWEN, 8192
    sc = I.make_scan_inputs(shape, T, I.rng_streams(13)[0], with_c=True, h0_scale=0.5)
    sc["C"] = sc["C"] * np.float32(2.0 ** -round(np.log2(np.sqrt(shape.d_state))))
    say("hyf_ssd_scan y qwen T", T)
    H, y = run_scan(shape, sc, T, with_y=True)
    for h in (0, 17, 31):
        sl = slice(h, h + 1)
        refH, refy = O.ssd_sequential(sc["x"][:, sl], sc["B"], sc["C"], sc["dt_raw"][:, sl], sc["a_log"][sl],
                                      sc["dt_bias"][sl], sc["d_skip"][sl], sc["H0"][sl])
        assert_close(H[sl], refH, "bf16", f"head {h} H")
        assert_close(y[:, sl], refy, "bf16", f"head {h} y")


def test_scan_is_deterministic():
    shape, T = I.QWEN, 3000
    sc = I.make_scan_inputs(shape, T, I.rng_streams(12)[0], with_c=False, h0_scale=0.5)
    say("hyf_ssd_scan determinism")
    a = run_scan(shape, sc, T)
    b = run_scan(shape, sc, T)
    assert np.array_equal(a, b)


def test_scan_per_token_outputs_are_deterministic():
    # The y-mode kernels use no atomics: the final state and every output repeat bit for bit.
    shape, T = I.QWEN, 3000
    sc = I.make_scan_inputs(shape, T, I.rng_streams(14)[0], with_c=True, h0_scale=0.5)
    say("hyf_ssd_scan y determinism")
    Ha, ya = run_scan(shape, sc, T, with_y=True)
    Hb, yb = run_scan(shape, sc, T, with_y=True)
    assert np.array_equal(Ha, Hb)
    assert np.array_equal(ya, yb)


def test_scan_zero_length_is_a_noop():
    shape = I.TINY
    sc = I.make_scan_inputs(shape, 4, I.rng_streams(13)[0], with_c=False, h0_scale=1.0)
    say("hyf_ssd_scan T=0")
    cfg = hf.make_config(shape)
    H = torch.from_numpy(sc["H0"]).to(DEV)
    f = torch.zeros(4, device=DEV)
    hf.check(hf.hyf_ssd_scan(cfg, None, None, None, None, f, f, f, H, None, 0, None, 0))
    torch.cuda.synchronize()
    assert np.array_equal(H.cpu().numpy(), sc["H0"])


# ---------------------------------------------------------------- projection level

LINEAR_CASES = [  # (dtype, K, Nout, Ms): K tails past a 128-wide slab, M across 16-row tiles
    ("bf16", 144, 7, [1, 16, 17, 40, 64, 65, 200]),
    ("bf16", 2560, 300, [1, 12, 16, 33, 64, 130]),
    ("bf16", 5120, 40, [8, 49]),
    # K past the last 128-wide slab on the double-buffered kernel (one 16-row tile, K >= 2048):
    # its loads past K are clamped and zeroed
    ("bf16", 2184, 300, [1, 8, 16]),
    # the MFMA GEMM (K a multiple of 64, M > 64), its tile chosen by the product's size.  64 x 64
    # tiles: one, two and three K steps (the three-stage pipeline's edges), ragged row and feature
    # tiles
    ("bf16", 64, 130, [65, 257]),
    ("bf16", 128, 129, [100]),
    ("bf16", 192, 256, [300]),
    # 128 x 128 tiles (176 of them, two stages)
    ("bf16", 256, 2720, [1000]),
    # 128 x 64 tiles (164), ragged rows and features
    ("bf16", 128, 2600, [500]),
    # 128 x 128 tiles (384), ragged features
    ("bf16", 128, 3000, [2000]),
    # 256 x 128 tiles (423, 16 waves, three stages), ragged rows and features
    ("bf16", 128, 6000, [2100]),
    # 256 x 256 tiles (256, two stages; the epilogue in two feature passes), ragged rows and
    # features, three K steps
    ("bf16", 192, 4000, [4090]),
    ("f32", 256, 100, [1, 20, 64, 65]),
]


@pytest.mark.parametrize("dtype,K,Nout,Ms", LINEAR_CASES, ids=[f"{c[0]}_K{c[1]}_N{c[2]}" for c in LINEAR_CASES])
def test_linear_matches_the_oracle(dtype, K, Nout, Ms):
    shape = small_shape(dtype)
    cfg = hf.make_config(shape)
    rng = I.rng_streams(K + Nout)
    Wt = I.make_rows(rng[0], Nout, K, 1.0 / np.sqrt(K), dtype)
    Wd = hf.to_device(Wt, shape)
    for M in Ms:
        X = I.make_rows(rng[1], M, K, 1.0, dtype)
        Xd = hf.to_device(X, shape)
        ref = O.project(X, Wt)
        for out_f32 in (1, 0):
            out = torch.full((M, Nout), float("nan"), device=DEV,
                             dtype=torch.float32 if out_f32 else hf.torch_dtype(shape))
            say("hyf_linear", dtype, "M", M, "K", K, "N", Nout, "f32 out" if out_f32 else "storage out")
            hf.check(hf.hyf_linear(cfg, Xd, M, K, Wd, Nout, out, out_f32), "hyf_linear")
            torch.cuda.synchronize()
            assert_close(out.float().cpu().numpy(), ref, dtype, f"linear M={M} K={K} out_f32={out_f32}")


@pytest.mark.parametrize("K", [2560, 2184])
def test_linear_rows_do_not_depend_on_the_batch(K):
    # A row's projection is bit-identical whatever other rows share the call (M <= 64): the K split
    # over waves depends on K alone, so the double-buffered one-tile kernel (M <= 16) and the
    # single-buffered one give the same bits, also for a K that ends inside a 128-wide slab.
    shape = I.QWEN
    cfg = hf.make_config(shape)
    rng = I.rng_streams(77)
    Nout = 200
    Wd = hf.to_device(I.make_rows(rng[0], Nout, K, 1.0 / np.sqrt(K), "bf16"), shape)
    X = hf.to_device(I.make_rows(rng[1], 64, K, 1.0, "bf16"), shape)
    outs = {}
    for M in (64, 33, 16, 5, 1):
        out = torch.empty(M, Nout, device=DEV, dtype=torch.float32)
        say("hyf_linear batch independence K", K, "M", M)
        hf.check(hf.hyf_linear(cfg, X, M, K, Wd, Nout, out, 1), "hyf_linear")
        torch.cuda.synchronize()
        outs[M] = out.cpu()
    for M in (33, 16, 5, 1):
        assert torch.equal(outs[M], outs[64][:M]), M


W4_CASES = [  # (K, Nout, Ms): one 128-wide group; fewer groups than waves; 17 groups (a ragged
    # split over 8 waves); the round projections of the Qwen3-4B-shaped layer (12 rows x w_in,
    # 8 rows x w_out); rows across 16-row tiles and past the 64-row slab of one workgroup;
    # more feature tiles than CUs
    (128, 17, [1, 16, 17, 64, 65, 130]),
    (384, 100, [3, 33]),
    (2176, 48, [40]),
    (2560, 7968, [12]),
    (2560, 2560, [8]),
    (256, 4129, [20, 5]),  # 259 feature tiles: two per workgroup, the last one past Nout
    (5120, 4200, [8, 20]),  # 40 groups: a wave loops over several batches of in-flight groups
]


@pytest.mark.parametrize("K,Nout,Ms", W4_CASES, ids=[f"K{c[0]}_N{c[1]}" for c in W4_CASES])
def test_four_bit_linear_matches_the_oracle(K, Nout, Ms):
    """Every code 0..15 appears (random bytes), one group has scale 0; the codes are exact in the
    kernel, so fp32 output differs from the oracle by fp32 accumulation only."""
    shape = I.QWEN
    cfg = hf.make_config(shape)
    rng = I.rng_streams(K * 7 + Nout)
    packed = rng[0].integers(0, 256, size=(Nout, K // 2), dtype=np.uint8)
    scales = (np.abs(rng[0].standard_normal((Nout, K // 128))) / (7.0 * np.sqrt(K))).astype(np.float32)
    scales[Nout // 2, (K // 128) // 2] = 0.0
    Wq = torch.from_numpy(packed).to(DEV)
    Sd = torch.from_numpy(scales).to(DEV)
    for M in Ms:
        X = I.make_rows(rng[1], M, K, 1.0, "bf16")
        Xd = hf.to_device(X, shape)
        ref = O.linear_w4(X, packed, scales)
        for out_f32 in (1, 0):
            out = torch.full((M, Nout), float("nan"), device=DEV, dtype=torch.float32 if out_f32 else torch.bfloat16)
            say("hyf_linear_w4 M", M, "K", K, "N", Nout, "f32 out" if out_f32 else "bf16 out")
            hf.check(hf.hyf_linear_w4(cfg, Xd, M, K, Wq, Sd, Nout, out, out_f32), "hyf_linear_w4")
            torch.cuda.synchronize()
            assert_close(out.float().cpu().numpy(), ref, "f32" if out_f32 else "bf16",
                         f"linear_w4 M={M} K={K} N={Nout} out_f32={out_f32}")


def test_four_bit_linear_of_quantized_xavier_weights():
    """Weights quantized by the oracle's round-to-nearest rule: the 4-bit projection of the w_in
    shape against the oracle's product of the same codes."""
    shape = I.QWEN
    cfg = hf.make_config(shape)
    rng = I.rng_streams(4242)
    K, Nout, M = shape.d_model, 1024, 12
    W = I.make_rows(rng[0], Nout, K, 1.0 / np.sqrt(K), "f32")
    packed, scales = O.quantize_w4(W)
    X = I.make_rows(rng[1], M, K, 1.0, "bf16")
    out = torch.empty(M, Nout, device=DEV, dtype=torch.float32)
    say("hyf_linear_w4 quantized weights M", M, "K", K, "N", Nout)
    hf.check(hf.hyf_linear_w4(cfg, hf.to_device(X, shape), M, K, torch.from_numpy(packed).to(DEV),
                              torch.from_numpy(scales).to(DEV), Nout, out, 1), "hyf_linear_w4")
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), O.linear_w4(X, packed, scales), "f32", "linear_w4 quantized")


def test_four_bit_linear_replays_in_a_graph():
    """One call captured in a HIP graph, replayed three times with new rows written eagerly
    between the replays: every replay matches the eager call on the same rows."""
    shape = I.QWEN
    cfg = hf.make_config(shape)
    rng = I.rng_streams(515)
    K, Nout, M = 512, 300, 12
    packed = torch.from_numpy(rng[0].integers(0, 256, size=(Nout, K // 2), dtype=np.uint8)).to(DEV)
    scales = torch.from_numpy((np.abs(rng[0].standard_normal((Nout, K // 128))) * 0.02).astype(np.float32)).to(DEV)
    X = torch.zeros(M, K, device=DEV, dtype=torch.bfloat16)
    out = torch.zeros(M, Nout, device=DEV, dtype=torch.float32)
    say("hyf_linear_w4 graph capture")
    hf.check(hf.hyf_linear_w4(cfg, X, M, K, packed, scales, Nout, out, 1), "hyf_linear_w4")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        hf.check(hf.hyf_linear_w4(cfg, X, M, K, packed, scales, Nout, out, 1), "hyf_linear_w4")
    for rep in range(3):
        Xn = hf.to_device(I.make_rows(rng[1], M, K, 1.0, "bf16"), shape)
        X.copy_(Xn)
        eager = torch.empty_like(out)
        hf.check(hf.hyf_linear_w4(cfg, Xn, M, K, packed, scales, Nout, eager, 1), "hyf_linear_w4")
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), rep


# ---------------------------------------------------------------- layer level


class Pair:
    """The HIP layer and the oracle side by side, fed the same rows."""

    def __init__(self, shape, seed, pool_slots=1, max_requests=1, max_rows=8, d_random=True):
        self.shape = shape
        self.rng = I.rng_streams(seed)
        self.w = I.make_weights(shape, self.rng[0], d_random=d_random)
        self.wo = {k: np.asarray(v, np.float64) for k, v in self.w.items()}
        self.gpu = hf.DrafterLayer(shape, self.w, pool_slots=pool_slots, max_requests=max_requests,
                                   max_rows=max_rows)
        self.ost = [O.new_state(shape) for _ in range(pool_slots)]

    def rows(self, n, stream=1):
        return I.make_rows(self.rng[stream], n, self.shape.d_model, 1.0 / np.sqrt(self.shape.d_model),
                           self.shape.dtype)

    def commit(self, feats_list, slots=None):
        cu = np.concatenate([[0], np.cumsum([len(f) for f in feats_list])]).astype(np.int64)
        allf = np.concatenate(feats_list) if cu[-1] else np.zeros((0, self.shape.d_model), np.float32)
        self.gpu.commit(hf.to_device(allf, self.shape) if cu[-1] else None, cu, slots)
        for i, f in enumerate(feats_list):
            s = slots[i] if slots is not None else i
            self.ost[s], _ = O.commit(self.shape, self.wo, self.ost[s], f)

    def draft(self, blocks, commits=None, slots=None):
        R = len(blocks)
        bi = hf.to_device(np.concatenate(blocks), self.shape)
        bo = torch.empty_like(bi)
        cf = cu = None
        if commits is not None:
            cu = np.concatenate([[0], np.cumsum([len(f) for f in commits])]).astype(np.int64)
            cf = hf.to_device(np.concatenate(commits), self.shape) if cu[-1] else None
            if cf is None:
                cf = hf.to_device(np.zeros((1, self.shape.d_model), np.float32), self.shape)
        self.gpu.draft(bi, bo, cf, cu, slots)
        outs = []
        for i in range(R):
            s = slots[i] if slots is not None else i
            if commits is not None:
                self.ost[s], _ = O.commit(self.shape, self.wo, self.ost[s], commits[i])
            outs.append(O.draft(self.shape, self.wo, self.ost[s], blocks[i]))
        torch.cuda.synchronize()
        return bo.float().cpu().numpy().reshape(R, hf.HYF_BLOCK, -1), np.stack(outs)

    def check_state(self, slot=0, what=""):
        torch.cuda.synchronize()
        g = self.gpu.state(slot)
        o = self.ost[slot]
        assert int(g["count"].item()) == o["count"], what
        assert_close(g["H"].cpu().numpy(), o["H"], self.shape.dtype, f"{what} H")
        n = min(o["count"], self.shape.window)
        assert_close(g["K"].float().cpu().numpy()[:, :n], o["K"][:, :n], self.shape.dtype, f"{what} K")
        assert_close(g["V"].float().cpu().numpy()[:, :n], o["V"][:, :n], self.shape.dtype, f"{what} V")


LAYER_SHAPES = [
    ("tiny_fp32", I.TINY),
    ("small_bf16", small_shape("bf16", window=40)),
    ("odd_bf16", small_shape("bf16", n_heads=5, head_dim=48, d_state=32, n_groups=5, window=20, chunk=32)),
    ("noncross_fp32", small_shape("f32", window=24, cross_slot=0)),
]


@pytest.mark.parametrize("name,shape", LAYER_SHAPES, ids=[c[0] for c in LAYER_SHAPES])
def test_rounds_match_the_oracle(name, shape):
    pr = Pair(shape, seed=21, max_rows=400)
    say("hyf_state_reset", name)
    pr.gpu.reset()
    say("hyf_draft_block on an empty state", name)
    g, o = pr.draft([pr.rows(8, 3)])
    assert_close(g, o, shape.dtype, f"{name} empty")
    say("hyf_memory_commit prefill 300", name)
    pr.commit([pr.rows(300)])
    pr.check_state(what=f"{name} prefill")
    acc_rng = pr.rng[4]
    for rnd in range(12):
        a = int(acc_rng.integers(1, 9))
        say("hyf_draft_block round", rnd, "a", a, name)
        g, o = pr.draft([pr.rows(8, 3)], commits=[pr.rows(a)])
        assert_close(g, o, shape.dtype, f"{name} round {rnd}")
    pr.check_state(what=f"{name} after rounds")
    say("hyf_memory_commit small", name)
    pr.commit([pr.rows(5)])
    pr.check_state(what=f"{name} small commit")


Y_LAYER_SHAPES = [
    ("tiny_fp32", I.TINY),
    ("small_bf16", small_shape("bf16", window=40)),
    ("odd_bf16", small_shape("bf16", n_heads=5, head_dim=48, d_state=32, n_groups=5, window=20, chunk=32)),
]


@pytest.mark.parametrize("name,shape", Y_LAYER_SHAPES, ids=[c[0] for c in Y_LAYER_SHAPES])
def test_commit_per_token_outputs_match_the_oracle(name, shape):
    # Ragged multi-request commits with y; rows of one request never leak into another's y, and the
    # state they leave is the one the oracle's commit leaves.
    pr = Pair(shape, seed=61, pool_slots=4, max_requests=4, max_rows=700)
    pr.gpu = hf.DrafterLayer(shape, pr.w, pool_slots=4, max_requests=4, max_rows=700, with_y=True)
    pr.gpu.reset()
    for step, lens in enumerate(([200, 0, 129, 1], [5, 300, 8, 128])):
        feats = [pr.rows(n) for n in lens]
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
        y = torch.full((int(cu[-1]), shape.n_heads, shape.head_dim), float("nan"), dtype=hf.torch_dtype(shape),
                       device=DEV)
        say("hyf_memory_commit y", name, "lens", lens)
        pr.gpu.commit(hf.to_device(np.concatenate(feats), shape), cu, y=y)
        torch.cuda.synchronize()
        got = y.float().cpu().numpy()
        for i, f in enumerate(feats):
            pr.ost[i], ref = O.commit(shape, pr.wo, pr.ost[i], f, want_y=True)
            assert_close(got[cu[i]:cu[i + 1]], ref, shape.dtype, f"{name} step {step} request {i} y")
        for i in range(4):
            pr.check_state(slot=i, what=f"{name} step {step} request {i}")
    # a round afterwards sees the same memory as the oracle
    say("hyf_draft_block after y commits", name)
    g, o = pr.draft([pr.rows(8, 3) for _ in range(4)], commits=[pr.rows(a) for a in (0, 3, 8, 1)])
    assert_close(g, o, shape.dtype, f"{name} round after y")


GDN_SHAPES = [
    ("tiny_fp32", I.TINY.replace(memory="gdn")),
    ("small_bf16", small_shape("bf16", window=40, memory="gdn")),
    ("odd_bf16", small_shape("bf16", n_heads=5, head_dim=48, d_state=32, n_groups=5, window=20, chunk=32, memory="gdn")),
    ("noncross_fp32", small_shape("f32", window=24, cross_slot=0, memory="gdn")),
]


@pytest.mark.parametrize("name,shape", GDN_SHAPES, ids=[c[0] for c in GDN_SHAPES])
def test_gated_delta_rule_rounds_match_the_oracle(name, shape):
    # prefill (the sequential prefix kernel), rounds (the round kernel's tiles), a small commit
    pr = Pair(shape, seed=71, max_rows=400)
    pr.gpu.reset()
    say("gdn hyf_draft_block on an empty state", name)
    g, o = pr.draft([pr.rows(8, 3)])
    assert_close(g, o, shape.dtype, f"gdn {name} empty")
    say("gdn hyf_memory_commit prefill 300", name)
    pr.commit([pr.rows(300)])
    pr.check_state(what=f"gdn {name} prefill")
    acc_rng = pr.rng[4]
    for rnd in range(8):
        a = int(acc_rng.integers(1, 9))
        say("gdn hyf_draft_block round", rnd, "a", a, name)
        g, o = pr.draft([pr.rows(8, 3)], commits=[pr.rows(a)])
        assert_close(g, o, shape.dtype, f"gdn {name} round {rnd}")
    pr.check_state(what=f"gdn {name} after rounds")
    say("gdn hyf_memory_commit small", name)
    pr.commit([pr.rows(13)])
    pr.check_state(what=f"gdn {name} small commit")


def test_gated_delta_rule_chunk_edges_in_one_call():
    # The chunked prefix commit over requests whose lengths sit on and around its 64-token chunks
    # and 128-token blocks (one call, eight requests), then a second prefill on top of each state.
    shape = small_shape("bf16", window=40, memory="gdn")
    lens = [17, 63, 64, 65, 127, 128, 129, 200]
    pr = Pair(shape, seed=73, pool_slots=8, max_requests=8, max_rows=2 * sum(lens))
    pr.gpu.reset()
    say("gdn chunk edges prefill", lens)
    pr.commit([pr.rows(n) for n in lens])
    for i in range(8):
        pr.check_state(slot=i, what=f"gdn chunk edges request {i} ({lens[i]} rows)")
    say("gdn chunk edges second prefill")
    pr.commit([pr.rows(n) for n in reversed(lens)])
    for i in range(8):
        pr.check_state(slot=i, what=f"gdn chunk edges request {i} second prefill")


def test_gated_delta_rule_prefix_with_d_state_224():
    # bf16 d_state 224 is taken by the chunked prefix kernels only (the token-by-token one keeps at
    # most 192 state columns per row): a prefill, rounds on top, and a second prefill.
    shape = small_shape("bf16", head_dim=64, d_state=224, window=40, memory="gdn")
    pr = Pair(shape, seed=75, max_rows=400)
    pr.gpu.reset()
    say("gdn d_state 224 prefill 300")
    pr.commit([pr.rows(300)])
    pr.check_state(what="gdn N224 prefill")
    for rnd in range(3):
        say("gdn d_state 224 round", rnd)
        g, o = pr.draft([pr.rows(8, 3)], commits=[pr.rows(2 + 3 * rnd)])
        assert_close(g, o, "bf16", f"gdn N224 round {rnd}")
    say("gdn d_state 224 second prefill 130")
    pr.commit([pr.rows(130)])
    pr.check_state(what="gdn N224 second prefill")


def test_gated_delta_rule_rounds_of_sixteen_requests():
    # Sixteen Qwen-shaped requests with ragged chunked prefixes, then rounds in which every request
    # commits its own number of accepted rows (512 (request, head) pairs per round kernel).
    shape = I.QWEN.replace(memory="gdn")
    R = 16
    pr = Pair(shape, seed=74, pool_slots=R, max_requests=R, max_rows=64 * R)
    pr.gpu.reset()
    lens = [17 + 3 * i for i in range(R)]
    say("gdn sixteen requests prefill", lens)
    pr.commit([pr.rows(n) for n in lens])
    acc_rng = pr.rng[4]
    for rnd in range(2):
        acc = [int(a) for a in acc_rng.integers(1, 9, size=R)]
        say("gdn sixteen requests round", rnd, acc)
        g, o = pr.draft([pr.rows(8, 3) for _ in range(R)], commits=[pr.rows(a) for a in acc])
        assert_close(g, o, "bf16", f"gdn sixteen requests round {rnd}")
    for i in (0, 7, 15):
        pr.check_state(slot=i, what=f"gdn sixteen requests state {i}")


def test_gated_delta_rule_qwen_prefill_batched_and_rounds():
    # Qwen-shaped gated delta-rule layer: two requests with ragged prefixes (one of them spans
    # several time blocks), then rounds over both
    shape = I.QWEN.replace(memory="gdn")
    pr = Pair(shape, seed=72, pool_slots=2, max_requests=2, max_rows=2100)
    pr.gpu.reset()
    say("gdn qwen prefill 1500 + 555")
    pr.commit([pr.rows(1500), pr.rows(555)])
    for s2 in (0, 1):
        pr.check_state(slot=s2, what=f"gdn qwen prefill {s2}")
    for rnd in range(3):
        say("gdn qwen round", rnd)
        g, o = pr.draft([pr.rows(8, 3), pr.rows(8, 3)], commits=[pr.rows(5), pr.rows(2)])
        assert_close(g, o, "bf16", f"gdn qwen round {rnd}")
    pr.check_state(slot=1, what="gdn qwen rounds")


LASTW_SHAPES = [
    ("tiny_fp32", I.TINY.replace(memory="lastw")),
    ("small_bf16", small_shape("bf16", window=40, memory="lastw")),
    ("odd_bf16", small_shape("bf16", n_heads=5, head_dim=48, d_state=32, n_groups=5, window=20, chunk=32,
                             memory="lastw")),
]


@pytest.mark.parametrize("name,shape", LASTW_SHAPES, ids=[c[0] for c in LASTW_SHAPES])
def test_last_w_memory_matches_the_oracle(name, shape):
    # The last-W memory: prefills longer and shorter than the window (the rescan pads the short
    # windows), rounds that commit 0-8 rows per request (commit, rescan, then draft), a round-sized
    # commit; states (H = the window's scan, rings with B and steps) and outputs against the oracle.
    pr = Pair(shape, seed=91, pool_slots=3, max_requests=3, max_rows=700)
    pr.gpu.reset()
    lens = [300, 7, 0]
    say("last-W prefill", name, lens)
    pr.commit([pr.rows(n) for n in lens])
    for i in range(2):
        pr.check_state(slot=i, what=f"lastw {name} prefill {i}")
    acc_rng = pr.rng[4]
    for rnd in range(6):
        acc = [int(a) for a in acc_rng.integers(0, 9, size=3)]
        say("last-W round", rnd, name, acc)
        g, o = pr.draft([pr.rows(8, 3) for _ in range(3)], commits=[pr.rows(a) for a in acc])
        for i in range(3):
            assert_close(g[i], o[i], shape.dtype, f"lastw {name} round {rnd} request {i}")
    say("last-W small commit", name)
    pr.commit([pr.rows(5)], slots=[2])
    for i in range(3):
        pr.check_state(slot=i, what=f"lastw {name} final {i}")
        st, ost = pr.gpu.state(i), pr.ost[i]
        n = min(ost["count"], shape.window)
        slots = (ost["count"] - n + np.arange(n)) % shape.window
        assert_close(st["Bring"].float().cpu().numpy()[slots], ost["Bring"][slots], shape.dtype, f"lastw B ring {i}")
        assert_close(st["DTring"].cpu().numpy()[:, slots], ost["DTring"][slots].T, "f32", f"lastw step ring {i}")


def w4_weights(shape, seed):
    """Xavier weights of the shape, quantized with the oracle's round-to-nearest 4-bit format: the
    GPU gets the codes and scales, the oracle the same codes and scales."""
    w = I.make_weights(shape, I.rng_streams(seed)[0], d_random=True)
    qi, si = O.quantize_w4(w["w_in"])
    qo, so = O.quantize_w4(w["w_out"])
    w.update(w_in_q=qi, w_in_s=si, w_out_q=qo, w_out_s=so)
    return w


W4_LAYER_SHAPES = [
    ("small_bf16", small_shape("bf16", window=40, weights="w4")),
    ("qwen_bf16", I.QWEN.replace(weights="w4")),
    ("gdn_bf16", small_shape("bf16", window=40, memory="gdn", weights="w4")),
]


@pytest.mark.parametrize("name,shape", W4_LAYER_SHAPES, ids=[c[0] for c in W4_LAYER_SHAPES])
def test_four_bit_layer_matches_the_oracle(name, shape):
    # The layer with 4-bit projection weights: a prefill (codes expanded to bf16, then the GEMM), rounds
    # (codes streamed by the 4-bit kernel), a round-sized commit, and a batched round of three requests.
    w = w4_weights(shape, 41)
    wo = {k: (np.asarray(v) if k.endswith("_q") else np.asarray(v, np.float64)) for k, v in w.items()
          if k not in ("w_in", "w_out")}
    layer = hf.DrafterLayer(shape, w, pool_slots=3, max_requests=3, max_rows=1000)
    layer.reset()
    rng = I.rng_streams(42)
    sc = 1.0 / np.sqrt(shape.d_model)
    rows = lambda n, st=1: I.make_rows(rng[st], n, shape.d_model, sc, shape.dtype)
    ost = [O.new_state(shape) for _ in range(3)]
    pre = [rows(n) for n in (300, 17, 600)]
    say("w4 layer prefill", name)
    layer.commit(hf.to_device(np.concatenate(pre), shape), np.concatenate([[0], np.cumsum([300, 17, 600])]))
    for i in range(3):
        ost[i], _ = O.commit(shape, wo, ost[i], pre[i])
    torch.cuda.synchronize()
    for i in range(3):
        g = layer.state(i)
        assert_close(g["H"].cpu().numpy(), ost[i]["H"], "bf16", f"w4 {name} prefill H {i}")
    for rnd in range(3):
        acc = [int(a) for a in rng[4].integers(1, 9, size=3)]
        commits = [rows(a, 2) for a in acc]
        blocks = [rows(8, 3) for _ in range(3)]
        bi = hf.to_device(np.concatenate(blocks), shape)
        bo = torch.empty_like(bi)
        say("w4 layer round", rnd, name)
        layer.draft(bi, bo, hf.to_device(np.concatenate(commits), shape), np.concatenate([[0], np.cumsum(acc)]))
        torch.cuda.synchronize()
        got = bo.float().cpu().numpy().reshape(3, 8, -1)
        for i in range(3):
            ost[i], ref = O.round_step(shape, wo, ost[i], commits[i], blocks[i])
            assert_close(got[i], ref, "bf16", f"w4 {name} round {rnd} request {i}")
    small = rows(5)
    say("w4 layer small commit", name)
    layer.commit(hf.to_device(small, shape), [0, 5], slots=[1])
    ost[1], _ = O.commit(shape, wo, ost[1], small)
    torch.cuda.synchronize()
    g = layer.state(1)
    assert int(g["count"].item()) == ost[1]["count"]
    assert_close(g["H"].cpu().numpy(), ost[1]["H"], "bf16", f"w4 {name} small commit H")


def test_qwen_full_size_prefill_and_rounds():
    # The 8192-row Qwen-shaped prefix and a few rounds, exactly as the benchmark launches them.
    shape = I.QWEN
    pr = Pair(shape, seed=31, max_rows=8192, d_random=False)
    pr.gpu.reset()
    say("hyf_memory_commit qwen prefill 8192")
    pr.commit([pr.rows(8192)])
    pr.check_state(what="qwen prefill")
    for rnd in range(3):
        a = [3, 8, 1][rnd]
        say("hyf_draft_block qwen round", rnd, "a", a)
        g, o = pr.draft([pr.rows(8, 3)], commits=[pr.rows(a)])
        assert_close(g, o, "bf16", f"qwen round {rnd}")
    pr.check_state(what="qwen rounds")


def test_draft_never_writes_the_state():
    shape = small_shape("bf16", window=40)
    pr = Pair(shape, seed=41, max_rows=100)
    pr.gpu.reset()
    pr.commit([pr.rows(57)])
    torch.cuda.synchronize()
    before = pr.gpu.state()["blob"].clone()
    say("hyf_draft_block read-only")
    pr.draft([pr.rows(8, 3)])
    assert torch.equal(pr.gpu.state()["blob"], before)


def test_state_after_a_round_is_independent_of_the_block_rows():
    # H and the ring after draft(commit=F, block=X) equal those after draft(commit=F, block=X'), and
    # those after a standalone commit of F, bit for bit: block rows never enter the memory.
    shape = small_shape("bf16", window=40)
    seeds = []
    for variant in range(3):
        pr = Pair(shape, seed=51, max_rows=100)
        pr.gpu.reset()
        pr.commit([pr.rows(33)])
        F = pr.rows(6)
        X = pr.rows(8, 3) if variant != 1 else pr.rows(8, 5)
        say("I3/I4 variant", variant)
        if variant < 2:
            pr.draft([X], commits=[F])
        else:
            pr.commit([F])
        torch.cuda.synchronize()
        seeds.append(pr.gpu.state()["blob"].clone())
    assert torch.equal(seeds[0], seeds[1])
    assert torch.equal(seeds[0], seeds[2])


def test_split_invariance_of_commits():
    # Cutting 10 committed rows into rounds of at most 8 leaves H within tolerance of one commit.
    shape = small_shape("f32", window=6)
    comps = [p for p in (list(c) for c in itertools.product(range(1, 9), repeat=2)) if sum(p) == 10]
    comps += [[1] * 10, [10], [8, 2], [2, 8], [3, 3, 4], [1, 8, 1]]
    ref = None
    for parts in comps:
        pr = Pair(shape, seed=61, max_rows=16)
        F = pr.rows(10)
        pr.gpu.reset()
        say("split", parts)
        i = 0
        for p in parts:
            pr.commit([F[i:i + p]])
            i += p
        pr.check_state(what=f"split {parts}")
        H = pr.gpu.state()["H"].cpu().numpy()
        if ref is None:
            ref = H
        assert_close(H, ref, "f32", f"split {parts}")


WIDE_SHAPES = [
    ("tiny_fp32", I.TINY),
    ("small_bf16_w40", small_shape("bf16", window=40)),
    ("gdn_bf16", small_shape("bf16", window=100, memory="gdn")),
    ("odd_bf16", small_shape("bf16", n_heads=5, head_dim=48, d_state=32, n_groups=5, window=20, chunk=32)),
    ("noncross_fp32", small_shape("f32", window=24, cross_slot=0)),
    # bf16 draft rounds over 256+ (request, head) pairs take one workgroup per pair: block rows
    # that see only themselves, the last-W memory, a window of one 64-slot chunk plus one slot
    ("noncross_bf16", small_shape("bf16", window=65, cross_slot=0)),
    ("lastw_bf16", small_shape("bf16", window=72, memory="lastw")),
    # heads of 128 dimensions over 256 (request, head) pairs: the wide layout (whole-head tiles,
    # 128-key splits)
    ("wide_p128_bf16", small_shape("bf16", head_dim=128, window=300)),
    ("wide_p128_gdn_fp32", small_shape("f32", head_dim=128, d_state=32, window=130, memory="gdn")),
]


@pytest.mark.parametrize("name,shape", WIDE_SHAPES, ids=[c[0] for c in WIDE_SHAPES])
def test_rounds_of_many_requests_match_the_oracle(name, shape):
    # 64 requests (256-320 (request, head) pairs) with ragged prefixes around the window, then
    # rounds in which every request commits 0-8 rows; every request against the oracle.
    R = 64
    pr = Pair(shape, seed=81, pool_slots=R, max_requests=R, max_rows=300 * R)
    pr.gpu.reset()
    lens = [(37 * i) % 300 for i in range(R)]
    say("wide layout prefill", name, "rows", sum(lens))
    pr.commit([pr.rows(n) for n in lens])
    acc_rng = pr.rng[4]
    for rnd in range(3):
        acc = [int(a) for a in acc_rng.integers(0, 9, size=R)]
        say("wide layout round", rnd, name)
        g, o = pr.draft([pr.rows(8, 3) for _ in range(R)], commits=[pr.rows(a) for a in acc])
        for i in range(R):
            assert_close(g[i], o[i], shape.dtype, f"{name} round {rnd} request {i}")
    for i in (0, 13, 63):
        pr.check_state(slot=i, what=f"{name} wide state {i}")


def test_batched_requests_with_a_slot_table():
    shape = small_shape("bf16", window=48)
    R, pool = 5, 8
    slots = [6, 1, 3, 0, 7]
    pr = Pair(shape, seed=71, pool_slots=pool, max_requests=R, max_rows=2000)
    pr.gpu.reset()
    lens = [300, 17, 0, 129, 64]
    say("batched prefill", lens)
    pr.commit([pr.rows(n) for n in lens], slots=slots)
    for s in slots:
        pr.check_state(s, what=f"prefill slot {s}")
    arng = pr.rng[4]
    for rnd in range(4):
        a = [int(arng.integers(0 if rnd == 2 else 1, 9)) for _ in range(R)]
        say("batched round", rnd, a)
        g, o = pr.draft([pr.rows(8, 3) for _ in range(R)], commits=[pr.rows(n) for n in a], slots=slots)
        assert_close(g, o, "bf16", f"batched round {rnd}")
    for s in slots:
        pr.check_state(s, what=f"rounds slot {s}")
    # untouched slots stay zero
    for s in set(range(pool)) - set(slots):
        assert int(torch.count_nonzero(pr.gpu.state(s)["blob"]).item()) == 0


def test_rejected_call_leaves_the_state_untouched():
    shape = I.TINY
    pr = Pair(shape, seed=81, max_rows=64)
    pr.gpu.reset()
    pr.commit([pr.rows(20)])
    torch.cuda.synchronize()
    before = pr.gpu.state()["blob"].clone()
    f = hf.to_device(pr.rows(4), shape)
    say("rejected calls")
    st = hf.hyf_memory_commit(pr.gpu.cfg, pr.gpu.w, pr.gpu.pool, 1, None, 1, f, [0, 4], None, pr.gpu.ws, 64)
    assert st == hf.HYF_EWORKSPACE
    bi = hf.to_device(pr.rows(8), shape)
    st = hf.hyf_draft_block(pr.gpu.cfg, pr.gpu.w, pr.gpu.pool, 1, None, 1, f, [0, 9], bi, torch.empty_like(bi),
                            pr.gpu.ws, pr.gpu.ws_bytes)
    assert st == hf.HYF_ECAPACITY
    torch.cuda.synchronize()
    assert torch.equal(pr.gpu.state()["blob"], before)


def test_round_is_deterministic():
    shape = I.QWEN
    outs = []
    for _ in range(2):
        pr = Pair(shape, seed=91, max_rows=600, d_random=False)
        pr.gpu.reset()
        pr.gpu.commit(hf.to_device(pr.rows(600), shape), [0, 600])
        bi = hf.to_device(pr.rows(8, 3), shape)
        bo = torch.empty_like(bi)
        say("determinism round")
        pr.gpu.draft(bi, bo, hf.to_device(pr.rows(5), shape), [0, 5])
        torch.cuda.synchronize()
        outs.append((bo.clone(), pr.gpu.state()["blob"].clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_graph_replay_matches_eager():
    # A captured episode (reset, prefill, 4 rounds) replayed several times, with eager work and
    # synchronizations in between, reproduces the eager outputs and state bit for bit.
    shape = small_shape("bf16", window=40)
    pr = Pair(shape, seed=101, max_rows=300)
    L = pr.gpu
    feats = hf.to_device(pr.rows(300), shape)
    rounds = [(hf.to_device(pr.rows(a), shape), [0, a], hf.to_device(pr.rows(8, 3), shape)) for a in (3, 8, 1, 5)]
    outs = [torch.empty_like(r[2]) for r in rounds]

    def episode(stream):
        hf.check(hf.hyf_state_reset(L.cfg, L.pool, 1, None, 1, stream))
        hf.check(hf.hyf_memory_commit(L.cfg, L.w, L.pool, 1, None, 1, feats, [0, 300], None, L.ws, L.ws_bytes,
                                      stream))
        for (cf, cu, bi), bo in zip(rounds, outs):
            hf.check(hf.hyf_draft_block(L.cfg, L.w, L.pool, 1, None, 1, cf, cu, bi, bo, L.ws, L.ws_bytes, stream))

    say("graph: eager reference")
    episode(None)
    torch.cuda.synchronize()
    ref_out = [o.clone() for o in outs]
    ref_state = L.state()["blob"].clone()
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    with torch.cuda.stream(cs):
        episode(cs)
    torch.cuda.synchronize()
    say("graph: capture")
    with torch.cuda.graph(g, stream=cs):
        episode(cs)
    for rep in range(3):
        for o in outs:
            o.zero_()
        L.reset()
        junk = torch.empty((16, shape.n_in), dtype=torch.float32, device=DEV)
        hf.check(hf.hyf_linear(L.cfg, feats, 16, shape.d_model, L.w_in, shape.n_in, junk, 1))
        torch.cuda.synchronize()
        say("graph: replay", rep)
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref_out):
            assert torch.equal(o, r)
        assert torch.equal(L.state()["blob"], ref_state)



def test_qwen_rounds_of_eight_requests_match_the_oracle():
    # 8 Qwen3-4B-shaped requests are 256 (request, head) pairs: one workgroup per pair with heads of
    # 80 dimensions (two 32-dimension runs and a run of 16); prefixes on both sides of the window.
    shape = I.QWEN
    R = 8
    pr = Pair(shape, seed=111, pool_slots=R, max_requests=R, max_rows=700 * R)
    pr.gpu.reset()
    lens = [700, 3, 512, 0, 130, 513, 64, 600]
    say("qwen 8 requests prefill", lens)
    pr.commit([pr.rows(n) for n in lens])
    acc_rng = pr.rng[4]
    for rnd in range(3):
        acc = [int(a) for a in acc_rng.integers(0, 9, size=R)]
        say("qwen 8 requests round", rnd, acc)
        g, o = pr.draft([pr.rows(8, 3) for _ in range(R)], commits=[pr.rows(a) for a in acc])
        for i in range(R):
            assert_close(g[i], o[i], "bf16", f"qwen 8 requests round {rnd} request {i}")
    for i in (0, 3, 5):
        pr.check_state(slot=i, what=f"qwen 8 requests state {i}")


def test_per_pair_rounds_are_deterministic_and_replay_in_a_graph():
    # 64 requests of 4 heads (one workgroup per pair): two eager episodes agree bit for bit, and a
    # captured episode replayed three times (with eager work in between) reproduces them.
    shape = small_shape("bf16", window=70)
    R = 64
    pr = Pair(shape, seed=121, pool_slots=R, max_requests=R, max_rows=200 * R)
    L = pr.gpu
    lens = [(53 * i) % 200 for i in range(R)]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    feats = hf.to_device(np.concatenate([pr.rows(n) for n in lens]), shape)
    rounds = []
    for a in (np.arange(R) % 9, (np.arange(R) * 5) % 9):
        cr = np.concatenate([[0], np.cumsum(a)]).astype(np.int64)
        rounds.append((hf.to_device(pr.rows(int(cr[-1])), shape), cr, hf.to_device(pr.rows(8 * R, 3), shape)))
    outs = [torch.empty_like(r[2]) for r in rounds]

    def episode(stream):
        hf.check(hf.hyf_state_reset(L.cfg, L.pool, R, None, R, stream))
        hf.check(hf.hyf_memory_commit(L.cfg, L.w, L.pool, R, None, R, feats, cu, None, L.ws, L.ws_bytes, stream))
        for (cf, cr, bi), bo in zip(rounds, outs):
            hf.check(hf.hyf_draft_block(L.cfg, L.w, L.pool, R, None, R, cf, cr, bi, bo, L.ws, L.ws_bytes, stream))

    ref = None
    for run in range(2):
        say("per-pair eager episode", run)
        episode(None)
        torch.cuda.synchronize()
        got = ([o.clone() for o in outs], L.pool.clone())
        if ref is None:
            ref = got
        else:
            assert all(torch.equal(a, b) for a, b in zip(got[0], ref[0])) and torch.equal(got[1], ref[1])
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    with torch.cuda.stream(cs):
        episode(cs)
    torch.cuda.synchronize()
    say("per-pair graph capture")
    with torch.cuda.graph(g, stream=cs):
        episode(cs)
    for rep in range(3):
        for o in outs:
            o.zero_()
        L.pool.zero_()
        torch.cuda.synchronize()
        say("per-pair graph replay", rep)
        g.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(outs, ref[0]))
        assert torch.equal(L.pool, ref[1])

DEV_COUNT_SHAPES = [
    ("tiny_fp32", I.TINY, 2),
    ("small_bf16", small_shape("bf16", window=40), 3),
    ("gdn_bf16", small_shape("bf16", window=24, memory="gdn"), 2),
    ("lastw_bf16", small_shape("bf16", window=24, memory="lastw"), 2),
    ("qwen", I.QWEN, 1),
]


def _padded_commits(shape, commits):
    """[R*8][d] storage-dtype rows, request i's rows at i*8 .. (the rest of each slot NaN)."""
    R = len(commits)
    pad = np.full((R * hf.HYF_BLOCK, shape.d_model), np.nan, np.float32)
    for i, c in enumerate(commits):
        pad[i * hf.HYF_BLOCK: i * hf.HYF_BLOCK + len(c)] = c
    return hf.to_device(pad, shape)


@pytest.mark.parametrize("name,shape,R", DEV_COUNT_SHAPES, ids=[c[0] for c in DEV_COUNT_SHAPES])
def test_device_counts_equal_the_host_table(name, shape, R):
    # The same rounds through hyf_draft_block (host cu) and hyf_draft_block_dev (padded rows, counts
    # on the device; the unused padding is NaN and must not leak): outputs and states bit for bit.
    pr = Pair(shape, seed=111, pool_slots=R, max_requests=R, max_rows=200)
    dev = hf.DrafterLayer(shape, pr.w, pool_slots=R, max_requests=R, max_rows=200)
    pre = [pr.rows(n) for n in ([40, 9, 1][:R] if R > 1 else [60])]
    cu = np.concatenate([[0], np.cumsum([len(p) for p in pre])]).astype(np.int64)
    for L in (pr.gpu, dev):
        L.reset()
        L.commit(hf.to_device(np.concatenate(pre), shape), cu)
    for rnd, a in enumerate(([3, 8, 0], [0, 1, 5], [8, 2, 7])):
        a = a[:R]
        commits = [pr.rows(n) for n in a]
        blocks = hf.to_device(np.concatenate([pr.rows(8, 3) for _ in range(R)]), shape)
        o_host, o_dev = torch.empty_like(blocks), torch.empty_like(blocks)
        cu_r = np.concatenate([[0], np.cumsum(a)]).astype(np.int64)
        cf = hf.to_device(np.concatenate(commits) if cu_r[-1] else np.zeros((1, shape.d_model), np.float32), shape)
        say("hyf_draft_block host table", name, a)
        pr.gpu.draft(blocks, o_host, cf, cu_r)
        counts = torch.tensor(a, dtype=torch.int32, device=DEV)
        say("hyf_draft_block_dev", name, a)
        hf.check(hf.hyf_draft_block_dev(dev.cfg, dev.w, dev.pool, R, None, R, _padded_commits(shape, commits), counts,
                                        blocks, o_dev, dev.ws, dev.ws_bytes), "hyf_draft_block_dev")
        torch.cuda.synchronize()
        assert torch.equal(o_host, o_dev), f"{name} round {rnd} outputs"
        assert torch.equal(pr.gpu.pool, dev.pool), f"{name} round {rnd} states"



def test_device_counts_equal_the_host_table_over_many_pairs():
    # 64 requests of 4 heads (one workgroup per (request, head)): hyf_draft_block with the host
    # table and hyf_draft_block_dev with padded rows and device counts agree bit for bit.
    shape = small_shape("bf16", window=40)
    R = 64
    pr = Pair(shape, seed=113, pool_slots=R, max_requests=R, max_rows=120 * R)
    dev = hf.DrafterLayer(shape, pr.w, pool_slots=R, max_requests=R, max_rows=120 * R)
    lens = [(29 * i) % 120 for i in range(R)]
    pre = np.concatenate([pr.rows(n) for n in lens])
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    for L in (pr.gpu, dev):
        L.reset()
        L.commit(hf.to_device(pre, shape), cu)
    for rnd in range(3):
        a = [int((7 * i + 3 * rnd) % 9) for i in range(R)]
        commits = [pr.rows(n) for n in a]
        blocks = hf.to_device(np.concatenate([pr.rows(8, 3) for _ in range(R)]), shape)
        o_host, o_dev = torch.empty_like(blocks), torch.empty_like(blocks)
        cu_r = np.concatenate([[0], np.cumsum(a)]).astype(np.int64)
        say("hyf_draft_block host table, 64 requests", rnd)
        pr.gpu.draft(blocks, o_host, hf.to_device(np.concatenate(commits), shape), cu_r)
        counts = torch.tensor(a, dtype=torch.int32, device=DEV)
        say("hyf_draft_block_dev, 64 requests", rnd)
        hf.check(hf.hyf_draft_block_dev(dev.cfg, dev.w, dev.pool, R, None, R, _padded_commits(shape, commits), counts,
                                        blocks, o_dev, dev.ws, dev.ws_bytes), "hyf_draft_block_dev")
        torch.cuda.synchronize()
        assert torch.equal(o_host, o_dev), f"round {rnd} outputs"
        assert torch.equal(pr.gpu.pool, dev.pool), f"round {rnd} states"

def test_device_count_round_replays_in_a_graph():
    # One hyf_draft_block_dev call captured once, replayed for four rounds whose rows and counts are
    # written into its fixed buffers on the device between replays (eager copies, then a sync):
    # every replay equals the eager host-table round on the same rows, outputs and state.
    shape = small_shape("bf16", window=40)
    R = 2
    pr = Pair(shape, seed=112, pool_slots=R, max_requests=R, max_rows=200)
    dev = hf.DrafterLayer(shape, pr.w, pool_slots=R, max_requests=R, max_rows=200)
    pre = hf.to_device(np.concatenate([pr.rows(50), pr.rows(70)]), shape)
    for L in (pr.gpu, dev):
        L.reset()
        L.commit(pre, np.array([0, 50, 120], np.int64))
    torch.cuda.synchronize()
    feats_buf = torch.zeros((R * hf.HYF_BLOCK, shape.d_model), dtype=hf.torch_dtype(shape), device=DEV)
    counts_buf = torch.zeros(R, dtype=torch.int32, device=DEV)
    block_buf = torch.zeros((R * hf.HYF_BLOCK, shape.d_model), dtype=hf.torch_dtype(shape), device=DEV)
    out_buf = torch.empty_like(block_buf)
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    snap = dev.pool.clone()
    say("graph: warm call and capture of hyf_draft_block_dev")
    with torch.cuda.stream(cs):
        hf.check(hf.hyf_draft_block_dev(dev.cfg, dev.w, dev.pool, R, None, R, feats_buf, counts_buf, block_buf,
                                        out_buf, dev.ws, dev.ws_bytes, cs))
    torch.cuda.synchronize()
    dev.pool.copy_(snap)  # the warm call committed zero rows (counts 0) but restore anyway
    with torch.cuda.graph(g, stream=cs):
        hf.check(hf.hyf_draft_block_dev(dev.cfg, dev.w, dev.pool, R, None, R, feats_buf, counts_buf, block_buf,
                                        out_buf, dev.ws, dev.ws_bytes, cs))
    torch.cuda.synchronize()
    for rnd, a in enumerate(([4, 1], [0, 8], [7, 3], [2, 0])):
        commits = [pr.rows(n) for n in a]
        blocks = hf.to_device(np.concatenate([pr.rows(8, 3) for _ in range(R)]), shape)
        feats_buf.copy_(_padded_commits(shape, commits).nan_to_num(0.0))
        counts_buf.copy_(torch.tensor(a, dtype=torch.int32))
        block_buf.copy_(blocks)
        torch.cuda.synchronize()
        say("graph: replay round", rnd, a)
        g.replay()
        torch.cuda.synchronize()
        cu_r = np.concatenate([[0], np.cumsum(a)]).astype(np.int64)
        cf = hf.to_device(np.concatenate(commits) if cu_r[-1] else np.zeros((1, shape.d_model), np.float32), shape)
        o_host = torch.empty_like(blocks)
        pr.gpu.draft(blocks, o_host, cf, cu_r)
        torch.cuda.synchronize()
        assert torch.equal(out_buf, o_host), f"replay {rnd} outputs"
        assert torch.equal(dev.pool, pr.gpu.pool), f"replay {rnd} states"
