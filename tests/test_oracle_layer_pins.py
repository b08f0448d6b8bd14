"""Pins of the oracle's layer wiring: which projection rows feed which operand, how the two
branches meet, and how two layers chain.

The expected values here are built without the oracle's layer helpers: the input projection is
assembled from separately drawn sub-matrices in the documented row order q | C | k | v | B | dt
(gated delta rule: ... | B | alpha | beta), attention is torch's scaled_dot_product_attention
with an explicit mask, the readout is an einsum written out here, and the output projection is
torch's linear.  Sources: HyFlash explainer ("HyFlash lifts on-device speculative decoding
16.2%"), "That is HyFlash": each layer has a local-attention branch over the last committed
features and the draft positions in both directions, and a recurrent branch that holds the
committed history and is only read while drafting; the drafter is a two-layer network.

A swapped k/v, a dropped or sign-flipped memory term, a concatenation in place of the per-head
sum, a wrong w_in row group, or an unrounded first-layer output fails one of these tests.
"""

import math

import numpy as np
import pytest
import torch

from hybrid_ssm_local_amd import inputs as I
from oracle import hyflash_oracle as O


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _lin(x, w):
    return torch.nn.functional.linear(torch.from_numpy(np.asarray(x, np.float64)),
                                      torch.from_numpy(np.asarray(w, np.float64))).numpy()


def _attend(q, keys, vals, mask):
    """torch's attention in float64 on the CPU; mask True = may attend; scale 1/sqrt(head_dim)."""
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(keys), torch.from_numpy(vals),
        attn_mask=torch.from_numpy(mask)).numpy()


def _parts(rng, shape):
    """Separately drawn sub-matrices of w_in (each [rows][d_model]) and w_out."""
    d, dq, gn, nh = shape.d_model, shape.dq, shape.gn, shape.n_heads
    sizes = dict(q=dq, C=gn, k=dq, v=dq, B=gn)
    if shape.memory == "gdn":
        sizes.update(alpha=nh, beta=nh)
    else:
        sizes.update(dt=nh)
    parts = {n: rng.standard_normal((s, d)) / math.sqrt(d) for n, s in sizes.items()}
    order = ("q", "C", "k", "v", "B") + (("alpha", "beta") if shape.memory == "gdn" else ("dt",))
    w_in = np.concatenate([parts[n] for n in order], axis=0)
    w_out = rng.standard_normal((shape.d_model, dq)) / math.sqrt(dq)
    return parts, w_in, w_out


def _hand_state(rng, shape, count):
    """A state built by hand: `count` committed rows of which the ring holds the last min(count, W)
    (row c in slot c mod W), and a random non-zero H.  Returns (state, the window's rows in order)."""
    nh, P, N, W = shape.n_heads, shape.head_dim, shape.d_state, shape.window
    hist_k = O.round_storage(rng.standard_normal((count, nh, P)), shape.dtype)
    hist_v = O.round_storage(rng.standard_normal((count, nh, P)), shape.dtype)
    st = O.new_state(shape)
    st["count"] = count
    for c in range(count):
        st["K"][:, c % W] = hist_k[c]
        st["V"][:, c % W] = hist_v[c]
    st["H"] = rng.standard_normal((nh, P, N))
    lo = max(count - W, 0)
    return st, hist_k[lo:], hist_v[lo:]


def _expected_draft(shape, parts, w_out, d_skip, st, win_k, win_v, x):
    """out = concat_h(attn_h + H_h C_q + D_h v_h) W_out^T, built from the sub-matrices."""
    nh, P, G = shape.n_heads, shape.head_dim, shape.n_groups
    nb = x.shape[0]
    q = _lin(x, parts["q"]).reshape(nb, nh, P)
    k = _lin(x, parts["k"]).reshape(nb, nh, P)
    v = _lin(x, parts["v"]).reshape(nb, nh, P)
    Cq = _lin(x, parts["C"]).reshape(nb, G, -1)
    if shape.memory == "gdn":
        Cq = Cq / np.sqrt(np.sum(Cq * Cq, axis=-1, keepdims=True) + 1e-6)
    n = win_k.shape[0]
    mask = np.ones((nb, n + nb), dtype=bool)
    if not shape.cross_slot:
        mask[:, n:] = np.eye(nb, dtype=bool)
    o = np.zeros((nb, nh, P))
    for h in range(nh):
        g = h // (nh // G)
        att = _attend(q[:, h], np.concatenate([win_k[:, h], k[:, h]]), np.concatenate([win_v[:, h], v[:, h]]), mask)
        mem = np.einsum("pn,jn->jp", st["H"][h], Cq[:, g]) + d_skip[h] * v[:, h]
        o[:, h] = att + mem
    return _lin(o.reshape(nb, nh * P), w_out)


@pytest.mark.parametrize("memory,G,cross,count", [("mamba2", 1, 1, 13), ("mamba2", 2, 1, 5), ("mamba2", 1, 0, 9),
                                                  ("gdn", 1, 1, 11), ("gdn", 2, 0, 3)])
def test_draft_wiring_with_a_nonzero_state(memory, G, cross, count):
    # count above the window (13, 11 > W = 6) exercises the wrapped ring; H and D are random.
    shape = I.LayerShape(d_model=24, n_heads=4, head_dim=8, d_state=6, n_groups=G, window=6, dtype="f32",
                         cross_slot=cross, memory=memory)
    rng = np.random.default_rng(100 + count)
    parts, w_in, w_out = _parts(rng, shape)
    d_skip = rng.standard_normal(shape.n_heads)
    wts = dict(w_in=w_in, w_out=w_out, d_skip=d_skip, a_log=np.zeros(shape.n_heads), dt_bias=np.zeros(shape.n_heads))
    st, wk, wv = _hand_state(rng, shape, count)
    x = rng.standard_normal((8, shape.d_model))
    got = O.draft(shape, wts, st, x)
    ref = _expected_draft(shape, parts, w_out, d_skip, st, wk, wv, x)
    assert _rel(got, ref) < 1e-12


def test_draft_memory_term_enters_with_its_sign_and_the_skip_uses_v():
    # Two drafts that differ only in H differ by exactly concat_h(H_h C_q) W_out^T; two that differ
    # only in D differ by concat_h(dD_h v_h) W_out^T with v the value rows (not the keys).
    shape = I.LayerShape(d_model=16, n_heads=2, head_dim=4, d_state=5, window=4, dtype="f32")
    rng = np.random.default_rng(5)
    parts, w_in, w_out = _parts(rng, shape)
    D = rng.standard_normal(2)
    wts = dict(w_in=w_in, w_out=w_out, d_skip=D, a_log=np.zeros(2), dt_bias=np.zeros(2))
    st, _, _ = _hand_state(rng, shape, 7)
    x = rng.standard_normal((8, 16))
    base = O.draft(shape, wts, st, x)
    st2 = O.copy_state(st)
    dH = rng.standard_normal(st["H"].shape)
    st2["H"] = st["H"] + dH
    Cq = _lin(x, parts["C"])
    diff = np.einsum("hpn,jn->jhp", dH, Cq).reshape(8, -1)
    assert _rel(O.draft(shape, wts, st2, x) - base, _lin(diff, w_out)) < 1e-10
    wts2 = dict(wts, d_skip=D + np.array([1.5, -0.5]))
    v = _lin(x, parts["v"]).reshape(8, 2, 4)
    diff = (np.array([1.5, -0.5])[None, :, None] * v).reshape(8, -1)
    assert _rel(O.draft(shape, wts2, st, x) - base, _lin(diff, w_out)) < 1e-10


def _identity_layer(memory, nh=2, P=3, N=4):
    """A layer whose features are laid out [x | B | step] (Mamba-2) or [x | B | alpha | beta] (gated
    delta rule): w_in's v rows pick x, its B rows pick B and its last rows pick the raw step (gates),
    so the commit's inputs are the raw features themselves.  q, C and k rows are random."""
    dq = nh * P
    ng = 2 if memory == "gdn" else 1
    d = dq + N + ng * nh
    d_pad = (d + 15) // 16 * 16  # the extra feature columns feed nothing
    shape = I.LayerShape(d_model=d_pad, n_heads=nh, head_dim=P, d_state=N, window=5, dtype="f32", memory=memory)
    rng = np.random.default_rng(9)
    eye = np.eye(d_pad)
    w_in = np.concatenate([rng.standard_normal((dq + N, d_pad)),         # q, C
                           rng.standard_normal((dq, d_pad)),             # k
                           eye[:dq],                                     # v  = x
                           eye[dq:dq + N],                               # B
                           eye[dq + N:dq + N + ng * nh]], axis=0)        # step (or alpha, beta)
    assert w_in.shape[0] == shape.n_in
    return shape, w_in, rng


def test_commit_routes_v_b_and_step_rows_closed_form():
    # With identity v / B / step rows, H after a commit has the closed form
    #   H = e^{Lam_n} H0 + sum_t e^{Lam_n - Lam_t} dt_t x_t outer B_t,  Lam = running sum of dt A,
    # written here from the raw features, and the ring holds the k projection and x itself.
    shape, w_in, rng = _identity_layer("mamba2")
    nh, P, N, dq = 2, 3, 4, 6
    a_log, dt_bias = np.array([0.3, 1.2]), np.array([-1.0, 0.5])
    wts = dict(w_in=w_in, w_out=np.zeros((shape.d_model, dq)), a_log=a_log, dt_bias=dt_bias, d_skip=np.zeros(nh))
    H0 = rng.standard_normal((nh, P, N))
    st0 = O.new_state(shape)
    st0["H"] = H0.copy()
    F = rng.standard_normal((7, shape.d_model))
    st, _ = O.commit(shape, wts, st0, F)
    x, B, raw = F[:, :dq].reshape(7, nh, P), F[:, dq:dq + N], F[:, dq + N:dq + N + nh]
    dt = np.log1p(np.exp(raw + dt_bias))
    lam = np.cumsum(dt * -np.exp(a_log), axis=0)
    for h in range(nh):
        ref = math.exp(lam[-1, h]) * H0[h]
        for t in range(7):
            ref = ref + math.exp(lam[-1, h] - lam[t, h]) * dt[t, h] * np.outer(x[t, h], B[t])
        assert _rel(st["H"][h], ref) < 1e-12
    # ring: the last 5 of 7 rows, row c in slot c mod 5; V is x, K the k projection, both rounded
    # to the storage dtype (fp32 here)
    kproj = _lin(F, w_in[dq + N:2 * dq + N]).reshape(7, nh, P)
    for c in range(2, 7):
        np.testing.assert_array_equal(st["V"][:, c % 5], x[c].astype(np.float32))
        np.testing.assert_allclose(st["K"][:, c % 5], kproj[c].astype(np.float32), rtol=1e-7)
    assert st["count"] == 7


def test_gdn_commit_routes_the_gate_rows():
    # Two committed rows from H = 0 through identity rows, unrolled by hand:
    #   H1 = b1 x1 k1^T,  H2 = a2 (H1 - b2 (H1 k2) k2^T) + b2 x2 k2^T,  k = B / sqrt(|B|^2 + 1e-6),
    # a = sigmoid(alpha raw + dt_bias), b = sigmoid(beta raw + a_log) (the gate biases' places).
    shape, w_in, rng = _identity_layer("gdn")
    nh, P, N, dq = 2, 3, 4, 6
    b_alpha, b_beta = np.array([1.0, 3.0]), np.array([-0.5, 0.25])
    wts = dict(w_in=w_in, w_out=np.zeros((shape.d_model, dq)), a_log=b_beta, dt_bias=b_alpha, d_skip=np.zeros(nh))
    F = rng.standard_normal((2, shape.d_model))
    st, _ = O.commit(shape, wts, O.new_state(shape), F)
    sig = lambda z: 1.0 / (1.0 + math.exp(-z))
    for h in range(nh):
        xs = [F[t, h * P:(h + 1) * P] for t in range(2)]
        ks = [F[t, dq:dq + N] / math.sqrt(F[t, dq:dq + N] @ F[t, dq:dq + N] + 1e-6) for t in range(2)]
        a = [sig(F[t, dq + N + h] + b_alpha[h]) for t in range(2)]
        b = [sig(F[t, dq + N + nh + h] + b_beta[h]) for t in range(2)]
        H1 = b[0] * np.outer(xs[0], ks[0])
        H2 = a[1] * (H1 - b[1] * np.outer(H1 @ ks[1], ks[1])) + b[1] * np.outer(xs[1], ks[1])
        assert _rel(st["H"][h], H2) < 1e-12


def test_two_layers_chain_through_the_rounded_residual():
    # Layer 2 drafts from block_in + round_bf16(layer 1's output); the rounding is done here with
    # torch's bfloat16 cast, and each layer's output with the hand-built expectation above.
    shape = I.LayerShape(d_model=16, n_heads=2, head_dim=8, d_state=4, window=4, dtype="bf16")
    rng = np.random.default_rng(21)
    layers = []
    for _ in range(2):
        parts, w_in, w_out = _parts(rng, shape)
        d_skip = rng.standard_normal(2)
        st, wk, wv = _hand_state(rng, shape, 6)
        wts = dict(w_in=w_in, w_out=w_out, d_skip=d_skip, a_log=np.zeros(2), dt_bias=np.zeros(2))
        layers.append((parts, wts, st, wk, wv))
    x = O.round_storage(rng.standard_normal((8, 16)), "bf16")
    o1, o2 = O.draft_two_layer(shape, layers[0][1], layers[1][1], layers[0][2], layers[1][2], x)
    p1, w1, s1, k1, v1 = layers[0]
    ref1 = _expected_draft(shape, p1, w1["w_out"], w1["d_skip"], s1, k1, v1, x)
    x2 = x + torch.from_numpy(ref1).to(torch.bfloat16).to(torch.float64).numpy()
    p2, w2, s2, k2, v2 = layers[1]
    ref2 = _expected_draft(shape, p2, w2["w_out"], w2["d_skip"], s2, k2, v2, x2)
    assert _rel(o1, ref1) < 1e-12
    assert _rel(o2, ref2) < 1e-12
    # the rounding matters at this tolerance: without it layer 2 differs measurably
    ref2_unrounded = _expected_draft(shape, p2, w2["w_out"], w2["d_skip"], s2, k2, v2, x + ref1)
    assert _rel(ref2_unrounded, ref2) > 1e-6


def test_four_bit_layer_equals_the_layer_of_its_dequantized_weights():
    # A layer whose w_in and w_out are 4-bit codes computes exactly what the same layer computes
    # with the dense weights the codes stand for (dequantize_w4, pinned on its own): commit and
    # draft, state and output.
    shape = I.LayerShape(d_model=256, n_heads=2, head_dim=128, d_state=16, window=6, dtype="bf16")
    rng = np.random.default_rng(31)
    parts, w_in, w_out = _parts(rng, shape)
    qi, si = O.quantize_w4(w_in)
    qo, so = O.quantize_w4(w_out)
    base = dict(a_log=rng.uniform(0, 2, 2), dt_bias=np.full(2, -1.0), d_skip=rng.standard_normal(2))
    w4 = dict(base, w_in_q=qi, w_in_s=si, w_out_q=qo, w_out_s=so)
    dense = dict(base, w_in=O.dequantize_w4(qi, si), w_out=O.dequantize_w4(qo, so))
    F = rng.standard_normal((9, 256)) / 16
    x = rng.standard_normal((8, 256)) / 16
    st4, _ = O.commit(shape, w4, O.new_state(shape), F)
    std, _ = O.commit(shape, dense, O.new_state(shape), F)
    assert np.array_equal(st4["H"], std["H"]) and np.array_equal(st4["K"], std["K"])
    assert np.array_equal(O.draft(shape, w4, st4, x), O.draft(shape, dense, std, x))
    # and the 4-bit layer is not the layer of the unquantized weights (the rounding is there)
    undq = dict(base, w_in=w_in, w_out=w_out)
    assert _rel(O.draft(shape, w4, st4, x), O.draft(shape, undq, O.commit(shape, undq, O.new_state(shape), F)[0], x)) > 1e-4


@pytest.mark.parametrize("total", [5, 6, 17])
def test_last_w_memory_is_the_scan_of_the_last_w_committed_rows(total):
    # The last-W memory (the paper's "SSM: last 512" ablation) after `total` committed rows over a
    # window of 6: its state equals the closed form of a scan from zero over exactly the last
    # min(total, 6) rows in commit order, written here from the rows' own x = v, B and step
    # projections (the sub-matrices) rounded as the ring stores them; every commit leaves that
    # state in H, and the draft reads it with H . C_q + D v.
    shape = I.LayerShape(d_model=24, n_heads=2, head_dim=4, d_state=3, window=6, dtype="bf16", memory="lastw")
    rng = np.random.default_rng(60 + total)
    parts, w_in, w_out = _parts(rng, shape)
    a_log, dt_bias, D = rng.uniform(0, 1.5, 2), np.array([-1.0, 0.5]), rng.standard_normal(2)
    wts = dict(w_in=w_in, w_out=w_out, a_log=a_log, dt_bias=dt_bias, d_skip=D)
    F = rng.standard_normal((total, 24)) / 4
    st, done = O.new_state(shape), 0
    while done < total:
        a = min(int(rng.integers(1, 5)), total - done)
        st, _ = O.commit(shape, wts, st, F[done:done + a])
        done += a
    assert st["count"] == total
    bf = lambda z: torch.from_numpy(np.asarray(z, np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    last = F[max(total - 6, 0):]
    x = bf(_lin(last, parts["v"])).reshape(len(last), 2, 4)
    B = bf(_lin(last, parts["B"]))
    raw = _lin(last, parts["dt"]).astype(np.float32).astype(np.float64)
    dt = np.log1p(np.exp(raw + dt_bias))
    ell = dt * -np.exp(a_log)
    H = np.zeros((2, 4, 3))
    for h in range(2):
        for t in range(len(last)):
            H[h] += math.exp(ell[t + 1:, h].sum()) * dt[t, h] * np.outer(x[t, h], B[t])
    assert _rel(O.lastw_state(shape, wts, st), H) < 1e-12
    assert _rel(st["H"], H) < 1e-12
    # the draft reads that state
    xb = rng.standard_normal((8, 24)) / 4
    ref_st = dict(st, H=H)
    hist = bf(_lin(F, parts["k"])).reshape(total, 2, 4), bf(_lin(F, parts["v"])).reshape(total, 2, 4)
    lo = max(total - 6, 0)
    ref = _expected_draft(shape, parts, w_out, D, ref_st, hist[0][lo:], hist[1][lo:], xb)
    assert _rel(O.draft(shape, wts, st, xb), ref) < 1e-12


# ---------------------------------------------------------------------------------------------
# The full drafter block (pre-norm residual block around the layer, then a SwiGLU MLP).  The
# expected values use torch's rms_norm and silu and the hand-built layer expectation above.


def _t(a):
    return torch.from_numpy(np.asarray(a, np.float64))


def _rms(x, g, eps):
    return torch.nn.functional.rms_norm(_t(x), (x.shape[-1],), weight=_t(g), eps=eps).numpy()


def _swiglu(z, wg, wu, wd):
    z = _t(z)
    a = torch.nn.functional.silu(z @ _t(wg).T) * (z @ _t(wu).T)
    return (a @ _t(wd).T).numpy()


def test_rms_norm_and_silu_against_worked_values_and_torch():
    # [3, 4]: mean square 12.5, so the row becomes [3, 4] / sqrt(12.5)
    got = O.rms_norm(np.array([[3.0, 4.0]]), np.ones(2), 0.0)
    assert np.allclose(got, [[3 / math.sqrt(12.5), 4 / math.sqrt(12.5)]], rtol=0, atol=1e-15)
    rng = np.random.default_rng(3)
    x, g = rng.standard_normal((5, 32)), rng.standard_normal(32)
    assert _rel(O.rms_norm(x, g, 1e-6), _rms(x, g, 1e-6)) < 1e-13
    # scale invariance with eps = 0, and unit root mean square with g = 1
    assert _rel(O.rms_norm(7.5 * x, g, 0.0), O.rms_norm(x, g, 0.0)) < 1e-13
    assert np.allclose(np.sqrt(np.mean(O.rms_norm(x, np.ones(32), 0.0) ** 2, axis=1)), 1.0, atol=1e-13)
    z = rng.standard_normal(50) * 6
    assert _rel(O.silu(z), torch.nn.functional.silu(_t(z)).numpy()) < 1e-13
    assert O.silu(np.array([0.0]))[0] == 0.0


def test_swiglu_mlp_against_torch():
    rng = np.random.default_rng(4)
    z = rng.standard_normal((6, 24))
    wg, wu, wd = rng.standard_normal((40, 24)), rng.standard_normal((40, 24)), rng.standard_normal((24, 40))
    assert _rel(O.swiglu_mlp(z, wg, wu, wd), _swiglu(z, wg, wu, wd)) < 1e-12
    # the gate is the one under silu: swapping gate and up changes the result
    assert _rel(O.swiglu_mlp(z, wu, wg, wd), _swiglu(z, wg, wu, wd)) > 1e-3


def _block_case(seed, memory="mamba2"):
    shape = I.LayerShape(d_model=24, n_heads=4, head_dim=8, d_state=6, window=6, dtype="f32", memory=memory)
    rng = np.random.default_rng(seed)
    parts, w_in, w_out = _parts(rng, shape)
    d_skip = rng.standard_normal(shape.n_heads)
    wts = dict(w_in=w_in, w_out=w_out, d_skip=d_skip, a_log=np.zeros(shape.n_heads),
               dt_bias=np.zeros(shape.n_heads))
    F = 40
    bw = dict(norm1=1 + 0.3 * rng.standard_normal(24), norm2=1 + 0.3 * rng.standard_normal(24),
              w_gate=rng.standard_normal((F, 24)) / 5, w_up=rng.standard_normal((F, 24)) / 5,
              w_down=rng.standard_normal((24, F)) / 6, eps=1e-5)
    st, wk, wv = _hand_state(rng, shape, 9)
    return shape, parts, wts, bw, st, wk, wv, rng


@pytest.mark.parametrize("memory", ["mamba2", "gdn"])
def test_block_draft_wiring(memory):
    # out = h + MLP(rms(h) g2) with h = x + Layer(rms(x) g1): the layer from the hand-built
    # expectation, the norms and the MLP from torch.  A missing residual, the second norm taken of
    # x instead of h, or the norms' weights swapped fails.
    shape, parts, wts, bw, st, wk, wv, rng = _block_case(31, memory)
    x = 3.0 * rng.standard_normal((8, 24))
    h = x + _expected_draft(shape, parts, wts["w_out"], wts["d_skip"], st, wk, wv, _rms(x, bw["norm1"], bw["eps"]))
    ref = h + _swiglu(_rms(h, bw["norm2"], bw["eps"]), bw["w_gate"], bw["w_up"], bw["w_down"])
    got = O.block_draft(shape, wts, bw, st, x)
    assert _rel(got, ref) < 1e-12
    wrong = [h + _swiglu(_rms(x, bw["norm2"], bw["eps"]), bw["w_gate"], bw["w_up"], bw["w_down"]),
             x + _swiglu(_rms(h, bw["norm2"], bw["eps"]), bw["w_gate"], bw["w_up"], bw["w_down"]),
             h + _swiglu(_rms(h, bw["norm1"], bw["eps"]), bw["w_gate"], bw["w_up"], bw["w_down"])]
    for w in wrong:
        assert _rel(w, ref) > 1e-4


def test_block_with_zero_output_weights_is_the_identity():
    # With the layer's w_out and the MLP's w_down zero, both residual branches vanish.
    shape, parts, wts, bw, st, _, _, rng = _block_case(32)
    x = rng.standard_normal((8, 24))
    out = O.block_draft(shape, dict(wts, w_out=np.zeros_like(wts["w_out"])), dict(bw, w_down=np.zeros((24, 40))), st, x)
    assert np.array_equal(out, x)


def test_block_commit_folds_the_normalized_features():
    # The memory commits rms(feats) g1: with identity v / B / step rows of w_in (the closed-form
    # layer above), H after the block's commit equals H after a plain commit of torch's normalized
    # rows.
    shape, w_in, rng = _identity_layer("mamba2")
    d = shape.d_model
    wts = dict(w_in=w_in, w_out=rng.standard_normal((d, shape.dq)), d_skip=np.zeros(2), a_log=np.zeros(2),
               dt_bias=np.zeros(2))
    bw = dict(norm1=1 + 0.2 * rng.standard_normal(d), norm2=np.ones(d), w_gate=np.zeros((8, d)),
              w_up=np.zeros((8, d)), w_down=np.zeros((d, 8)), eps=1e-6)
    feats = 2.0 * rng.standard_normal((7, d))
    st_b, _ = O.block_commit(shape, wts, bw, O.new_state(shape), feats)
    st_p, _ = O.commit(shape, wts, O.new_state(shape), _rms(feats, bw["norm1"], bw["eps"]))
    assert _rel(st_b["H"], st_p["H"]) < 1e-12 and _rel(st_b["V"], st_p["V"]) < 1e-12
    st_raw, _ = O.commit(shape, wts, O.new_state(shape), feats)
    assert _rel(st_b["H"], st_raw["H"]) > 1e-3
