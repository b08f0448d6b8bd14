"""CPU oracle for the HyFlash drafter-layer hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or run
this module: only the tests, the smoke check of the package entry file and the
CPU-baseline leg of the benchmark do.  It shares no code with the HIP library.

Plain NumPy in float64, written for a reader to check against the HyFlash
pages by eye, not for speed.  Sources (page title, then section):

* HyFlash paper page, Abstract: local attention over recent context and the
  draft positions; a recurrent memory that compresses the committed history of
  target features into a fixed-size state.
* HyFlash explainer, "That is HyFlash": every layer has a local-attention
  branch (last committed features plus all seven draft positions, in both
  directions) and a Mamba-2 branch that holds the committed history, is only
  read while drafting, and is updated after verification by the newly
  committed features alone.
* HyFlash explainer, "Jargon": Mamba-2 folds each input into a fixed-size
  state with an input-dependent step size and a learned decay; a block is
  seven draft positions.
* HyFlash explainer, FAQ "Why does the memory update only from committed
  features?": drafting reads the state and never writes it.
* HyFlash explainer, "Where it earns its keep": the recurrent state is fp32.

The pages print no formulas.  Readings taken here (each listed in the design
notes of the repository):

* Recurrence: the plain Mamba-2 / SSD form with one scalar decay per head,
      h_t = exp(dt_t * A) * h_{t-1} + dt_t * (x_t outer B_t),   y_t = h_t . C_t + D * x_t,
  dt_t = softplus(raw_t + dt_bias), A = -exp(A_log); y uses the state after
  token t.  The SSM input x is the value projection v.  B and C are shared by
  the heads of a group (one group by default).
* Attention: scale 1/sqrt(head_dim), no positional encoding, no causal mask
  inside the block (all block rows, anchor included, are queries and keys);
  keys are the last min(count, window) committed rows plus the block rows.
* The two branches are summed per head, then one output projection.
* Ring slot of committed row c (0-based over the request's life) is c mod W.
* Stored values (ring K/V) are rounded to the storage dtype; everything else
  stays float64.
* 4-bit weights (the pages name GPTQ, no format): group-wise symmetric
  round-to-nearest, 128 k per group, scale max|w|/7 in float32, two codes per
  byte (lower k in the low nibble); see quantize_w4.  A layer with 4-bit weights
  projects through the dequantized weights (layer_projection).

* The full drafter block (explainer, "That is HyFlash": every layer of the
  drafter holds the two branches; "Where it earns its keep": a drafter
  backbone of a few milliseconds; the pages give no backbone beyond that):
  the plainest pre-norm residual block around the two-branch layer,
      h = x + Layer(RMSNorm(x) * g1),   out = h + MLP(RMSNorm(h) * g2),
  RMSNorm(x) = x / sqrt(mean(x^2) + eps), MLP(z) = (silu(z Wg^T) * (z Wu^T)) Wd^T
  (SwiGLU); the memory commits RMSNorm(feats) * g1, the layer's own input.

Parity is pinned for every function below by tests that compare against
closed forms, library routines or brute force (see tests/test_oracle_pins.py
and tests/test_oracle_layer_pins.py).
"""

from __future__ import annotations

import numpy as np

F64 = np.float64


# ----------------------------------------------------------------------------
# small helpers


def softplus(z):
    """log(1 + e^z), evaluated without overflow (NumPy's logaddexp with 0)."""
    return np.logaddexp(0.0, np.asarray(z, dtype=F64))


def round_storage(a, dtype: str) -> np.ndarray:
    """Round float64 values to the storage dtype (nearest even), returned as float64.

    bf16 rounding goes through float32 first; torch's CPU cast does the
    float32 -> bfloat16 step.
    """
    a32 = np.asarray(a, dtype=F64).astype(np.float32)
    if dtype == "f32":
        return a32.astype(F64)
    import torch

    return torch.from_numpy(np.ascontiguousarray(a32)).to(torch.bfloat16).to(torch.float64).numpy()


def head_groups(n_heads: int, n_groups: int) -> np.ndarray:
    """Group index of each head (B and C are shared by the heads of a group)."""
    assert n_heads % n_groups == 0
    return np.arange(n_heads) // (n_heads // n_groups)


def per_head(bc, n_heads: int, n_groups: int) -> np.ndarray:
    """[T][G*N] -> [T][nh][N]: each head sees its group's B (or C) row."""
    T, GN = bc.shape
    N = GN // n_groups
    return np.asarray(bc, dtype=F64).reshape(T, n_groups, N)[:, head_groups(n_heads, n_groups), :]


def step_and_decay(dt_raw, dt_bias, a_log):
    """Input-dependent step dt = softplus(raw + bias) and log-decay ell = dt * A, A = -exp(A_log).

    HyFlash explainer, "Jargon", Mamba-2 entry (input-dependent step size, learned decay).
    Returns (dt, ell), each [T][nh] float64.
    """
    dt = softplus(np.asarray(dt_raw, F64) + np.asarray(dt_bias, F64)[None, :])
    A = -np.exp(np.asarray(a_log, F64))
    return dt, dt * A[None, :]


# ----------------------------------------------------------------------------
# the recurrent memory (Mamba-2 / SSD) on pre-projected inputs


def ssd_sequential(x, B, C, dt_raw, a_log, dt_bias, d_skip, H0, n_groups: int = 1):
    """The definition: one token at a time.

    x [T][nh][P], B and C [T][G*N] (C may be None), dt_raw [T][nh], H0 [nh][P][N].
    Returns (H_T [nh][P][N], y [T][nh][P] or None), float64.
    """
    x = np.asarray(x, F64)
    T, nh, P = x.shape
    Bh = per_head(B, nh, n_groups)
    Ch = per_head(C, nh, n_groups) if C is not None else None
    dt, ell = step_and_decay(dt_raw, dt_bias, a_log)
    D = np.asarray(d_skip, F64)
    H = np.array(H0, dtype=F64, copy=True)
    y = np.zeros((T, nh, P), F64) if Ch is not None else None
    for t in range(T):
        decay = np.exp(ell[t])                                   # [nh]
        write = (dt[t][:, None] * x[t])[:, :, None] * Bh[t][:, None, :]   # [nh][P][N]
        H = decay[:, None, None] * H + write
        if y is not None:
            y[t] = np.einsum("hpn,hn->hp", H, Ch[t]) + D[:, None] * x[t]
    return H, y


def ssd_chunked(x, B, C, dt_raw, a_log, dt_bias, d_skip, H0, chunk: int, n_groups: int = 1):
    """The chunked SSD algorithm; equal to ssd_sequential up to rounding.

    Per chunk of `chunk` tokens:
      1. Lam = inclusive cumulative sum of ell inside the chunk;
      2. chunk state S = sum_tau exp(Lam_end - Lam_tau) * dt_tau * x_tau outer B_tau;
      3. outputs (if C): intra-chunk quadratic form
            y_t = sum_{tau <= t} (C_t . B_tau) * exp(Lam_t - Lam_tau) * dt_tau * x_tau
         plus the carried state exp(Lam_t) * (H_prev . C_t), plus D * x_t;
      4. state pass H = exp(Lam_end) * H_prev + S.
    Exponents are always differences of log-decays (never ratios of exps).
    """
    x = np.asarray(x, F64)
    T, nh, P = x.shape
    Bh = per_head(B, nh, n_groups)
    Ch = per_head(C, nh, n_groups) if C is not None else None
    dt, ell = step_and_decay(dt_raw, dt_bias, a_log)
    D = np.asarray(d_skip, F64)
    H = np.array(H0, dtype=F64, copy=True)
    y = np.zeros((T, nh, P), F64) if Ch is not None else None
    for c0 in range(0, T, chunk):
        s = slice(c0, min(c0 + chunk, T))
        Lam = np.cumsum(ell[s], axis=0)                          # [Lc][nh]
        w_end = np.exp(Lam[-1][None, :] - Lam) * dt[s]           # [Lc][nh]
        S = np.einsum("th,thp,thn->hpn", w_end, x[s], Bh[s])
        if y is not None:
            Lc = Lam.shape[0]
            causal = np.tril(np.ones((Lc, Lc), dtype=bool))      # [t][tau], tau <= t
            diff = np.where(causal[:, :, None], Lam[:, None, :] - Lam[None, :, :], -np.inf)
            M = np.exp(diff) * dt[s][None, :, :]                 # [t][tau][nh]
            CB = np.einsum("thn,shn->tsh", Ch[s], Bh[s])          # [t][tau][nh]
            y_intra = np.einsum("tsh,shp->thp", CB * M, x[s])
            y_carry = np.exp(Lam)[:, :, None] * np.einsum("hpn,thn->thp", H, Ch[s])
            y[s] = y_intra + y_carry + D[None, :, None] * x[s]
        H = np.exp(Lam[-1])[:, None, None] * H + S
    return H, y


# ----------------------------------------------------------------------------
# the gated delta-rule memory (the memory the pages swap in for Mamba-2)


def sigmoid(z):
    """1 / (1 + e^-z), evaluated as e^z / (1 + e^z) for z < 0 so that neither branch overflows and
    small values keep their relative precision."""
    z = np.asarray(z, dtype=F64)
    e = np.exp(-np.abs(z))
    return np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def l2_normalize(a, eps: float = 1e-6):
    """a / sqrt(|a|^2 + eps) along the last axis."""
    a = np.asarray(a, dtype=F64)
    return a / np.sqrt(np.sum(a * a, axis=-1, keepdims=True) + eps)


def gdn_sequential(x, B, alpha_raw, beta_raw, b_alpha, b_beta, H0, n_groups: int = 1):
    """The gated delta rule, one token at a time.

    HyFlash explainer, "That is HyFlash" and FAQ (a fixed-size memory of the committed history);
    HyFlash paper, the memory ablation (Gated DeltaNet-2 in place of Mamba-2).  Per head, with the
    key k = B_t normalized to unit length, the value x_t (the value projection), the retention gate
    a = sigmoid(alpha_raw + b_alpha) and the write gate b = sigmoid(beta_raw + b_beta):
        H <- a * H (I - b k k^T) + b * x_t k^T        (H is [P][N]: value rows, key columns)
    x [T][nh][P], B [T][G*N], alpha_raw and beta_raw [T][nh], H0 [nh][P][N].  Returns H_T.
    """
    x = np.asarray(x, F64)
    T, nh, P = x.shape
    k = l2_normalize(per_head(B, nh, n_groups))                  # [T][nh][N]
    a = sigmoid(np.asarray(alpha_raw, F64) + np.asarray(b_alpha, F64)[None, :])
    b = sigmoid(np.asarray(beta_raw, F64) + np.asarray(b_beta, F64)[None, :])
    H = np.array(H0, dtype=F64, copy=True)
    for t in range(T):
        Hk = np.einsum("hpn,hn->hp", H, k[t])                    # H k
        H = a[t][:, None, None] * (H - b[t][:, None, None] * Hk[:, :, None] * k[t][:, None, :]) \
            + b[t][:, None, None] * x[t][:, :, None] * k[t][:, None, :]
    return H


def gdn_chunked(x, B, alpha_raw, beta_raw, b_alpha, b_beta, H0, chunk: int, n_groups: int = 1):
    """The gated delta rule over chunks of `chunk` tokens: the same H_T as gdn_sequential.

    The pages print only the rule's name; this chunked form is derived from the rule above.  Within a
    chunk (H0 the state before it, g = log a, G its running sum, gamma = exp(G)) the rule unrolls to
        H_t = gamma_t H0 + sum_{s <= t} exp(G_t - G_s) u_s k_s^T,
        u_t = b_t (x_t - gamma_t H0 k_t - sum_{s < t} exp(G_t - G_s) (k_s . k_t) u_s),
    so with A the strictly lower part of b_t exp(G_t - G_s) (k_t . k_s), U = X - Y H0^T where
    (I + A) X = diag(b) V and (I + A) Y = diag(b gamma) K, and the chunk ends at
        H = gamma_last H0 + (X - Y H0^T)^T diag(exp(G_last - G_s)) K.
    """
    x = np.asarray(x, F64)
    T, nh, P = x.shape
    k = l2_normalize(per_head(B, nh, n_groups))                  # [T][nh][N]
    a = sigmoid(np.asarray(alpha_raw, F64) + np.asarray(b_alpha, F64)[None, :])
    b = sigmoid(np.asarray(beta_raw, F64) + np.asarray(b_beta, F64)[None, :])
    H = np.array(H0, dtype=F64, copy=True)
    for c0 in range(0, T, chunk):
        c1 = min(c0 + chunk, T)
        L = c1 - c0
        for h in range(nh):
            K = k[c0:c1, h]                                      # [L][N]
            V = x[c0:c1, h]                                      # [L][P]
            bb = b[c0:c1, h]
            G = np.cumsum(np.log(a[c0:c1, h]))
            decay = np.exp(np.minimum(G[:, None] - G[None, :], 0.0))
            A = np.tril(bb[:, None] * decay * (K @ K.T), -1)
            M = np.eye(L) + A
            X = np.linalg.solve(M, bb[:, None] * V)
            Y = np.linalg.solve(M, (bb * np.exp(G))[:, None] * K)
            Kd = np.exp(G[-1] - G)[:, None] * K
            H[h] = np.exp(G[-1]) * H[h] + (X - Y @ H[h].T).T @ Kd
    return H


# ----------------------------------------------------------------------------
# the layer: projections, ring, attention, readout, output projection


def split_projection(proj, shape):
    """Columns of [rows][n_in] in storage order q | C | k | v | B | dt -> dict of views."""
    n = proj.shape[0]
    out = {}
    for name, (a, b) in shape.in_groups.items():
        out[name] = proj[:, a:b]
    nh, P = shape.n_heads, shape.head_dim
    for name in ("q", "k", "v"):
        out[name] = out[name].reshape(n, nh, P)
    return out


def project(rows, w):
    """rows [n][in] times an nn.Linear weight [out][in] -> [n][out], float64."""
    return np.asarray(rows, F64) @ np.asarray(w, F64).T


def layer_projection(rows, wts: dict, which: str):
    """The layer's input ("in") or output ("out") projection: with 4-bit weights (the dict holds
    w_<which>_q codes and w_<which>_s scales) the product of the dequantized weights (linear_w4),
    else the dense weight w_<which>."""
    if f"w_{which}_q" in wts:
        return linear_w4(rows, wts[f"w_{which}_q"], wts[f"w_{which}_s"])
    return project(rows, wts[f"w_{which}"])


def new_state(shape) -> dict:
    """Empty per-request state: nothing committed, H = 0, empty ring.  The last-W memory also keeps,
    per ring slot, the row's B (storage dtype) and raw step (fp32)."""
    nh, P, N, W = shape.n_heads, shape.head_dim, shape.d_state, shape.window
    st = dict(count=0, H=np.zeros((nh, P, N), F64),
              K=np.zeros((nh, W, P), F64), V=np.zeros((nh, W, P), F64))
    if shape.memory == "lastw":
        st["Bring"] = np.zeros((W, shape.gn), F64)
        st["DTring"] = np.zeros((W, nh), F64)
    return st


def copy_state(st: dict) -> dict:
    return {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in st.items()}


def ring_append(shape, st: dict, k, v, B=None, dt_raw=None) -> None:
    """Committed row c (0-based over the request) goes to slot c mod W; values stored rounded (k, v
    and B to the storage dtype, the raw step to fp32)."""
    W = shape.window
    kr = round_storage(k, shape.dtype)
    vr = round_storage(v, shape.dtype)
    br = round_storage(B, shape.dtype) if B is not None else None
    dr = round_storage(dt_raw, "f32") if dt_raw is not None else None
    for i in range(kr.shape[0]):
        slot = st["count"] % W
        st["K"][:, slot, :] = kr[i]
        st["V"][:, slot, :] = vr[i]
        if br is not None:
            st["Bring"][slot] = br[i]
            st["DTring"][slot] = dr[i]
        st["count"] += 1


def window_in_order(shape, st: dict):
    """Ring slots of the last min(count, W) committed rows, oldest first."""
    n = min(st["count"], shape.window)
    return (st["count"] - n + np.arange(n)) % shape.window


def lastw_state(shape, wts: dict, st: dict):
    """The memory of the paper's last-W ablation ("SSM: last 512"): the Mamba-2 state of a scan
    from H = 0 over only the last min(count, W) committed rows, in commit order, from the stored
    (rounded) x = v, B and raw steps of the ring."""
    slots = window_in_order(shape, st)
    x = st["V"][:, slots, :].transpose(1, 0, 2)
    H0 = np.zeros((shape.n_heads, shape.head_dim, shape.d_state), F64)
    H, _ = ssd_sequential(x, st["Bring"][slots], None, st["DTring"][slots], wts["a_log"], wts["dt_bias"],
                          wts["d_skip"], H0, shape.n_groups)
    return H


def ring_window(shape, st: dict):
    """Keys/values of the last min(count, W) committed rows, as [n][nh][P] (order irrelevant)."""
    n = min(st["count"], shape.window)
    if n == st["count"]:
        slots = np.arange(n)
    else:
        slots = (st["count"] - n + np.arange(n)) % shape.window
    return st["K"][:, slots, :].transpose(1, 0, 2), st["V"][:, slots, :].transpose(1, 0, 2)


def commit(shape, wts: dict, st: dict, feats, want_y: bool = False):
    """Fold newly committed feature rows into the memory and the window (the only writer).

    Returns (new state, y or None).  The input state is not modified.
    """
    st = copy_state(st)
    feats = np.asarray(feats, F64)
    if feats.shape[0] == 0:
        return st, (np.zeros((0, shape.n_heads, shape.head_dim)) if want_y else None)
    pr = split_projection(layer_projection(feats, wts, "in"), shape)
    if shape.memory == "lastw":
        # the last-W memory: after the rows enter the ring, the state is the scan of the window
        if want_y:
            raise ValueError("per-token outputs are defined for the Mamba-2 memory only")
        ring_append(shape, st, pr["k"], pr["v"], pr["B"], pr["dt"])
        st["H"] = lastw_state(shape, wts, st)
        return st, None
    if shape.memory == "gdn":
        if want_y:
            raise ValueError("per-token outputs are defined for the Mamba-2 memory only")
        H, y = gdn_sequential(pr["v"], pr["B"], pr["alpha"], pr["beta"], wts["dt_bias"], wts["a_log"], st["H"],
                              shape.n_groups), None
    else:
        H, y = ssd_sequential(pr["v"], pr["B"], pr["C"] if want_y else None, pr["dt"],
                              wts["a_log"], wts["dt_bias"], wts["d_skip"], st["H"], shape.n_groups)
    st["H"] = H
    ring_append(shape, st, pr["k"], pr["v"])
    return st, y


def block_attention(q, k_ctx, v_ctx, k_blk, v_blk, cross_slot: int = 1):
    """Softmax attention of the block rows over (context rows + block rows), per head.

    q, k_blk, v_blk [nb][nh][P]; k_ctx, v_ctx [n][nh][P].  No causal mask; with
    cross_slot = 0 block row j sees only itself among the block keys.
    """
    q = np.asarray(q, F64)
    nb, nh, P = q.shape
    out = np.zeros((nb, nh, P), F64)
    for h in range(nh):
        keys = np.concatenate([np.asarray(k_ctx, F64)[:, h], np.asarray(k_blk, F64)[:, h]], axis=0)
        vals = np.concatenate([np.asarray(v_ctx, F64)[:, h], np.asarray(v_blk, F64)[:, h]], axis=0)
        s = q[:, h] @ keys.T / np.sqrt(P)                       # [nb][n + nb]
        if not cross_slot:
            n = k_ctx.shape[0]
            off = ~np.eye(nb, dtype=bool)
            s[:, n:][off] = -np.inf
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h] = p @ vals
    return out


def memory_readout(H, Cq, v, d_skip, n_groups: int = 1):
    """mem_j,h = H_h . C_q,j + D_h * v_j,h; H is only read."""
    nb, nh, P = v.shape
    Ch = per_head(Cq, nh, n_groups)
    return np.einsum("hpn,jhn->jhp", np.asarray(H, F64), Ch) + np.asarray(d_skip, F64)[None, :, None] * v


def draft(shape, wts: dict, st: dict, block_in):
    """One draft step over the block rows (anchor + draft slots).  Reads the state, never writes it.

    Returns out [nb][d_model] float64.
    """
    x = np.asarray(block_in, F64)
    nb = x.shape[0]
    pr = split_projection(layer_projection(x, wts, "in"), shape)
    k_ctx, v_ctx = ring_window(shape, st)
    attn = block_attention(pr["q"], k_ctx, v_ctx, pr["k"], pr["v"], shape.cross_slot)
    Cq = l2_normalize(pr["C"].reshape(nb, shape.n_groups, -1)).reshape(nb, -1) if shape.memory == "gdn" else pr["C"]
    mem = memory_readout(st["H"], Cq, pr["v"], wts["d_skip"], shape.n_groups)
    o = (attn + mem).reshape(nb, shape.dq)
    return layer_projection(o, wts, "out")


def round_step(shape, wts: dict, st: dict, commit_feats, block_in):
    """One verification round: commit the accepted rows first, then draft the next block."""
    st2, _ = commit(shape, wts, st, commit_feats)
    return st2, draft(shape, wts, st2, block_in)


def draft_two_layer(shape, wts1: dict, wts2: dict, st1: dict, st2: dict, block_in):
    """Two chained layers: the second layer's block input is block_in plus the first layer's output."""
    o1 = draft(shape, wts1, st1, block_in)
    x2 = np.asarray(block_in, F64) + round_storage(o1, shape.dtype)
    return o1, draft(shape, wts2, st2, x2)


# ---------------------------------------------------------------------------------------------
# Weight-only 4-bit projections (paper page, Figures & tables: the BF16 vs INT4 speedup table;
# explainer, "Where it earns its keep": the drafter's weights quantized to 4 bits).  The pages
# name GPTQ but give no format; the reading taken here is group-wise symmetric round-to-nearest
# (calibration needs data, so none is done):
#   groups of W4_GROUP consecutive k of one output row f share a scale s = max|w| / 7;
#   q = round(w / s) (half away from zero), in -7 .. 7 (0 where s = 0); the dequantized weight is
#   q * s;  stored as the nibble q + 8, two per byte along k, the lower k in the low nibble.
# ---------------------------------------------------------------------------------------------
W4_GROUP = 128


def quantize_w4(W, group: int = W4_GROUP):
    """Round-to-nearest 4-bit codes of W [Nout][K] (K a multiple of group): returns
    (packed uint8 [Nout][K/2], scales float32 [Nout][K/group]).  The scales are rounded to
    float32 first, and the codes are taken against the rounded scale, so that codes and
    scales describe the dequantized weight exactly."""
    W = np.asarray(W, dtype=np.float64)
    n_out, K = W.shape
    assert K % group == 0
    Wg = W.reshape(n_out, K // group, group)
    s = (np.abs(Wg).max(axis=2) / 7.0).astype(np.float32)
    s64 = s.astype(np.float64)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(s64 > 0, Wg / np.where(s64 > 0, s64, 1.0), 0.0)
    q = np.sign(r) * np.floor(np.abs(r) + 0.5)  # half away from zero
    q = np.clip(q, -7, 7).astype(np.int64).reshape(n_out, K)
    nib = (q + 8).astype(np.uint8)
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return packed, s


def dequantize_w4(packed, scales, group: int = W4_GROUP):
    """The weights that 4-bit codes and their scales stand for: [Nout][K] float64."""
    packed = np.asarray(packed, dtype=np.uint8)
    n_out, half = packed.shape
    K = 2 * half
    q = np.empty((n_out, K), dtype=np.int64)
    q[:, 0::2] = (packed & 15).astype(np.int64) - 8
    q[:, 1::2] = (packed >> 4).astype(np.int64) - 8
    s = np.repeat(np.asarray(scales, dtype=np.float64), group, axis=1)
    return q * s


def linear_w4(X, packed, scales, group: int = W4_GROUP):
    """out[m][f] = sum_k X[m][k] * Wdq[f][k] with Wdq the dequantized weights, in float64."""
    return np.asarray(X, dtype=np.float64) @ dequantize_w4(packed, scales, group).T


# ---------------------------------------------------------------------------------------------
# The full drafter block: the two-branch layer between pre-norms and residuals, then a SwiGLU
# MLP.  The pages fix the layer, not the backbone around it; this is the plainest pre-norm block.
# bw holds norm1 [d], norm2 [d], w_gate [F][d], w_up [F][d], w_down [d][F] and eps.
# ---------------------------------------------------------------------------------------------


def rms_norm(x, g, eps: float):
    """x / sqrt(mean over the row of x^2 + eps) * g, row by row."""
    x = np.asarray(x, F64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(g, F64)


def silu(z):
    """z * sigmoid(z)."""
    z = np.asarray(z, F64)
    return z * sigmoid(z)


def swiglu_mlp(z, w_gate, w_up, w_down):
    """(silu(z Wg^T) * (z Wu^T)) Wd^T."""
    z = np.asarray(z, F64)
    a = silu(z @ np.asarray(w_gate, F64).T) * (z @ np.asarray(w_up, F64).T)
    return a @ np.asarray(w_down, F64).T


def block_commit(shape, wts: dict, bw: dict, st: dict, feats):
    """The block's memory commit: the layer commits its own input, RMSNorm(feats) * g1."""
    return commit(shape, wts, st, rms_norm(feats, bw["norm1"], bw["eps"]))


def block_draft(shape, wts: dict, bw: dict, st: dict, block_in):
    """One draft step of the full block; reads the state, never writes it.  Returns [nb][d]."""
    x = np.asarray(block_in, F64)
    h = x + draft(shape, wts, st, rms_norm(x, bw["norm1"], bw["eps"]))
    return h + swiglu_mlp(rms_norm(h, bw["norm2"], bw["eps"]), bw["w_gate"], bw["w_up"], bw["w_down"])


def block_round(shape, wts: dict, bw: dict, st: dict, commit_feats, block_in):
    """One verification round of the full block: commit the accepted rows, then draft."""
    st2, _ = block_commit(shape, wts, bw, st, commit_feats)
    return st2, block_draft(shape, wts, bw, st2, block_in)
