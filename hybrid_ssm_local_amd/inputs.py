"""Seeded synthetic inputs for the HyFlash drafter layer.

This module only draws random numbers and casts them to the storage dtype.  It
holds none of the layer's arithmetic, so both the CPU oracle (tests) and the
HIP path (tests, bench) can take their inputs from here without sharing any
of the method.

Shapes follow the workloads the HyFlash pages discuss: a Qwen3-4B-shaped and a
Phi-4-shaped drafter layer, a block of seven draft slots plus the anchor, a
bounded window of recent committed target features, and acceptance lengths of
one to eight committed features per verification round (HyFlash explainer,
"Jargon": parallel block drafting, acceptance length, committed target
features).  The pages publish no activations or trained weights, so every
value is synthetic: features ~ N(0,1)·scale, Xavier-normal weights per
sub-matrix, A_log ~ U(ln 1, ln 16), dt_bias = -2, D = 1.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

F32 = "f32"
BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class LayerShape:
    d_model: int
    n_heads: int
    head_dim: int
    d_state: int
    n_groups: int = 1
    window: int = 512
    block: int = 8
    chunk: int = 64
    dtype: str = BF16
    cross_slot: int = 1
    memory: str = "mamba2"  # or "gdn": the gated delta-rule memory; "lastw": Mamba-2 over the window only
    weights: str = "dense"  # or "w4": the projections' weights as 4-bit codes and scales

    @property
    def dq(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def gn(self) -> int:
        return self.n_groups * self.d_state

    # Row groups of the packed input projection, in storage order:
    # q | C | k | v | B | dt  (each row is one output feature of length d_model);
    # the gated delta-rule memory has the two gates in place of dt: ... | B | alpha | beta.
    @property
    def in_groups(self):
        dq, gn, nh = self.dq, self.gn, self.n_heads
        if self.memory == "gdn":
            names = ("q", "C", "k", "v", "B", "alpha", "beta")
            sizes = (dq, gn, dq, dq, gn, nh, nh)
        else:
            names = ("q", "C", "k", "v", "B", "dt")
            sizes = (dq, gn, dq, dq, gn, nh)
        out, off = {}, 0
        for n, s in zip(names, sizes):
            out[n] = (off, off + s)
            off += s
        return out

    @property
    def n_in(self) -> int:
        return 3 * self.dq + 2 * self.gn + (2 if self.memory == "gdn" else 1) * self.n_heads

    def replace(self, **kw) -> "LayerShape":
        return dataclasses.replace(self, **kw)


# Named workloads (sizes as the HyFlash pages' two target geometries suggest).
TINY = LayerShape(d_model=256, n_heads=4, head_dim=64, d_state=64, window=128, chunk=64, dtype=F32)
QWEN = LayerShape(d_model=2560, n_heads=32, head_dim=80, d_state=128, window=512, chunk=64, dtype=BF16)
PHI4 = LayerShape(d_model=5120, n_heads=40, head_dim=128, d_state=128, window=512, chunk=64, dtype=BF16)
PHI4_LONG = PHI4.replace(chunk=256)

WORKLOADS = {
    "tiny_fp32": dict(shape=TINY, prefix=1024, rounds=20, seed=0, feat_scale=1.0, block_scale=1.0),
    "qwen3_4b_bf16": dict(shape=QWEN, prefix=8192, rounds=256, seed=1,
                          feat_scale=1.0 / math.sqrt(2560), block_scale=1.0 / math.sqrt(2560)),
    "phi4_bf16_2layer": dict(shape=PHI4, prefix=32768, rounds=512, seed=2, layers=2,
                             feat_scale=1.0 / math.sqrt(5120), block_scale=1.0 / math.sqrt(5120)),
    "qwen3_4b_batched64": dict(shape=QWEN, requests=64, prefix_range=(2048, 16384), rounds=128, seed=3,
                               feat_scale=1.0 / math.sqrt(2560), block_scale=1.0 / math.sqrt(2560)),
    "phi4_long131k": dict(shape=PHI4_LONG, prefix=131072, rounds=128, seed=4,
                          feat_scale=1.0 / math.sqrt(5120), block_scale=1.0 / math.sqrt(5120)),
}


def to_storage(a: np.ndarray, dtype: str) -> np.ndarray:
    """Cast to the storage dtype (round to nearest even) and return float32 holding those values."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == F32:
        return a
    import torch

    return torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()


def rng_streams(seed: int, n: int = 8):
    """Independent PCG64 streams (weights, prefix, rounds, block inputs, acceptance, extra...)."""
    ss = np.random.SeedSequence(seed)
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(n)]


def xavier(rng, fan_out: int, fan_in: int) -> np.ndarray:
    std = math.sqrt(2.0 / (fan_in + fan_out))
    return rng.standard_normal((fan_out, fan_in), dtype=np.float32) * np.float32(std)


def make_weights(shape: LayerShape, rng, d_random: bool = False) -> dict:
    """Weights in nn.Linear layout ([out_features][in_features]), stored dtype values as float32.

    w_in:  [n_in][d_model], rows q | C | k | v | B | dt, each group Xavier-normal on its own.
    w_out: [d_model][n_heads*head_dim].
    """
    d = shape.d_model
    parts = []
    for name, (a, b) in shape.in_groups.items():
        parts.append(xavier(rng, b - a, d))
    w_in = to_storage(np.concatenate(parts, axis=0), shape.dtype)
    w_out = to_storage(xavier(rng, d, shape.dq), shape.dtype)
    a_log = rng.uniform(math.log(1.0), math.log(16.0), size=shape.n_heads).astype(np.float32)
    dt_bias = np.full(shape.n_heads, -2.0, dtype=np.float32)
    if shape.memory == "gdn":
        # gate biases: dt_bias carries the retention gate's (alpha = sigmoid(2..5): 0.88-0.99),
        # a_log the write gate's (beta = sigmoid(0) = 0.5 at a zero projection)
        dt_bias = rng.uniform(2.0, 5.0, size=shape.n_heads).astype(np.float32)
        a_log = np.zeros(shape.n_heads, dtype=np.float32)
    if d_random:
        d_skip = rng.standard_normal(shape.n_heads, dtype=np.float32)
    else:
        d_skip = np.ones(shape.n_heads, dtype=np.float32)
    return dict(w_in=w_in, w_out=w_out, a_log=a_log, dt_bias=dt_bias, d_skip=d_skip)


def make_block_weights(shape: LayerShape, rng, d_ff: int | None = None) -> dict:
    """The full block's own weights: the first RMSNorm's gains (1 + 0.1 N(0, 1)) / sqrt(d_model), so
    the layer sees rows of root mean square 1 / sqrt(d_model) like the layer's own synthetic
    features, the second's 1 + 0.1 N(0, 1) (float32), and the SwiGLU MLP's gate and up
    [d_ff][d_model] and down [d_model][d_ff] Xavier-normal in the storage dtype.  d_ff defaults to
    3 d_model."""
    d = shape.d_model
    F = 3 * d if d_ff is None else d_ff
    return dict(norm1=((1 + 0.1 * rng.standard_normal(d)) / math.sqrt(d)).astype(np.float32),
                norm2=(1 + 0.1 * rng.standard_normal(d)).astype(np.float32),
                w_gate=to_storage(xavier(rng, F, d), shape.dtype), w_up=to_storage(xavier(rng, F, d), shape.dtype),
                w_down=to_storage(xavier(rng, d, F), shape.dtype), eps=1e-6)


def make_rows(rng, n: int, d: int, scale: float, dtype: str) -> np.ndarray:
    return to_storage(rng.standard_normal((n, d), dtype=np.float32) * np.float32(scale), dtype)


def acceptance_lengths(rng, n: int, lo: int = 1, hi: int = 8) -> np.ndarray:
    return rng.integers(lo, hi + 1, size=n).astype(np.int64)


def make_scan_inputs(shape: LayerShape, T: int, rng, with_c: bool = True, h0_scale: float = 0.0) -> dict:
    """Pre-projected scan inputs: x [T][nh][P], B/C [T][G*N] (storage dtype), dt_raw [T][nh] f32,
    per-head a_log / dt_bias / d_skip, and an initial state H0 [nh][P][N] f32."""
    nh, P, GN = shape.n_heads, shape.head_dim, shape.gn
    x = to_storage(rng.standard_normal((T, nh, P), dtype=np.float32), shape.dtype)
    B = to_storage(rng.standard_normal((T, GN), dtype=np.float32), shape.dtype)
    C = to_storage(rng.standard_normal((T, GN), dtype=np.float32), shape.dtype) if with_c else None
    dt_raw = rng.standard_normal((T, nh), dtype=np.float32)
    a_log = rng.uniform(math.log(1.0), math.log(16.0), size=nh).astype(np.float32)
    dt_bias = np.full(nh, -2.0, dtype=np.float32)
    d_skip = rng.standard_normal(nh, dtype=np.float32)
    H0 = (rng.standard_normal((nh, P, shape.d_state), dtype=np.float32) * np.float32(h0_scale)
          if h0_scale else np.zeros((nh, P, shape.d_state), dtype=np.float32))
    return dict(x=x, B=B, C=C, dt_raw=dt_raw, a_log=a_log, dt_bias=dt_bias, d_skip=d_skip, H0=H0)


def random_w4(rng, n_out: int, k: int):
    """Random 4-bit codes and scales of an [n_out][k] weight (k a multiple of 128) for timing runs:
    codes uniform 0..15 packed two per byte, scales 1 / (7 sqrt(k)) to 2 / (7 sqrt(k)).  Returns
    (codes uint8 [n_out][k/2], scales float32 [n_out][k/128])."""
    codes = rng.integers(0, 256, size=(n_out, k // 2), dtype=np.uint8)
    scales = (rng.uniform(1.0, 2.0, size=(n_out, k // 128)) / (7.0 * math.sqrt(k))).astype(np.float32)
    return codes, scales
