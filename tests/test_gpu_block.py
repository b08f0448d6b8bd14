"""Parity of the full drafter block (hyf_block_commit / hyf_block_draft, through the C ABI) with the
oracle's block_commit / block_draft: pre-norm, the two-branch layer, residual, pre-norm, SwiGLU MLP,
residual; the memory commits the normalized rows.

Tolerance as for the layer (max-norm relative per output tensor): fp32 1e-4; bf16 2e-2 with max abs
error 5e-2.  Each GPU step prints its case before it runs.
"""

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
    rel = err / max(np.max(np.abs(ref)) if ref.size else 0.0, 1e-30)
    if dtype == "f32":
        assert rel <= 1e-4, f"{what}: rel {rel:.3e} (abs {err:.3e})"
    else:
        assert rel <= 2e-2 and err <= 5e-2, f"{what}: rel {rel:.3e} abs {err:.3e}"


def small_shape(dtype, **kw):
    base = dict(d_model=256, n_heads=4, head_dim=64, d_state=64, window=40, chunk=64, dtype=dtype)
    base.update(kw)
    return I.LayerShape(**base)


class BlockPair:
    """The HIP block and the oracle side by side, fed the same rows."""

    def __init__(self, shape, seed, pool_slots=1, max_requests=1, max_rows=8, d_ff=None):
        self.shape = shape
        self.rng = I.rng_streams(seed)
        self.w = I.make_weights(shape, self.rng[0], d_random=True)
        self.bw = I.make_block_weights(shape, self.rng[5], d_ff)
        self.wo = {k: np.asarray(v, np.float64) for k, v in self.w.items()}
        self.bwo = {k: (np.asarray(v, np.float64) if k != "eps" else v) for k, v in self.bw.items()}
        self.gpu = hf.DrafterBlock(shape, self.w, self.bw, pool_slots=pool_slots, max_requests=max_requests,
                                   max_rows=max_rows)
        self.gpu.reset()
        self.ost = [O.new_state(shape) for _ in range(pool_slots)]

    def rows(self, n, stream=1, scale=1.0):
        # N(0, scale^2 / d_model) elements: root mean square `scale / sqrt(d_model)` before the norm
        return I.make_rows(self.rng[stream], n, self.shape.d_model, scale / np.sqrt(self.shape.d_model),
                           self.shape.dtype)

    def commit(self, feats_list):
        cu = np.concatenate([[0], np.cumsum([len(f) for f in feats_list])]).astype(np.int64)
        self.gpu.commit(hf.to_device(np.concatenate(feats_list), self.shape), cu)
        for i, f in enumerate(feats_list):
            self.ost[i], _ = O.block_commit(self.shape, self.wo, self.bwo, self.ost[i], f)

    def draft(self, blocks, commits=None):
        R = len(blocks)
        bi = hf.to_device(np.concatenate(blocks), self.shape)
        bo = torch.empty_like(bi)
        cf = cu = None
        if commits is not None:
            cu = np.concatenate([[0], np.cumsum([len(f) for f in commits])]).astype(np.int64)
            cf = hf.to_device(np.concatenate(commits) if cu[-1] else np.zeros((1, self.shape.d_model), np.float32),
                              self.shape)
        self.gpu.draft(bi, bo, cf, cu)
        outs = []
        for i in range(R):
            if commits is not None:
                self.ost[i], _ = O.block_commit(self.shape, self.wo, self.bwo, self.ost[i], commits[i])
            outs.append(O.block_draft(self.shape, self.wo, self.bwo, self.ost[i], blocks[i]))
        torch.cuda.synchronize()
        return bo.float().cpu().numpy().reshape(R, hf.HYF_BLOCK, -1), np.stack(outs)

    def check_state(self, slot, what):
        torch.cuda.synchronize()
        g = self.gpu.state(slot)
        o = self.ost[slot]
        assert int(g["count"].item()) == o["count"], what
        assert_close(g["H"].cpu().numpy(), o["H"], self.shape.dtype, f"{what} H")
        n = min(o["count"], self.shape.window)
        assert_close(g["V"].float().cpu().numpy()[:, :n], o["V"][:, :n], self.shape.dtype, f"{what} V")


BLOCK_SHAPES = [
    ("tiny_fp32", I.TINY, None),
    ("small_bf16", small_shape("bf16"), 256),
    ("gdn_bf16", small_shape("bf16", memory="gdn"), 320),
    ("lastw_fp32", small_shape("f32", window=24, memory="lastw"), 96),
]


@pytest.mark.parametrize("name,shape,d_ff", BLOCK_SHAPES, ids=[c[0] for c in BLOCK_SHAPES])
def test_block_rounds_match_the_oracle(name, shape, d_ff):
    # Two requests: ragged prefills (rows 3x the layer tests' scale, so the norm matters), then rounds that commit
    # 0-8 rows each and draft; outputs and states against the oracle's block.
    pr = BlockPair(shape, seed=91, pool_slots=2, max_requests=2, max_rows=600, d_ff=d_ff)
    say("hyf_block_commit", name)
    pr.commit([pr.rows(300, scale=3.0), pr.rows(77, scale=3.0)])
    for s in range(2):
        pr.check_state(s, f"{name} prefill request {s}")
    for rnd, a in enumerate(([3, 8], [0, 1], [5, 2])):
        say("hyf_block_draft", name, "round", rnd, a)
        g, o = pr.draft([pr.rows(8, 3, scale=2.0) for _ in range(2)],
                        commits=[pr.rows(n, scale=3.0) for n in a])
        assert_close(g, o, shape.dtype, f"{name} round {rnd}")
    for s in range(2):
        pr.check_state(s, f"{name} after rounds request {s}")


def test_block_draft_never_writes_the_state():
    shape = small_shape("bf16")
    pr = BlockPair(shape, seed=92, max_rows=200, d_ff=128)
    pr.commit([pr.rows(150)])
    torch.cuda.synchronize()
    before = pr.gpu.state(0)["blob"].clone()
    say("hyf_block_draft without commit rows")
    g, o = pr.draft([pr.rows(8, 3)])
    assert_close(g, o, "bf16", "draft only")
    assert torch.equal(before, pr.gpu.state(0)["blob"])


def test_block_qwen_shape_rounds():
    # The Qwen3-4B-shaped layer inside the block (d_ff 3 d_model = 7680): a 1024-row prefix, then
    # three rounds, one request.
    shape = I.QWEN
    pr = BlockPair(shape, seed=93, max_rows=1100)
    say("hyf_block_commit qwen 1024 rows")
    pr.commit([pr.rows(1024, scale=1.0)])
    pr.check_state(0, "qwen prefix")
    for rnd, a in enumerate((4, 8, 1)):
        say("hyf_block_draft qwen round", rnd, a)
        g, o = pr.draft([pr.rows(8, 3)], commits=[pr.rows(a)])
        assert_close(g, o, "bf16", f"qwen round {rnd}")
    pr.check_state(0, "qwen after rounds")


def test_two_blocks_chain():
    # Two blocks, each with its own memory: block 2 drafts from block 1's output (storage dtype).
    shape = small_shape("bf16")
    b1 = BlockPair(shape, seed=94, max_rows=200, d_ff=192)
    b2 = BlockPair(shape, seed=95, max_rows=200, d_ff=192)
    feats = b1.rows(120)
    b1.commit([feats])
    b2.commit([feats])
    x = b1.rows(8, 3)
    say("two blocks")
    bi = hf.to_device(x, shape)
    o1 = torch.empty_like(bi)
    o2 = torch.empty_like(bi)
    b1.gpu.draft(bi, o1)
    b2.gpu.draft(o1, o2)
    torch.cuda.synchronize()
    r1 = O.block_draft(shape, b1.wo, b1.bwo, b1.ost[0], x)
    r2 = O.block_draft(shape, b2.wo, b2.bwo, b2.ost[0], O.round_storage(r1, "bf16"))
    assert_close(o1.float().cpu().numpy(), r1, "bf16", "block 1")
    assert_close(o2.float().cpu().numpy(), r2, "bf16", "block 2")
