"""The allocation-free draft call (hyf_draft_block_noalloc) against hyf_draft_block, through the
C ABI: the same outputs and the same state, bit for bit, on calls in a row whose second call is
smaller than the first (the scratch array keeps the first call's contents), and both against the
oracle (fp32 1e-4; bf16 2e-2 relative with max abs 5e-2)."""

import numpy as np
import pytest
import torch

from hybrid_ssm_local_amd import hyflash as hf
from hybrid_ssm_local_amd import inputs as I
from oracle import hyflash_oracle as O

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def _close(got, ref, what):
    err = float(np.max(np.abs(got - ref)))
    rel = err / max(float(np.max(np.abs(ref))), 1e-30)
    assert rel <= 2e-2 and err <= 5e-2, f"{what}: rel {rel:.3e} abs {err:.3e}"


def test_allocation_free_draft_matches_the_workspace_call():
    shape = I.QWEN
    R = 4
    rng = I.rng_streams(91)
    w = I.make_weights(shape, rng[0], d_random=True)
    wo = {k: np.asarray(v, np.float64) for k, v in w.items()}
    layer = hf.DrafterLayer(shape, w, pool_slots=R, max_requests=R, max_rows=4 * 600)
    scale = 1.0 / np.sqrt(shape.d_model)
    rows = lambda n, s=1: I.make_rows(rng[s], n, shape.d_model, scale, shape.dtype)
    lens = [600, 37, 512, 129]
    pre = [rows(n) for n in lens]
    say("noalloc: prefill", lens)
    layer.reset()
    layer.commit(hf.to_device(np.concatenate(pre), shape), np.concatenate([[0], np.cumsum(lens)]))
    ost = [O.commit(shape, wo, O.new_state(shape), f)[0] for f in pre]
    torch.cuda.synchronize()
    pool_b = layer.pool.clone()
    # call 1: four requests with commit rows; call 2: two requests (a smaller call); call 3: one
    # request, no commit rows
    calls = [([0, 1, 2, 3], [3, 8, 1, 5]), ([2, 0], [2, 7]), ([1], None)]
    for c, (slots, acc) in enumerate(calls):
        n = len(slots)
        blocks = [rows(8, 3) for _ in range(n)]
        bi = hf.to_device(np.concatenate(blocks), shape)
        out_a, out_b = torch.empty_like(bi), torch.full_like(bi, float("nan"))
        cf = cu = None
        commits = None
        if acc is not None:
            commits = [rows(a, 2) for a in acc]
            cu = np.concatenate([[0], np.cumsum(acc)]).astype(np.int64)
            cf = hf.to_device(np.concatenate(commits), shape)
        say("noalloc: call", c, "slots", slots, "acc", acc, "hyf_draft_block")
        layer.draft(bi, out_a, cf, cu, slots)
        say("noalloc: call", c, "hyf_draft_block_noalloc")
        hf.check(hf.hyf_draft_block_noalloc(layer.cfg, layer.w, pool_b, R, slots, n, cf, cu, bi, out_b),
                 "hyf_draft_block_noalloc")
        torch.cuda.synchronize()
        assert torch.equal(out_a, out_b), f"call {c}: outputs differ"
        assert torch.equal(layer.pool, pool_b), f"call {c}: states differ"
        ref = []
        for i, s in enumerate(slots):
            if commits is not None:
                ost[s], _ = O.commit(shape, wo, ost[s], commits[i])
            ref.append(O.draft(shape, wo, ost[s], blocks[i]))
        _close(out_b.float().cpu().numpy(), np.concatenate(ref), f"call {c} against the oracle")
    # a call over the scratch array's size is refused before any device work
    big = 64
    pool_big = torch.zeros(big * layer.state_bytes, dtype=torch.uint8, device="cuda")
    bi = torch.zeros((big * 8, shape.d_model), dtype=torch.bfloat16, device="cuda")
    bo = torch.full_like(bi, 7.0)
    cu = np.arange(0, 8 * big + 1, 8, dtype=np.int64)
    cf = torch.zeros((8 * big, shape.d_model), dtype=torch.bfloat16, device="cuda")
    say("noalloc: oversized call")
    assert hf.hyf_draft_block_noalloc(layer.cfg, layer.w, pool_big, big, None, big, cf, cu, bi, bo) == \
        hf.HYF_ECAPACITY
    torch.cuda.synchronize()
    assert bool(torch.all(bo == 7.0)) and int(pool_big.count_nonzero()) == 0
