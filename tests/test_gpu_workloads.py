"""Parity at the full sizes of the larger workloads, on outputs the oracle can compute one by one.

* Phi-4-shaped drafter, two layers, 32768-feature prefix;
* 64 batched Qwen3-4B-shaped requests with prefixes of 2K-16K features;
* Phi-4-shaped layer with chunk 256 and a 131072-feature prefix.

The oracle recomputes sampled heads of sampled requests from the projection columns those heads
use (one matmul over the request's rows, then its chunked scan, pinned to the sequential
recurrence), and runs whole rounds where its cost allows (the shortest batched prefix, a
1024-feature two-layer prefix).  Tolerances as in test_gpu_parity.
"""

import numpy as np
import pytest
import torch

from hybrid_ssm_local_amd import hyflash as hf
from hybrid_ssm_local_amd import inputs as I
from oracle import hyflash_oracle as O
from test_gpu_parity import Pair, assert_close, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def head_reference(shape, w, feats, h, chunk):
    """Oracle H of head h and its ring rows after committing `feats` to an empty state."""
    nh, P, N, W = shape.n_heads, shape.head_dim, shape.d_state, shape.window
    g = shape.in_groups
    grp = h // (nh // shape.n_groups)
    w_in = np.asarray(w["w_in"], np.float64)
    rows = np.concatenate([w_in[g["v"][0] + h * P: g["v"][0] + (h + 1) * P],
                           w_in[g["B"][0] + grp * N: g["B"][0] + (grp + 1) * N],
                           w_in[g["dt"][0] + h: g["dt"][0] + h + 1]])
    T = feats.shape[0]
    proj = np.empty((T, rows.shape[0]))
    for i in range(0, T, 8192):  # float64 in slices of 8192 rows
        proj[i:i + 8192] = np.asarray(feats[i:i + 8192], np.float64) @ rows.T
    x, B, dt = proj[:, None, :P], proj[:, P:P + N], proj[:, P + N:]
    sl = slice(h, h + 1)
    H, _ = O.ssd_chunked(x, B, None, dt, w["a_log"][sl].astype(np.float64), w["dt_bias"][sl].astype(np.float64),
                         w["d_skip"][sl].astype(np.float64), np.zeros((1, P, N)), chunk)
    m = min(T, W)
    last = np.asarray(feats[T - m:], np.float64)
    k = last @ w_in[g["k"][0] + h * P: g["k"][0] + (h + 1) * P].T
    v = proj[T - m:, :P]
    return H[0], O.round_storage(k, shape.dtype), O.round_storage(v, shape.dtype)


def check_heads(layer, shape, w, feats, slot, heads, chunk, what):
    torch.cuda.synchronize()
    st = layer.state(slot)
    T, W = feats.shape[0], shape.window
    assert int(st["count"].item()) == T, what
    m = min(T, W)
    slots = [(T - m + j) % W for j in range(m)]
    for h in heads:
        say("oracle head", h, what)
        H, k, v = head_reference(shape, w, feats, h, chunk)
        assert_close(st["H"][h].cpu().numpy(), H, shape.dtype, f"{what} head {h} H")
        assert_close(st["K"][h].float().cpu().numpy()[slots], k, shape.dtype, f"{what} head {h} K")
        assert_close(st["V"][h].float().cpu().numpy()[slots], v, shape.dtype, f"{what} head {h} V")


def oracle_state(layer, slot=0):
    """The GPU's state of one request as an oracle state (count, H, ring K and V in float64), so the
    oracle's rounds can start from the state the GPU's prefill left."""
    torch.cuda.synchronize()
    st = layer.state(slot)
    return dict(count=int(st["count"].item()), H=st["H"].cpu().numpy().astype(np.float64),
                K=st["K"].float().cpu().numpy().astype(np.float64), V=st["V"].float().cpu().numpy().astype(np.float64))


def compare_state(layer, slot, ost, shape, heads, what):
    torch.cuda.synchronize()
    st = layer.state(slot)
    assert int(st["count"].item()) == ost["count"], what
    n = min(ost["count"], shape.window)
    for h in heads:
        assert_close(st["H"][h].cpu().numpy(), ost["H"][h], shape.dtype, f"{what} head {h} H")
        assert_close(st["K"][h].float().cpu().numpy()[:n], ost["K"][h][:n], shape.dtype, f"{what} head {h} K")
        assert_close(st["V"][h].float().cpu().numpy()[:n], ost["V"][h][:n], shape.dtype, f"{what} head {h} V")


def gdn_head_reference(shape, w, feats, h):
    """Oracle H of head h of the gated delta-rule memory after committing `feats` to an empty state
    (the chunked form, pinned to the token-by-token rule)."""
    nh, P, N = shape.n_heads, shape.head_dim, shape.d_state
    g = shape.in_groups
    grp = h // (nh // shape.n_groups)
    w_in = np.asarray(w["w_in"], np.float64)
    rows = np.concatenate([w_in[g["v"][0] + h * P: g["v"][0] + (h + 1) * P],
                           w_in[g["B"][0] + grp * N: g["B"][0] + (grp + 1) * N],
                           w_in[g["alpha"][0] + h: g["alpha"][0] + h + 1],
                           w_in[g["beta"][0] + h: g["beta"][0] + h + 1]])
    T = feats.shape[0]
    proj = np.empty((T, rows.shape[0]))
    for i in range(0, T, 8192):
        proj[i:i + 8192] = np.asarray(feats[i:i + 8192], np.float64) @ rows.T
    x, B = proj[:, None, :P], proj[:, P:P + N]
    al, be = proj[:, P + N:P + N + 1], proj[:, P + N + 1:P + N + 2]
    sl = slice(h, h + 1)
    H = O.gdn_chunked(x, B, al, be, w["dt_bias"][sl].astype(np.float64), w["a_log"][sl].astype(np.float64),
                      np.zeros((1, P, N)), 64)
    return H[0]


def test_phi4_two_layer_prefill_32768_sampled_heads():
    shape = I.PHI4
    wl = I.WORKLOADS["phi4_bf16_2layer"]
    rng = I.rng_streams(wl["seed"])
    ws = [I.make_weights(shape, rng[0]), I.make_weights(shape, rng[5])]
    T = wl["prefix"]
    feats = I.make_rows(rng[1], T, shape.d_model, wl["feat_scale"], shape.dtype)
    f = hf.to_device(feats, shape)
    for li, w in enumerate(ws):
        layer = hf.DrafterLayer(shape, w, max_rows=T)
        layer.reset()
        say("hyf_memory_commit phi4 prefill", T, "layer", li)
        layer.commit(f, [0, T])
        check_heads(layer, shape, w, feats, 0, (0, 17, 39), shape.chunk, f"phi4 layer {li}")
        del layer
    torch.cuda.empty_cache()


def test_phi4_two_layer_rounds_match_the_oracle():
    # The layers chain while drafting (the second layer drafts from block_in + the first layer's
    # output); both commit the same accepted target features.  1024-feature prefix, 4 rounds.
    shape = I.PHI4
    p1, p2 = Pair(shape, seed=201, max_rows=1024), Pair(shape, seed=202, max_rows=1024)
    rows = I.rng_streams(203)
    feats = I.make_rows(rows[1], 1024, shape.d_model, 1.0 / np.sqrt(shape.d_model), shape.dtype)
    for p in (p1, p2):
        p.gpu.reset()
        say("phi4 two-layer prefill 1024")
        p.commit([feats])
    for rnd, a in enumerate((5, 1, 8, 3)):
        cf = I.make_rows(rows[2], a, shape.d_model, 1.0 / np.sqrt(shape.d_model), shape.dtype)
        bi = I.make_rows(rows[3], 8, shape.d_model, 1.0 / np.sqrt(shape.d_model), shape.dtype)
        say("phi4 two-layer round", rnd, "a", a)
        cfd = hf.to_device(cf, shape)
        x1 = hf.to_device(bi, shape)
        o1 = torch.empty_like(x1)
        p1.gpu.draft(x1, o1, cfd, [0, a])
        x2 = (x1.float() + o1.float()).to(x1.dtype)
        o2 = torch.empty_like(x2)
        p2.gpu.draft(x2, o2, cfd, [0, a])
        torch.cuda.synchronize()
        for p in (p1, p2):
            p.ost[0], _ = O.commit(shape, p.wo, p.ost[0], cf)
        r1, r2 = O.draft_two_layer(shape, p1.wo, p2.wo, p1.ost[0], p2.ost[0], bi)
        assert_close(o1.float().cpu().numpy(), r1, shape.dtype, f"layer 1 round {rnd}")
        assert_close(o2.float().cpu().numpy(), r2, shape.dtype, f"layer 2 round {rnd}")
    p1.check_state(what="layer 1")
    p2.check_state(what="layer 2")


def test_phi4_two_layer_rounds_after_the_full_prefix():
    # Both Phi-4-shaped layers commit the 32768-feature prefix on the GPU; the oracle takes over the
    # states the GPU left and follows four two-layer rounds (layer 2 drafts from block_in + layer 1's
    # output), compared output by output and on sampled heads of the states.
    shape = I.PHI4
    wl = I.WORKLOADS["phi4_bf16_2layer"]
    rng = I.rng_streams(wl["seed"])
    ws = [I.make_weights(shape, rng[0]), I.make_weights(shape, rng[5])]
    wo = [{k: np.asarray(v, np.float64) for k, v in w.items()} for w in ws]
    T = wl["prefix"]
    f = hf.to_device(I.make_rows(rng[1], T, shape.d_model, wl["feat_scale"], shape.dtype), shape)
    layers = []
    for li, w in enumerate(ws):
        layer = hf.DrafterLayer(shape, w, max_rows=T)
        layer.reset()
        say("phi4 two-layer full prefill", T, "layer", li)
        layer.commit(f, [0, T])
        layers.append(layer)
    del f
    ost = [oracle_state(layers[0]), oracle_state(layers[1])]
    for rnd, a in enumerate((3, 8, 1, 5)):
        cf = I.make_rows(rng[2], a, shape.d_model, wl["feat_scale"], shape.dtype)
        bi = I.make_rows(rng[3], 8, shape.d_model, wl["block_scale"], shape.dtype)
        cfd, x1 = hf.to_device(cf, shape), hf.to_device(bi, shape)
        o1 = torch.empty_like(x1)
        say("phi4 two-layer round after the full prefix", rnd, "a", a)
        layers[0].draft(x1, o1, cfd, [0, a])
        x2 = (x1.float() + o1.float()).to(x1.dtype)
        o2 = torch.empty_like(x2)
        layers[1].draft(x2, o2, cfd, [0, a])
        torch.cuda.synchronize()
        for li in (0, 1):
            ost[li], _ = O.commit(shape, wo[li], ost[li], cf)
        r1, r2 = O.draft_two_layer(shape, wo[0], wo[1], ost[0], ost[1], bi)
        assert_close(o1.float().cpu().numpy(), r1, shape.dtype, f"full-prefix layer 1 round {rnd}")
        assert_close(o2.float().cpu().numpy(), r2, shape.dtype, f"full-prefix layer 2 round {rnd}")
    for li in (0, 1):
        compare_state(layers[li], 0, ost[li], shape, (0, 19, 39), f"full-prefix layer {li + 1}")
    del layers
    torch.cuda.empty_cache()


def test_batched_64_requests_prefill_and_rounds():
    shape = I.QWEN
    wl = I.WORKLOADS["qwen3_4b_batched64"]
    R = wl["requests"]
    rng = I.rng_streams(wl["seed"])
    w = I.make_weights(shape, rng[0])
    lo, hi = wl["prefix_range"]
    lens = rng[4].integers(lo, hi + 1, size=R)
    feats = [I.make_rows(rng[1], int(n), shape.d_model, wl["feat_scale"], shape.dtype) for n in lens]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    layer = hf.DrafterLayer(shape, w, pool_slots=R, max_requests=R, max_rows=int(cu[-1]))
    layer.reset()
    say("hyf_memory_commit batched prefill", R, "requests", int(cu[-1]), "rows")
    layer.commit(hf.to_device(np.concatenate(feats), shape), cu)
    short = int(np.argmin(lens))
    for r in (short, 17, 50):
        check_heads(layer, shape, w, feats[r], r, (3, 30), shape.chunk, f"request {r} ({lens[r]} rows)")
    # Rounds for all 64 requests (0-8 accepted rows each); the oracle follows the shortest request from
    # its own prefill, and three more requests from the states the GPU's prefill left.
    wo = {k: np.asarray(v, np.float64) for k, v in w.items()}
    say("oracle prefill of request", short, int(lens[short]))
    st, _ = O.commit(shape, wo, O.new_state(shape), feats[short])
    follow = [r for r in (5, 17, 50, 63) if r != short][:3]
    ost = {r: oracle_state(layer, r) for r in follow}
    for rnd in range(3):
        a = rng[4].integers(0, 9, size=R)
        commits = [I.make_rows(rng[2], int(n), shape.d_model, wl["feat_scale"], shape.dtype) for n in a]
        blocks = [I.make_rows(rng[3], 8, shape.d_model, wl["block_scale"], shape.dtype) for _ in range(R)]
        cuc = np.concatenate([[0], np.cumsum(a)]).astype(np.int64)
        bi = hf.to_device(np.concatenate(blocks), shape)
        bo = torch.empty_like(bi)
        nz = [c for c in commits if len(c)] or [np.zeros((1, shape.d_model), np.float32)]
        cf = hf.to_device(np.concatenate(nz), shape)
        say("batched round", rnd, "rows", int(cuc[-1]))
        layer.draft(bi, bo, cf, cuc)
        torch.cuda.synchronize()
        st, ref = O.round_step(shape, wo, st, commits[short], blocks[short])
        got = bo.float().cpu().numpy().reshape(R, 8, -1)
        assert_close(got[short], ref, shape.dtype, f"batched round {rnd} request {short}")
        for r in follow:
            ost[r], ref = O.round_step(shape, wo, ost[r], commits[r], blocks[r])
            assert_close(got[r], ref, shape.dtype, f"batched round {rnd} request {r}")
        lens = lens + a
    counts = [int(layer.state(r)["count"].item()) for r in range(R)]
    assert counts == [int(n) for n in lens]
    for r in follow:
        compare_state(layer, r, ost[r], shape, (0, 13, 31), f"batched request {r} after rounds")
    del layer
    torch.cuda.empty_cache()


def test_long_phi4_131072_prefill_sampled_heads():
    shape = I.PHI4_LONG
    wl = I.WORKLOADS["phi4_long131k"]
    rng = I.rng_streams(wl["seed"])
    w = I.make_weights(shape, rng[0])
    T = wl["prefix"]
    feats = I.make_rows(rng[1], T, shape.d_model, wl["feat_scale"], shape.dtype)
    layer = hf.DrafterLayer(shape, w, max_rows=T)
    layer.reset()
    say("hyf_memory_commit phi4 prefill", T, "chunk", shape.chunk)
    layer.commit(hf.to_device(feats, shape), [0, T])
    check_heads(layer, shape, w, feats, 0, (0, 21, 39), shape.chunk, "phi4 long")
    del layer
    torch.cuda.empty_cache()


def test_long_phi4_gated_delta_rule_prefix_and_rounds():
    # The gated delta-rule memory at the long-context Phi-4 shape: a 32768-feature prefix through the
    # chunked kernels (sampled heads against the oracle's chunked form), then three rounds from the
    # state the GPU left, compared output by output and on sampled heads.
    shape = I.PHI4_LONG.replace(memory="gdn")
    wl = I.WORKLOADS["phi4_long131k"]
    rng = I.rng_streams(wl["seed"] + 100)
    w = I.make_weights(shape, rng[0])
    wo = {k: np.asarray(v, np.float64) for k, v in w.items()}
    T = 32768
    feats = I.make_rows(rng[1], T, shape.d_model, wl["feat_scale"], shape.dtype)
    layer = hf.DrafterLayer(shape, w, max_rows=T)
    layer.reset()
    say("gdn phi4 prefill", T)
    layer.commit(hf.to_device(feats, shape), [0, T])
    torch.cuda.synchronize()
    st = layer.state(0)
    for h in (0, 21, 39):
        say("gdn oracle head", h)
        assert_close(st["H"][h].cpu().numpy(), gdn_head_reference(shape, w, feats, h), shape.dtype,
                     f"gdn phi4 head {h} H")
    ost = oracle_state(layer)
    for rnd, a in enumerate((4, 8, 2)):
        cf = I.make_rows(rng[2], a, shape.d_model, wl["feat_scale"], shape.dtype)
        bi = I.make_rows(rng[3], 8, shape.d_model, wl["block_scale"], shape.dtype)
        x = hf.to_device(bi, shape)
        out = torch.empty_like(x)
        say("gdn phi4 round", rnd, "a", a)
        layer.draft(x, out, hf.to_device(cf, shape), [0, a])
        torch.cuda.synchronize()
        ost, ref = O.round_step(shape, wo, ost, cf, bi)
        assert_close(out.float().cpu().numpy(), ref, shape.dtype, f"gdn phi4 round {rnd}")
    compare_state(layer, 0, ost, shape, (0, 21, 39), "gdn phi4 after rounds")
    del layer
    torch.cuda.empty_cache()
