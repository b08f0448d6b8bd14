"""Host-only checks of the C ABI: the library loads, exports what the header declares, and
validates arguments before any device work (no GPU needed: every call here fails validation
or is a pure host query)."""

import ctypes
import subprocess

import numpy as np

import pytest

from hybrid_ssm_local_amd import hyflash as hf
from hybrid_ssm_local_amd import inputs as I


def test_library_exports_every_declared_function():
    names = hf.header_functions()
    assert len(names) >= 12
    out = subprocess.run(["nm", "-D", "--defined-only", hf.LIB_PATH], capture_output=True, text=True, check=True)
    exported = {line.split()[-1] for line in out.stdout.splitlines() if " T " in line}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    L = hf.lib()
    for n in names:
        assert getattr(L, n) is not None
    assert hf.hyf_abi_version() == 2


def test_struct_sizes_match_the_header():
    assert ctypes.sizeof(hf.HyfConfig) == 48
    assert ctypes.sizeof(hf.HyfWeights) == 72  # nine pointers
    assert ctypes.sizeof(hf.HyfStateLayout) == 56
    assert ctypes.sizeof(hf.HyfBlockWeights) == 40  # four pointers, d_ff, eps


@pytest.mark.parametrize("shape", [I.TINY, I.QWEN, I.PHI4, I.PHI4_LONG])
def test_named_shapes_are_accepted(shape):
    cfg = hf.make_config(shape)
    assert hf.hyf_config_check(cfg) == hf.HYF_OK
    assert hf.hyf_n_in(cfg) == shape.n_in


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 72, hf.HYF_ESHAPE), ("head_dim", 0, hf.HYF_ESHAPE), ("d_state", 300, hf.HYF_ESHAPE),
    ("n_groups", 3, hf.HYF_ESHAPE), ("window", 0, hf.HYF_ESHAPE), ("block", 7, hf.HYF_ESHAPE),
    ("chunk", 8, hf.HYF_ESHAPE), ("chunk", 48, hf.HYF_ESHAPE), ("dtype", 5, hf.HYF_EDTYPE), ("memory", 3, hf.HYF_EINVAL),
    ("cross_slot", 2, hf.HYF_EINVAL), ("weights", 2, hf.HYF_EINVAL), ("d_model", 100, hf.HYF_ESHAPE),
])
def test_bad_configs_are_rejected(field, value, status):
    cfg = hf.make_config(I.QWEN)
    setattr(cfg, field, value)
    assert hf.hyf_config_check(cfg) == status
    assert hf.hyf_state_bytes(cfg) == 0
    assert hf.hyf_workspace_bytes(cfg, 1, 8) == 0


def test_state_layout_and_the_pages_fp32_state_size():
    # One Phi-4-shaped layer's H is 40 x 128 x 128 fp32 = 2.5 MiB (the pages' FP32 recurrent state).
    L = hf.hyf_state_layout_get(hf.make_config(I.PHI4))
    assert L.k_off - L.h_off == 40 * 128 * 128 * 4 == int(2.5 * 2**20)
    assert L.count_off == 0 and L.h_off == 256
    assert L.v_off - L.k_off == L.total - L.v_off == 40 * 512 * 128 * 2
    for sh in (I.TINY, I.QWEN):
        L = hf.hyf_state_layout_get(hf.make_config(sh))
        es = 4 if sh.dtype == "f32" else 2
        assert L.k_off - L.h_off >= sh.n_heads * sh.head_dim * sh.d_state * 4
        assert L.v_off - L.k_off >= sh.n_heads * sh.window * sh.head_dim * es
        assert all(v % 256 == 0 for v in (L.h_off, L.k_off, L.v_off, L.total))
        assert hf.hyf_state_bytes(hf.make_config(sh)) == L.total


def test_workspace_grows_with_requests_and_rows():
    cfg = hf.make_config(I.QWEN)
    a = hf.hyf_workspace_bytes(cfg, 1, 8)
    b = hf.hyf_workspace_bytes(cfg, 1, 8192)
    c = hf.hyf_workspace_bytes(cfg, 64, 8192)
    assert 0 < a < b < c
    assert hf.hyf_workspace_bytes(cfg, 0, 8) == 0
    assert hf.hyf_workspace_bytes(cfg, hf.HYF_MAX_REQUESTS + 1, 8) == 0
    assert hf.hyf_ssd_scan_workspace_bytes(cfg, 8192) > 0
    # per-token outputs keep one state per 128-token block
    assert hf.hyf_workspace_bytes(cfg, 1, 8192, 1) >= b
    assert hf.hyf_ssd_scan_workspace_bytes(cfg, 8192, 1) >= 64 * 32 * 80 * 128 * 4


def test_per_token_outputs_beyond_lds_are_unsupported():
    # fp32 with head_dim + 2 d_state > 320: a 128-token block of x, B and C exceeds one
    # workgroup's LDS, so y is refused before any device work (the state-only scan still runs).
    shape = I.LayerShape(d_model=256, n_heads=2, head_dim=128, d_state=128, window=16, chunk=64, dtype="f32")
    cfg = hf.make_config(shape)
    assert hf.hyf_config_check(cfg) == hf.HYF_OK
    fake = 1 << 20
    w = hf.HyfWeights(fake, fake, fake, fake, fake)
    assert hf.hyf_ssd_scan(cfg, fake, fake, fake, fake, fake, fake, fake, fake, fake, 4, fake, 1 << 30, 0) == \
        hf.HYF_EUNSUPPORTED
    assert hf.hyf_memory_commit(cfg, w, fake, 1, None, 1, fake, [0, 4], fake, fake, 1 << 30, 0) == \
        hf.HYF_EUNSUPPORTED
    # bf16 of the same sizes fits
    cfg_b = hf.make_config(I.LayerShape(d_model=256, n_heads=2, head_dim=128, d_state=128, window=16, chunk=64,
                                        dtype="bf16"))
    assert hf.hyf_ssd_scan(cfg_b, fake, fake, fake, fake, fake, fake, fake, fake, fake, 4, fake, 16, 0) == \
        hf.HYF_EWORKSPACE


def test_invalid_calls_fail_before_any_device_work():
    cfg = hf.make_config(I.TINY)
    w = hf.HyfWeights(None, None, None, None, None)
    fake = 1 << 20  # never dereferenced: validation fails first
    assert hf.hyf_memory_commit(cfg, w, fake, 1, None, 1, fake, [0, 4], None, fake, 1 << 30, 0) == hf.HYF_EINVAL
    good_w = hf.HyfWeights(fake, fake, fake, fake, fake)
    # misaligned pool, bad offsets, too many requests, slot outside the pool, duplicate slots
    assert hf.hyf_memory_commit(cfg, good_w, fake + 8, 1, None, 1, fake, [0, 4], None, fake, 1 << 30, 0) == \
        hf.HYF_EINVAL
    assert hf.hyf_memory_commit(cfg, good_w, fake, 1, None, 1, fake, [1, 4], None, fake, 1 << 30, 0) == hf.HYF_EINVAL
    assert hf.hyf_memory_commit(cfg, good_w, fake, 2, None, 2, fake, [0, 4, 2], None, fake, 1 << 30, 0) == \
        hf.HYF_EINVAL
    assert hf.hyf_memory_commit(cfg, good_w, fake, 1, [3], 1, fake, [0, 4], None, fake, 1 << 30, 0) == \
        hf.HYF_ECAPACITY
    assert hf.hyf_memory_commit(cfg, good_w, fake, 4, [1, 1], 2, fake, [0, 1, 2], None, fake, 1 << 30, 0) == \
        hf.HYF_EINVAL
    n = hf.HYF_MAX_REQUESTS + 1
    assert hf.hyf_memory_commit(cfg, good_w, fake, n, None, n, fake, list(range(n + 1)), None, fake, 1 << 30, 0) == \
        hf.HYF_ECAPACITY
    # workspace too small
    assert hf.hyf_memory_commit(cfg, good_w, fake, 1, None, 1, fake, [0, 4], None, fake, 16, 0) == \
        hf.HYF_EWORKSPACE
    # a round may commit at most `block` rows per request
    assert hf.hyf_draft_block(cfg, good_w, fake, 1, None, 1, fake, [0, 9], fake, fake, fake, 1 << 30, 0) == \
        hf.HYF_ECAPACITY
    # commit rows without offsets
    assert hf.hyf_draft_block(cfg, good_w, fake, 1, None, 1, fake, None, fake, fake, fake, 1 << 30, 0) == \
        hf.HYF_EINVAL
    # scan: y requested without C, negative length
    assert hf.hyf_ssd_scan(cfg, fake, fake, None, fake, fake, fake, fake, fake, fake, 4, fake, 1 << 30, 0) == \
        hf.HYF_EINVAL
    assert hf.hyf_ssd_scan(cfg, fake, fake, None, fake, fake, fake, fake, fake, None, -1, fake, 1 << 30, 0) == \
        hf.HYF_ECAPACITY
    # misaligned operand
    assert hf.hyf_ssd_scan(cfg, fake + 4, fake, None, fake, fake, fake, fake, fake, None, 10, fake, 1 << 30, 0) == \
        hf.HYF_EINVAL


def test_empty_commit_is_accepted_without_device_work():
    cfg = hf.make_config(I.TINY)
    fake = 1 << 20
    w = hf.HyfWeights(fake, fake, fake, fake, fake)
    assert hf.hyf_memory_commit(cfg, w, fake, 1, None, 1, None, [0, 0], None, None, 0, 0) == hf.HYF_OK
    assert hf.hyf_ssd_scan(cfg, None, None, None, None, fake, fake, fake, fake, None, 0, None, 0, 0) == hf.HYF_OK


def test_status_strings():
    assert hf.status_str(hf.HYF_OK) == "ok"
    assert "workspace" in hf.status_str(hf.HYF_EWORKSPACE)


@pytest.mark.parametrize("elem_bytes", [2, 4])
def test_time_tiled_layout_places_each_element_as_documented(elem_bytes):
    # the header's formula, element by element, on a ragged length
    T, F = 300, 48
    a = np.arange(T * F, dtype=np.float64).reshape(T, F)
    out = hf.time_tiled(a, T, elem_bytes, pad=-1.0).reshape(-1)
    vn = 16 // elem_bytes
    kt, nj = 4 * vn, hf.HYF_TBLK // (4 * vn)
    for t in range(0, T, 7):
        for f in range(0, F, 5):
            tt = t % hf.HYF_TBLK
            off = (((f // 16) * nj + tt // kt) * 64 + ((tt % kt) // vn) * 16 + f % 16) * vn + tt % vn
            assert out[(t // hf.HYF_TBLK) * F * hf.HYF_TBLK + off] == a[t, f]
    assert out.size == 3 * F * hf.HYF_TBLK and (out == -1.0).sum() == (3 * hf.HYF_TBLK - T) * F


def test_gated_delta_rule_configs():
    # the gated delta-rule memory adds a second gate row per head to w_in; its commit has no y, and
    # the scan entry point on pre-projected inputs is the Mamba-2 memory's only
    shape = I.QWEN.replace(memory="gdn")
    cfg = hf.make_config(shape)
    assert cfg.memory == hf.HYF_MEM_GDN and hf.hyf_config_check(cfg) == hf.HYF_OK
    assert hf.hyf_n_in(cfg) == shape.n_in == 3 * shape.dq + 2 * shape.gn + 2 * shape.n_heads
    assert hf.hyf_n_in(hf.make_config(I.QWEN)) == I.QWEN.n_in
    assert hf.hyf_workspace_bytes(cfg, 1, 8192) > hf.hyf_workspace_bytes(hf.make_config(I.QWEN), 1, 8192)
    fake = 1 << 20
    w = hf.HyfWeights(fake, fake, fake, fake, fake)
    assert hf.hyf_ssd_scan(cfg, fake, fake, None, fake, fake, fake, fake, fake, None, 4, fake, 1 << 30, 0) == \
        hf.HYF_EUNSUPPORTED
    assert hf.hyf_memory_commit(cfg, w, fake, 1, None, 1, fake, [0, 4], fake, fake, 1 << 30, 0) == \
        hf.HYF_EUNSUPPORTED


def test_four_bit_projection_rejects_bad_calls_before_device_work():
    fake = 1 << 20  # never dereferenced: validation fails first
    cfg = hf.make_config(I.QWEN)
    assert cfg.dtype == hf.HYF_BF16
    ok = (fake, 12, 2560, fake, fake, 7968, fake, 1, 0)
    # K not a multiple of 128, no rows of weights, too many rows
    assert hf.hyf_linear_w4(cfg, fake, 12, 2560 + 64, fake, fake, 7968, fake, 1, 0) == hf.HYF_ESHAPE
    assert hf.hyf_linear_w4(cfg, fake, 12, 2560, fake, fake, 0, fake, 1, 0) == hf.HYF_ESHAPE
    assert hf.hyf_linear_w4(cfg, fake, 64 * 65535 + 1, 2560, fake, fake, 7968, fake, 1, 0) == hf.HYF_ESHAPE
    # misaligned codes, null scales
    assert hf.hyf_linear_w4(cfg, fake, 12, 2560, fake + 8, fake, 7968, fake, 1, 0) == hf.HYF_EINVAL
    assert hf.hyf_linear_w4(cfg, fake, 12, 2560, fake, None, 7968, fake, 1, 0) == hf.HYF_EINVAL
    # no rows: nothing to do
    assert hf.hyf_linear_w4(cfg, fake, 0, *ok[2:]) == hf.HYF_OK
    # the activations must be bf16
    assert hf.hyf_linear_w4(hf.make_config(I.TINY), *ok) == hf.HYF_EUNSUPPORTED


def test_allocation_free_draft_rejects_bad_and_oversized_calls_before_device_work():
    # The same host checks as hyf_draft_block, and HYF_ECAPACITY when the call's workspace would
    # not fit the library's scratch array (64 Qwen3-4B-shaped requests), all before any HIP call.
    cfg = hf.make_config(I.QWEN)
    fake = 1 << 20
    w = hf.HyfWeights(fake, fake, fake, fake, fake)
    R = 64
    assert hf.hyf_workspace_bytes(cfg, R, 8 * R) > hf.HYF_NOALLOC_SCRATCH_BYTES
    cu = list(range(0, 8 * R + 1, 8))
    assert hf.hyf_draft_block_noalloc(cfg, w, fake, R, None, R, fake, cu, fake, fake, 0) == hf.HYF_ECAPACITY
    assert hf.hyf_draft_block_noalloc(cfg, w, fake, 1, None, 1, fake, [0, 9], fake, fake, 0) == hf.HYF_ECAPACITY
    assert hf.hyf_draft_block_noalloc(cfg, w, fake, 1, None, 1, fake, None, fake, fake, 0) == hf.HYF_EINVAL
    assert hf.hyf_draft_block_noalloc(cfg, w, fake + 8, 1, None, 1, None, None, fake, fake, 0) == hf.HYF_EINVAL
    bad_w = hf.HyfWeights(None, fake, fake, fake, fake)
    assert hf.hyf_draft_block_noalloc(cfg, bad_w, fake, 1, None, 1, None, None, fake, fake, 0) == hf.HYF_EINVAL


def test_four_bit_layer_weights_config_and_checks():
    # 4-bit projection weights need bf16 and d_model, nh*head_dim multiples of 128; the codes and
    # scales are checked (not w_in / w_out) before any device work.
    qwen = I.QWEN.replace(weights="w4")
    assert hf.hyf_config_check(hf.make_config(qwen)) == hf.HYF_OK
    assert hf.hyf_config_check(hf.make_config(I.TINY.replace(weights="w4"))) == hf.HYF_EUNSUPPORTED
    odd = I.LayerShape(d_model=192, n_heads=3, head_dim=64, d_state=64, weights="w4")
    assert hf.hyf_config_check(hf.make_config(odd)) == hf.HYF_EUNSUPPORTED
    cfg = hf.make_config(qwen)
    fake = 1 << 20
    dense_only = hf.HyfWeights(fake, fake, fake, fake, fake)
    assert hf.hyf_draft_block(cfg, dense_only, fake, 1, None, 1, None, None, fake, fake, fake, 1 << 30, 0) == \
        hf.HYF_EINVAL
    misaligned = hf.HyfWeights(None, None, fake, fake, fake, fake + 8, fake, fake, fake)
    assert hf.hyf_draft_block(cfg, misaligned, fake, 1, None, 1, None, None, fake, fake, fake, 1 << 30, 0) == \
        hf.HYF_EINVAL
    # the prefill workspace holds the expanded w_in rows from C on
    dense_ws = hf.hyf_workspace_bytes(hf.make_config(I.QWEN), 1, 8192)
    w4_ws = hf.hyf_workspace_bytes(cfg, 1, 8192)
    rows = qwen.n_in - qwen.in_groups["C"][0]
    assert w4_ws >= dense_ws + rows * qwen.d_model * 2 - 256


def test_last_w_memory_layout_keeps_b_and_step_rings():
    # The last-W memory's state blob adds a B ring [W][G*N] (storage dtype) and a raw-step ring
    # [nh][W] (fp32) after the K and V rings; the other memories have none.
    for shape in (I.QWEN, I.TINY):
        lw = shape.replace(memory="lastw")
        L0 = hf.hyf_state_layout_get(hf.make_config(shape))
        L = hf.hyf_state_layout_get(hf.make_config(lw))
        assert L0.b_off == 0 and L0.dt_off == 0
        assert (L.h_off, L.k_off, L.v_off) == (L0.h_off, L0.k_off, L0.v_off)
        es = 2 if shape.dtype == "bf16" else 4
        assert L.b_off == L0.total and L.dt_off >= L.b_off + shape.window * shape.gn * es
        assert L.total >= L.dt_off + shape.n_heads * shape.window * 4 and L.total % 256 == 0
    # per-token outputs are Mamba-2 over the whole history only
    cfg = hf.make_config(I.TINY.replace(memory="lastw"))
    fake = 1 << 20
    w = hf.HyfWeights(fake, fake, fake, fake, fake)
    assert hf.hyf_memory_commit(cfg, w, fake, 1, None, 1, fake, [0, 4], fake, fake, 1 << 30, 0) == \
        hf.HYF_EUNSUPPORTED


def test_full_block_checks_before_device_work():
    # The block's own weights are checked (pointers, alignment, d_ff a multiple of 16 and at least
    # 16, eps in [0, 1]), the workspace covers the layer's and the block's buffers, block_out may
    # not overlap block_in; every rejection comes before any HIP call.
    cfg = hf.make_config(I.QWEN)
    fake = 1 << 20
    w = hf.HyfWeights(fake, fake, fake, fake, fake)
    bw = hf.HyfBlockWeights(fake, fake, fake, fake, 7680, 1e-6)
    lay = hf.hyf_workspace_bytes(cfg, 1, 8)
    blk = hf.hyf_block_workspace_bytes(cfg, bw, 1, 8)
    # layer workspace + 8 commit rows and 8 block rows of x, the layer's output, h, z, gate|up, a, y
    assert blk >= lay + (8 + 8 + 8) * 2560 * 2 + 8 * 2560 * 4 * 2 + 8 * 2560 * 2 + 8 * 2 * 7680 * 4 + 8 * 7680 * 2
    assert hf.hyf_block_workspace_bytes(cfg, bw, 2, 8) > blk
    for bad in (hf.HyfBlockWeights(fake, fake, fake, fake, 7688, 1e-6), hf.HyfBlockWeights(fake, fake, fake, fake, 0, 1e-6),
                hf.HyfBlockWeights(fake, fake, fake, fake, 7680, -1.0)):
        assert hf.hyf_block_workspace_bytes(cfg, bad, 1, 8) == 0
        assert hf.hyf_block_draft(cfg, w, bad, fake, 1, None, 1, None, None, fake, 2 * fake, fake, blk, 0) == hf.HYF_ESHAPE
    nul = hf.HyfBlockWeights(None, fake, fake, fake, 7680, 1e-6)
    mis = hf.HyfBlockWeights(fake, fake, fake + 4, fake, 7680, 1e-6)
    for bad in (nul, mis):
        assert hf.hyf_block_draft(cfg, w, bad, fake, 1, None, 1, None, None, fake, 2 * fake, fake, blk, 0) == hf.HYF_EINVAL
        assert hf.hyf_block_commit(cfg, w, bad, fake, 1, None, 1, fake, [0, 8], fake, blk, 0) == hf.HYF_EINVAL
    # block_out overlapping block_in, a short workspace, too many commit rows
    assert hf.hyf_block_draft(cfg, w, bw, fake, 1, None, 1, None, None, fake, fake + 4096, fake, blk, 0) == hf.HYF_EINVAL
    blk0 = hf.hyf_block_workspace_bytes(cfg, bw, 1, 0)  # a draft without commit rows
    assert hf.hyf_block_draft(cfg, w, bw, fake, 1, None, 1, None, None, fake, 2 * fake, fake, blk0 - 256, 0) == \
        hf.HYF_EWORKSPACE
    assert hf.hyf_block_draft(cfg, w, bw, fake, 1, None, 1, fake, [0, 9], fake, 2 * fake, fake, blk, 0) == \
        hf.HYF_ECAPACITY
    assert hf.hyf_block_commit(cfg, w, bw, fake, 1, None, 1, fake, [0, 8], fake, blk - 256, 0) == hf.HYF_EWORKSPACE
