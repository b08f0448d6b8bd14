"""Python binding of libhyflash (ctypes).

Argument marshalling only: every step of the drafter layer runs in the HIP kernels behind the
C ABI declared in include/hyflash.h.  PyTorch provides device memory and the stream.  If the
built library is missing, importing the binding's entry points raises; there is no CPU path.
"""

from __future__ import annotations

import ctypes
import os
import re

import numpy as np

from .inputs import BF16, F32, LayerShape

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libhyflash.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "hyflash.h")

HYF_OK, HYF_EINVAL, HYF_ESHAPE, HYF_ECAPACITY, HYF_EDTYPE, HYF_EWORKSPACE, HYF_EUNSUPPORTED, HYF_EHIP = range(8)
HYF_F32, HYF_BF16 = 0, 1
HYF_MEM_MAMBA2, HYF_MEM_GDN, HYF_MEM_LASTW = 0, 1, 2
HYF_WEIGHTS_DENSE, HYF_WEIGHTS_W4 = 0, 1
HYF_BLOCK = 8
HYF_MAX_REQUESTS = 128
HYF_NOALLOC_SCRATCH_BYTES = 16 << 20


class HyfConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "d_model", "n_heads", "head_dim", "d_state", "n_groups", "window", "block", "chunk",
        "dtype", "memory", "cross_slot", "weights")]


class HyfWeights(ctypes.Structure):
    _fields_ = [("w_in", ctypes.c_void_p), ("w_out", ctypes.c_void_p), ("a_log", ctypes.c_void_p),
                ("dt_bias", ctypes.c_void_p), ("d_skip", ctypes.c_void_p), ("w_in_q", ctypes.c_void_p),
                ("w_in_s", ctypes.c_void_p), ("w_out_q", ctypes.c_void_p), ("w_out_s", ctypes.c_void_p)]


class HyfStateLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in ("count_off", "h_off", "k_off", "v_off", "total", "b_off", "dt_off")]


class HyfBlockWeights(ctypes.Structure):
    _fields_ = [("norm1", ctypes.c_void_p), ("norm2", ctypes.c_void_p), ("w_gate_up", ctypes.c_void_p),
                ("w_down", ctypes.c_void_p), ("d_ff", ctypes.c_int32), ("eps", ctypes.c_float)]


class HyfError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        super().__init__(f"{what}: status {status} ({status_str(status)})")
        self.status = status


_lib = None
_P = ctypes.POINTER
_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_SIGS = {
    "hyf_abi_version": (ctypes.c_int, []),
    "hyf_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "hyf_config_check": (ctypes.c_int, [_P(HyfConfig)]),
    "hyf_n_in": (_i64, [_P(HyfConfig)]),
    "hyf_state_layout_get": (ctypes.c_int, [_P(HyfConfig), _P(HyfStateLayout)]),
    "hyf_state_bytes": (_sz, [_P(HyfConfig)]),
    "hyf_workspace_bytes": (_sz, [_P(HyfConfig), _i32, _i64, _i32]),
    "hyf_ssd_scan_workspace_bytes": (_sz, [_P(HyfConfig), _i64, _i32]),
    "hyf_state_reset": (ctypes.c_int, [_P(HyfConfig), _vp, _i32, _vp, _i32, _vp]),
    "hyf_memory_commit": (ctypes.c_int, [_P(HyfConfig), _P(HyfWeights), _vp, _i32, _vp, _i32, _vp, _vp, _vp,
                                         _vp, _sz, _vp]),
    "hyf_draft_block": (ctypes.c_int, [_P(HyfConfig), _P(HyfWeights), _vp, _i32, _vp, _i32, _vp, _vp, _vp, _vp,
                                       _vp, _sz, _vp]),
    "hyf_draft_block_noalloc": (ctypes.c_int, [_P(HyfConfig), _P(HyfWeights), _vp, _i32, _vp, _i32, _vp, _vp, _vp,
                                               _vp, _vp]),
    "hyf_linear": (ctypes.c_int, [_P(HyfConfig), _vp, _i64, _i32, _vp, _i32, _vp, _i32, _vp]),
    "hyf_linear_w4": (ctypes.c_int, [_P(HyfConfig), _vp, _i64, _i32, _vp, _vp, _i32, _vp, _i32, _vp]),
    "hyf_ssd_scan": (ctypes.c_int, [_P(HyfConfig), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _sz,
                                    _vp]),
    "hyf_draft_block_dev": (ctypes.c_int, [_P(HyfConfig), _P(HyfWeights), _vp, _i32, _vp, _i32, _vp, _vp, _vp,
                                           _vp, _vp, _sz, _vp]),
    "hyf_block_workspace_bytes": (_sz, [_P(HyfConfig), _P(HyfBlockWeights), _i32, _i64]),
    "hyf_block_commit": (ctypes.c_int, [_P(HyfConfig), _P(HyfWeights), _P(HyfBlockWeights), _vp, _i32, _vp, _i32,
                                        _vp, _vp, _vp, _sz, _vp]),
    "hyf_block_draft": (ctypes.c_int, [_P(HyfConfig), _P(HyfWeights), _P(HyfBlockWeights), _vp, _i32, _vp, _i32,
                                       _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
}


def lib():
    """The loaded libhyflash; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libhyflash is not built ({LIB_PATH}); run python -m hybrid_ssm_local_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def header_functions() -> list[str]:
    """Names of the functions include/hyflash.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(hyf_\w+)\s*\(", text, re.M)))


def status_str(st: int) -> str:
    return lib().hyf_status_str(st).decode()


def check(st: int, what: str = "libhyflash") -> None:
    if st != HYF_OK:
        raise HyfError(st, what)


def make_config(shape: LayerShape, memory: int | None = None) -> HyfConfig:
    if memory is None:
        memory = {"gdn": HYF_MEM_GDN, "lastw": HYF_MEM_LASTW}.get(shape.memory, HYF_MEM_MAMBA2)
    return HyfConfig(shape.d_model, shape.n_heads, shape.head_dim, shape.d_state, shape.n_groups, shape.window,
                     shape.block, shape.chunk, HYF_BF16 if shape.dtype == BF16 else HYF_F32, memory,
                     shape.cross_slot, HYF_WEIGHTS_W4 if shape.weights == "w4" else HYF_WEIGHTS_DENSE)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return ctypes.c_void_p(t)
    return ctypes.c_void_p(t.data_ptr())


def _host_i32(a):
    if a is None:
        return None, None
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return arr, arr.ctypes.data_as(ctypes.c_void_p)


def _host_i64(a):
    if a is None:
        return None, None
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.int64))
    return arr, arr.ctypes.data_as(ctypes.c_void_p)


def _stream(stream):
    if stream is None:
        import torch

        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


# ------------------------------------------------------------------ the C entry points, same names


def hyf_abi_version() -> int:
    return lib().hyf_abi_version()


def hyf_config_check(cfg: HyfConfig) -> int:
    return lib().hyf_config_check(ctypes.byref(cfg))


def hyf_n_in(cfg: HyfConfig) -> int:
    return lib().hyf_n_in(ctypes.byref(cfg))


def hyf_state_layout_get(cfg: HyfConfig) -> HyfStateLayout:
    out = HyfStateLayout()
    check(lib().hyf_state_layout_get(ctypes.byref(cfg), ctypes.byref(out)), "hyf_state_layout_get")
    return out


def hyf_state_bytes(cfg: HyfConfig) -> int:
    return lib().hyf_state_bytes(ctypes.byref(cfg))


def hyf_workspace_bytes(cfg: HyfConfig, max_requests: int, max_rows: int, with_y: int = 0) -> int:
    return lib().hyf_workspace_bytes(ctypes.byref(cfg), max_requests, max_rows, int(with_y))


def hyf_ssd_scan_workspace_bytes(cfg: HyfConfig, T: int, with_y: int = 0) -> int:
    return lib().hyf_ssd_scan_workspace_bytes(ctypes.byref(cfg), T, int(with_y))


def hyf_state_reset(cfg, pool, pool_slots, slots, n_req, stream=None) -> int:
    _s, sp = _host_i32(slots)
    return lib().hyf_state_reset(ctypes.byref(cfg), _ptr(pool), pool_slots, sp, n_req, _stream(stream))


def hyf_memory_commit(cfg, w: HyfWeights, pool, pool_slots, slots, n_req, feats, cu_rows, y, ws, ws_bytes,
                      stream=None) -> int:
    _s, sp = _host_i32(slots)
    _c, cp = _host_i64(cu_rows)
    return lib().hyf_memory_commit(ctypes.byref(cfg), ctypes.byref(w), _ptr(pool), pool_slots, sp, n_req,
                                   _ptr(feats), cp, _ptr(y), _ptr(ws), ws_bytes, _stream(stream))


def hyf_draft_block(cfg, w: HyfWeights, pool, pool_slots, slots, n_req, commit_feats, cu_commit, block_in,
                    block_out, ws, ws_bytes, stream=None) -> int:
    _s, sp = _host_i32(slots)
    _c, cp = _host_i64(cu_commit)
    return lib().hyf_draft_block(ctypes.byref(cfg), ctypes.byref(w), _ptr(pool), pool_slots, sp, n_req,
                                 _ptr(commit_feats), cp, _ptr(block_in), _ptr(block_out), _ptr(ws), ws_bytes,
                                 _stream(stream))


def hyf_draft_block_dev(cfg, w: HyfWeights, pool, pool_slots, slots, n_req, commit_feats, commit_rows, block_in,
                        block_out, ws, ws_bytes, stream=None) -> int:
    """commit_feats [n_req*HYF_BLOCK][d] and commit_rows int32 [n_req] are device tensors (or None)."""
    _s, sp = _host_i32(slots)
    return lib().hyf_draft_block_dev(ctypes.byref(cfg), ctypes.byref(w), _ptr(pool), pool_slots, sp, n_req,
                                     _ptr(commit_feats), _ptr(commit_rows), _ptr(block_in), _ptr(block_out), _ptr(ws),
                                     ws_bytes, _stream(stream))


def hyf_draft_block_noalloc(cfg, w: HyfWeights, pool, pool_slots, slots, n_req, commit_feats, cu_commit, block_in,
                            block_out, stream=None) -> int:
    _s, sp = _host_i32(slots)
    _c, cp = _host_i64(cu_commit)
    return lib().hyf_draft_block_noalloc(ctypes.byref(cfg), ctypes.byref(w), _ptr(pool), pool_slots, sp, n_req,
                                         _ptr(commit_feats), cp, _ptr(block_in), _ptr(block_out), _stream(stream))


def hyf_block_workspace_bytes(cfg, bw: HyfBlockWeights, max_requests: int, max_rows: int) -> int:
    return lib().hyf_block_workspace_bytes(ctypes.byref(cfg), ctypes.byref(bw), max_requests, max_rows)


def hyf_block_commit(cfg, w: HyfWeights, bw: HyfBlockWeights, pool, pool_slots, slots, n_req, feats, cu_rows, ws,
                     ws_bytes, stream=None) -> int:
    _s, sp = _host_i32(slots)
    _c, cp = _host_i64(cu_rows)
    return lib().hyf_block_commit(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(bw), _ptr(pool), pool_slots, sp,
                                  n_req, _ptr(feats), cp, _ptr(ws), ws_bytes, _stream(stream))


def hyf_block_draft(cfg, w: HyfWeights, bw: HyfBlockWeights, pool, pool_slots, slots, n_req, commit_feats,
                    cu_commit, block_in, block_out, ws, ws_bytes, stream=None) -> int:
    _s, sp = _host_i32(slots)
    _c, cp = _host_i64(cu_commit)
    return lib().hyf_block_draft(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(bw), _ptr(pool), pool_slots, sp,
                                 n_req, _ptr(commit_feats), cp, _ptr(block_in), _ptr(block_out), _ptr(ws), ws_bytes,
                                 _stream(stream))


def hyf_linear(cfg, X, M, K, W, Nout, out, out_f32, stream=None) -> int:
    return lib().hyf_linear(ctypes.byref(cfg), _ptr(X), M, K, _ptr(W), Nout, _ptr(out), out_f32, _stream(stream))


def hyf_linear_w4(cfg, X, M, K, Wq, scales, Nout, out, out_f32, stream=None) -> int:
    return lib().hyf_linear_w4(ctypes.byref(cfg), _ptr(X), M, K, _ptr(Wq), _ptr(scales), Nout, _ptr(out), out_f32,
                               _stream(stream))


def hyf_ssd_scan(cfg, x, B, C, dt_raw, a_log, dt_bias, d_skip, H, y, T, ws, ws_bytes, stream=None) -> int:
    return lib().hyf_ssd_scan(ctypes.byref(cfg), _ptr(x), _ptr(B), _ptr(C), _ptr(dt_raw), _ptr(a_log),
                              _ptr(dt_bias), _ptr(d_skip), _ptr(H), _ptr(y), T, _ptr(ws), ws_bytes,
                              _stream(stream))


# ------------------------------------------------------------------ device-memory owner


HYF_TBLK = 128


def time_blocked(a, T: int, pad=0.0) -> np.ndarray:
    """[T][features...] -> [ceil(T/HYF_TBLK)][F][HYF_TBLK], the layout hyf_ssd_scan reads.

    Tokens past T in the last block are filled with `pad`."""
    f = np.asarray(a, np.float32).reshape(T, -1)
    F = f.shape[1]
    nb = (T + HYF_TBLK - 1) // HYF_TBLK
    out = np.full((nb * HYF_TBLK, F), pad, dtype=np.float32)
    out[:T] = f
    return np.ascontiguousarray(out.reshape(nb, HYF_TBLK, F).transpose(0, 2, 1))


def time_tiled(a, T: int, elem_bytes: int, pad=0.0) -> np.ndarray:
    """[T][F] -> the tiled time-blocked layout hyf_ssd_scan reads for x and B (F a multiple of 16).

    Blocks of HYF_TBLK tokens; inside a block, feature f and token t sit at element
    (((f // 16) * NJ + t // KT) * 64 + ((t % KT) // VN) * 16 + f % 16) * VN + t % VN, with
    VN = 16 // elem_bytes and KT = 4 * VN, NJ = HYF_TBLK // KT.  Returned as [blocks][F][HYF_TBLK]
    (the same size as time_blocked; only the order inside a block differs)."""
    blk = time_blocked(a, T, pad)
    nb, F, _ = blk.shape
    if F % 16:
        raise ValueError("tiled layout needs a multiple of 16 features")
    vn = 16 // elem_bytes
    kt = 4 * vn
    t = blk.reshape(nb, F // 16, 16, HYF_TBLK // kt, 4, vn).transpose(0, 1, 3, 4, 2, 5)
    return np.ascontiguousarray(t).reshape(nb, F, HYF_TBLK)


def elem_bytes(shape: LayerShape) -> int:
    return 2 if shape.dtype == BF16 else 4


def torch_dtype(shape: LayerShape):
    import torch

    return torch.bfloat16 if shape.dtype == BF16 else torch.float32


def to_device(a, shape: LayerShape, device="cuda", storage=True):
    """numpy float32 -> device tensor in the storage dtype (values are already storage-exact)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device=device, dtype=torch_dtype(shape) if storage else torch.float32)


class DrafterLayer:
    """Owns one layer's device weights, a state pool and a workspace; forwards to the C ABI."""

    def __init__(self, shape: LayerShape, weights: dict, pool_slots: int = 1, max_requests: int = 1,
                 max_rows: int = 8, with_y: bool = False, device: str = "cuda"):
        import torch

        self.shape, self.device = shape, device
        self.cfg = make_config(shape)
        check(hyf_config_check(self.cfg), "hyf_config_check")
        self.a_log = to_device(weights["a_log"], shape, device, storage=False)
        self.dt_bias = to_device(weights["dt_bias"], shape, device, storage=False)
        self.d_skip = to_device(weights["d_skip"], shape, device, storage=False)
        if shape.weights == "w4":
            # 4-bit weights: codes [out][in/2] uint8, scales [out][in/128] fp32
            q = {k: torch.from_numpy(np.ascontiguousarray(weights[k])).to(device)
                 for k in ("w_in_q", "w_in_s", "w_out_q", "w_out_s")}
            self.w4 = q
            self.w = HyfWeights(None, None, self.a_log.data_ptr(), self.dt_bias.data_ptr(), self.d_skip.data_ptr(),
                                q["w_in_q"].data_ptr(), q["w_in_s"].data_ptr(), q["w_out_q"].data_ptr(),
                                q["w_out_s"].data_ptr())
        else:
            self.w_in = to_device(weights["w_in"], shape, device)
            self.w_out = to_device(weights["w_out"], shape, device)
            self.w = HyfWeights(self.w_in.data_ptr(), self.w_out.data_ptr(), self.a_log.data_ptr(),
                                self.dt_bias.data_ptr(), self.d_skip.data_ptr())
        self.pool_slots = pool_slots
        self.state_bytes = hyf_state_bytes(self.cfg)
        self.layout = hyf_state_layout_get(self.cfg)
        self.pool = torch.zeros(pool_slots * self.state_bytes, dtype=torch.uint8, device=device)
        self.ws_bytes = hyf_workspace_bytes(self.cfg, max_requests, max_rows, with_y)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)

    def reset(self, slots=None, n_req=None, stream=None):
        n = n_req if n_req is not None else (len(slots) if slots is not None else self.pool_slots)
        check(hyf_state_reset(self.cfg, self.pool, self.pool_slots, slots, n, stream), "hyf_state_reset")

    def commit(self, feats, cu_rows, slots=None, y=None, stream=None):
        """Commit rows; y (optional, [rows][nh][P] storage dtype) receives the per-token outputs
        (needs a layer built with with_y=True)."""
        n_req = len(cu_rows) - 1
        check(hyf_memory_commit(self.cfg, self.w, self.pool, self.pool_slots, slots, n_req, feats, cu_rows, y,
                                self.ws, self.ws_bytes, stream), "hyf_memory_commit")

    def draft(self, block_in, block_out, commit_feats=None, cu_commit=None, slots=None, stream=None):
        n_req = block_in.shape[0] // HYF_BLOCK if block_in.dim() == 2 else block_in.shape[0]
        check(hyf_draft_block(self.cfg, self.w, self.pool, self.pool_slots, slots, n_req, commit_feats, cu_commit,
                              block_in, block_out, self.ws, self.ws_bytes, stream), "hyf_draft_block")

    def state(self, slot: int = 0) -> dict:
        """Views of one state blob: count, H [nh][P][N] fp32, K and V rings [nh][W][P]."""
        import torch

        sh, L = self.shape, self.layout
        base = slot * self.state_bytes
        blob = self.pool[base: base + self.state_bytes]
        nh, P, N, W = sh.n_heads, sh.head_dim, sh.d_state, sh.window
        es = 2 if sh.dtype == BF16 else 4
        count = blob[L.count_off: L.count_off + 8].view(torch.int64)
        H = blob[L.h_off: L.h_off + nh * P * N * 4].view(torch.float32).view(nh, P, N)
        K = blob[L.k_off: L.k_off + nh * W * P * es].view(torch_dtype(sh)).view(nh, W, P)
        V = blob[L.v_off: L.v_off + nh * W * P * es].view(torch_dtype(sh)).view(nh, W, P)
        out = dict(count=count, H=H, K=K, V=V, blob=blob)
        if L.b_off:
            out["Bring"] = blob[L.b_off: L.b_off + W * sh.gn * es].view(torch_dtype(sh)).view(W, sh.gn)
            out["DTring"] = blob[L.dt_off: L.dt_off + nh * W * 4].view(torch.float32).view(nh, W)
        return out


class DrafterBlock:
    """The full drafter block around one layer: the layer's weights and state (a DrafterLayer)
    plus the block's norms and MLP; forwards to hyf_block_commit / hyf_block_draft."""

    def __init__(self, shape: LayerShape, weights: dict, block_weights: dict, pool_slots: int = 1,
                 max_requests: int = 1, max_rows: int = 8, device: str = "cuda"):
        import torch

        self.layer = DrafterLayer(shape, weights, pool_slots, max_requests, max_rows, device=device)
        self.shape = shape
        bwt = block_weights
        self.norm1 = torch.from_numpy(np.asarray(bwt["norm1"], np.float32)).to(device)
        self.norm2 = torch.from_numpy(np.asarray(bwt["norm2"], np.float32)).to(device)
        self.w_gate_up = to_device(np.concatenate([bwt["w_gate"], bwt["w_up"]], axis=0), shape, device)
        self.w_down = to_device(bwt["w_down"], shape, device)
        self.bw = HyfBlockWeights(self.norm1.data_ptr(), self.norm2.data_ptr(), self.w_gate_up.data_ptr(),
                                  self.w_down.data_ptr(), int(np.asarray(bwt["w_gate"]).shape[0]), float(bwt["eps"]))
        self.ws_bytes = hyf_block_workspace_bytes(self.layer.cfg, self.bw, max_requests, max_rows)
        if self.ws_bytes == 0:
            raise HyfError(1, "hyf_block_workspace_bytes")
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)

    def reset(self, slots=None, n_req=None, stream=None):
        self.layer.reset(slots, n_req, stream)

    def commit(self, feats, cu_rows, slots=None, stream=None):
        n_req = len(cu_rows) - 1
        L = self.layer
        check(hyf_block_commit(L.cfg, L.w, self.bw, L.pool, L.pool_slots, slots, n_req, feats, cu_rows, self.ws,
                               self.ws_bytes, stream), "hyf_block_commit")

    def draft(self, block_in, block_out, commit_feats=None, cu_commit=None, slots=None, stream=None):
        n_req = block_in.shape[0] // HYF_BLOCK if block_in.dim() == 2 else block_in.shape[0]
        L = self.layer
        check(hyf_block_draft(L.cfg, L.w, self.bw, L.pool, L.pool_slots, slots, n_req, commit_feats, cu_commit,
                              block_in, block_out, self.ws, self.ws_bytes, stream), "hyf_block_draft")

    def state(self, slot: int = 0) -> dict:
        return self.layer.state(slot)
