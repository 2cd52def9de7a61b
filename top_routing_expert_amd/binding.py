"""Thin Python binding of libmoe_mi355x.so (include/moe.h).

Argument marshalling only: torch tensors are turned into device pointers and
the current HIP stream, and the C functions of the same names are called.
Every step of the MoE path runs in the library's HIP kernels; there is no
Python or CPU fallback, and a missing library raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

from .configs import MoEShape

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_mi355x.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EHIP, MOE_ESCRATCH = 0, -1, -2, -3, -4
MOE_F32, MOE_BF16 = 0, 1
ENTRY = {"route": 1, "permute": 2, "ffn": 3, "combine": 4, "layer": 5, "route_stats": 6,
         "ffn_backward": 7, "route_backward": 8}

CONFIG_FIELDS = ("T", "d", "E", "k", "f", "n_group", "topk_group", "presel", "renorm",
                 "ep_ranks", "dtype")
LAYER_BUF_FIELDS = ("logits", "topk_idx", "topk_w", "expert_offsets", "rank_offsets", "slot_of",
                    "src_of", "x_perm", "h", "y_perm")

# every function include/moe.h declares
EXPORTS = ("moe_strerror", "moe_validate", "moe_workspace_bytes", "moe_route", "moe_permute",
           "moe_ffn_gate_up", "moe_ffn_down", "moe_grouped_ffn", "moe_combine", "moe_layer_fwd",
           "moe_packed_weight_bytes", "moe_pack_weights", "moe_ffn_gate_up_packed",
           "moe_ffn_gate_up_packed_gather", "moe_ffn_down_packed", "moe_layer_fwd_packed",
           "moe_route_stats", "moe_quantize_fp8", "moe_dequantize_fp8", "moe_combine_backward",
           "moe_ffn_backward", "moe_route_backward", "moe_unpermute_backward",
           "moe_ffn_gate_up_packed_train", "moe_packed_weight_bytes_backward",
           "moe_pack_weights_backward", "moe_permute_noalloc", "moe_noalloc_scratch_bytes",
           "moe_fp8_weight_bytes", "moe_pack_weights_fp8", "moe_ffn_gate_up_fp8_gather",
           "moe_layer_fwd_packed_waved")


class MoEConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in CONFIG_FIELDS]


class MoELayerBufs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in LAYER_BUF_FIELDS]


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status} ({strerror(status)})")


_lib = None


def lib() -> ctypes.CDLL:
    """Loads the in-tree library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        cfgp = ctypes.POINTER(MoEConfig)
        L.moe_strerror.restype = ctypes.c_char_p
        L.moe_strerror.argtypes = [i32]
        L.moe_validate.argtypes = [cfgp]
        L.moe_workspace_bytes.argtypes = [cfgp, i32, ctypes.POINTER(sz)]
        L.moe_route.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_permute.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_permute_noalloc.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.moe_noalloc_scratch_bytes.argtypes = []
        L.moe_fp8_weight_bytes.argtypes = [cfgp, ctypes.POINTER(sz)]
        L.moe_pack_weights_fp8.argtypes = [cfgp, vp, vp, vp, vp]
        L.moe_ffn_gate_up_fp8_gather.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp]
        L.moe_ffn_gate_up.argtypes = [cfgp, vp, vp, vp, vp, vp, vp]
        L.moe_ffn_down.argtypes = [cfgp, vp, vp, vp, vp, vp]
        L.moe_grouped_ffn.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.moe_combine.argtypes = [cfgp, vp, vp, vp, vp, vp]
        L.moe_layer_fwd.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp,
                                    ctypes.POINTER(MoELayerBufs), vp, sz, vp]
        L.moe_packed_weight_bytes.argtypes = [cfgp, ctypes.POINTER(sz), ctypes.POINTER(sz)]
        L.moe_pack_weights.argtypes = [cfgp, vp, vp, vp, vp, vp, vp]
        L.moe_ffn_gate_up_packed.argtypes = [cfgp, vp, vp, vp, vp, vp]
        L.moe_ffn_gate_up_packed_gather.argtypes = [cfgp, vp, vp, vp, vp, vp, vp]
        L.moe_route_stats.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_quantize_fp8.argtypes = [cfgp, vp, vp, vp, vp]
        L.moe_dequantize_fp8.argtypes = [cfgp, vp, vp, vp, vp, vp]
        L.moe_ffn_down_packed.argtypes = [cfgp, vp, vp, vp, vp, vp]
        L.moe_combine_backward.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp]
        L.moe_ffn_backward.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                       vp, vp, sz, vp]
        L.moe_packed_weight_bytes_backward.argtypes = [cfgp, ctypes.POINTER(sz),
                                                       ctypes.POINTER(sz)]
        L.moe_pack_weights_backward.argtypes = [cfgp, vp, vp, vp, vp, vp, vp]
        L.moe_ffn_gate_up_packed_train.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.moe_route_backward.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                         vp]
        L.moe_unpermute_backward.argtypes = [cfgp, vp, vp, vp, vp, vp]
        L.moe_layer_fwd_packed.argtypes = [cfgp, vp, vp, vp, vp, vp, vp,
                                           ctypes.POINTER(MoELayerBufs), vp, sz, vp]
        L.moe_layer_fwd_packed_waved.argtypes = [cfgp, vp, vp, vp, vp, vp, vp,
                                                 ctypes.POINTER(MoELayerBufs), vp, sz, i32, vp, vp]
        for name in EXPORTS[1:]:
            getattr(L, name).restype = i32
        L.moe_noalloc_scratch_bytes.restype = sz
        _lib = L
    return _lib


def strerror(status: int) -> str:
    return lib().moe_strerror(int(status)).decode()


def config(shape: MoEShape | None = None, **over) -> MoEConfig:
    """MoEConfig from a workload shape (or keyword fields)."""
    vals = {n: 0 for n in CONFIG_FIELDS}
    vals.update(n_group=1, topk_group=1, renorm=1, ep_ranks=1, dtype=MOE_BF16)
    if shape is not None:
        for n in CONFIG_FIELDS[:-1]:
            vals[n] = getattr(shape, n)
        vals["dtype"] = MOE_BF16 if shape.dtype == "bf16" else MOE_F32
    vals.update(over)
    return MoEConfig(**vals)


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("tensor arguments must live in device memory")
    if not t.is_contiguous():
        raise ValueError("tensor arguments must be contiguous (dense row-major)")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ws(ws):
    if ws is None:
        return None, 0
    return _ptr(ws), ws.numel() * ws.element_size()


def _check(fn: str, status: int) -> None:
    if status != MOE_OK:
        raise MoEError(fn, status)


def validate(cfg: MoEConfig) -> int:
    return lib().moe_validate(ctypes.byref(cfg))


def workspace_bytes(cfg: MoEConfig, entry: str) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_workspace_bytes", lib().moe_workspace_bytes(ctypes.byref(cfg), ENTRY[entry],
                                                            ctypes.byref(n)))
    return n.value


def workspace(cfg: MoEConfig, entry: str, device="cuda") -> torch.Tensor | None:
    """A caller-owned device workspace of the size the library asks for."""
    n = workspace_bytes(cfg, entry)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def moe_route(cfg, x, w_router, bias, logits, topk_idx, topk_w, ws=None, stream=None):
    wp, wn = _ws(ws)
    _check("moe_route", lib().moe_route(ctypes.byref(cfg), _ptr(x), _ptr(w_router), _ptr(bias),
                                        _ptr(logits), _ptr(topk_idx), _ptr(topk_w), wp, wn,
                                        _stream(stream)))


def moe_permute(cfg, x, topk_idx, expert_offsets, rank_offsets, slot_of, src_of, x_perm,
                ws=None, stream=None):
    wp, wn = _ws(ws)
    _check("moe_permute", lib().moe_permute(ctypes.byref(cfg), _ptr(x), _ptr(topk_idx),
                                            _ptr(expert_offsets), _ptr(rank_offsets),
                                            _ptr(slot_of), _ptr(src_of), _ptr(x_perm), wp, wn,
                                            _stream(stream)))


def moe_permute_noalloc(cfg, x, topk_idx, expert_offsets, rank_offsets, slot_of, src_of, x_perm,
                        stream=None):
    _check("moe_permute_noalloc", lib().moe_permute_noalloc(
        ctypes.byref(cfg), _ptr(x), _ptr(topk_idx), _ptr(expert_offsets), _ptr(rank_offsets),
        _ptr(slot_of), _ptr(src_of), _ptr(x_perm), _stream(stream)))


def noalloc_scratch_bytes() -> int:
    return int(lib().moe_noalloc_scratch_bytes())


def moe_ffn_gate_up(cfg, x_perm, expert_offsets, w_gate, w_up, h, stream=None):
    _check("moe_ffn_gate_up", lib().moe_ffn_gate_up(ctypes.byref(cfg), _ptr(x_perm),
                                                    _ptr(expert_offsets), _ptr(w_gate), _ptr(w_up),
                                                    _ptr(h), _stream(stream)))


def moe_ffn_down(cfg, h, expert_offsets, w_down, y_perm, stream=None):
    _check("moe_ffn_down", lib().moe_ffn_down(ctypes.byref(cfg), _ptr(h), _ptr(expert_offsets),
                                              _ptr(w_down), _ptr(y_perm), _stream(stream)))


def moe_grouped_ffn(cfg, x_perm, expert_offsets, w_gate, w_up, w_down, h, y_perm, stream=None):
    _check("moe_grouped_ffn", lib().moe_grouped_ffn(ctypes.byref(cfg), _ptr(x_perm),
                                                    _ptr(expert_offsets), _ptr(w_gate), _ptr(w_up),
                                                    _ptr(w_down), _ptr(h), _ptr(y_perm),
                                                    _stream(stream)))


def moe_combine(cfg, y_perm, slot_of, topk_w, out, stream=None):
    _check("moe_combine", lib().moe_combine(ctypes.byref(cfg), _ptr(y_perm), _ptr(slot_of),
                                            _ptr(topk_w), _ptr(out), _stream(stream)))


def moe_layer_fwd(cfg, x, w_router, bias, w_gate, w_up, w_down, out, bufs: dict | None = None,
                  ws=None, stream=None):
    b = None
    if bufs:
        b = MoELayerBufs(**{n: _ptr(bufs.get(n)) for n in LAYER_BUF_FIELDS})
    wp, wn = _ws(ws)
    _check("moe_layer_fwd", lib().moe_layer_fwd(ctypes.byref(cfg), _ptr(x), _ptr(w_router),
                                                _ptr(bias), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                                                _ptr(out), ctypes.byref(b) if b else None, wp, wn,
                                                _stream(stream)))


def packed_weight_bytes(cfg) -> tuple[int, int]:
    gu, dn = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check("moe_packed_weight_bytes", lib().moe_packed_weight_bytes(ctypes.byref(cfg),
                                                                    ctypes.byref(gu),
                                                                    ctypes.byref(dn)))
    return gu.value, dn.value


def moe_pack_weights(cfg, w_gate, w_up, w_down, packed_gate_up, packed_down, stream=None):
    _check("moe_pack_weights", lib().moe_pack_weights(ctypes.byref(cfg), _ptr(w_gate), _ptr(w_up),
                                                      _ptr(w_down), _ptr(packed_gate_up),
                                                      _ptr(packed_down), _stream(stream)))


def pack_weights(cfg, w_gate, w_up, w_down, device="cuda", stream=None):
    """Allocates the packed images (uint8 device tensors) and fills them; an
    image whose weights are None is neither allocated nor written (None)."""
    gu, dn = packed_weight_bytes(cfg)
    pgu = torch.empty(gu, dtype=torch.uint8, device=device) if w_gate is not None else None
    pd = torch.empty(dn, dtype=torch.uint8, device=device) if w_down is not None else None
    moe_pack_weights(cfg, w_gate, w_up, w_down, pgu, pd, stream)
    return pgu, pd


def moe_ffn_gate_up_packed(cfg, x_perm, expert_offsets, packed_gate_up, h, stream=None):
    _check("moe_ffn_gate_up_packed",
           lib().moe_ffn_gate_up_packed(ctypes.byref(cfg), _ptr(x_perm), _ptr(expert_offsets),
                                        _ptr(packed_gate_up), _ptr(h), _stream(stream)))


def moe_ffn_gate_up_packed_gather(cfg, x, src_of, expert_offsets, packed_gate_up, h, stream=None):
    _check("moe_ffn_gate_up_packed_gather",
           lib().moe_ffn_gate_up_packed_gather(ctypes.byref(cfg), _ptr(x), _ptr(src_of),
                                               _ptr(expert_offsets), _ptr(packed_gate_up), _ptr(h),
                                               _stream(stream)))


def fp8_weight_bytes(cfg) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_fp8_weight_bytes", lib().moe_fp8_weight_bytes(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def moe_pack_weights_fp8(cfg, w_gate, w_up, image, stream=None):
    _check("moe_pack_weights_fp8", lib().moe_pack_weights_fp8(
        ctypes.byref(cfg), _ptr(w_gate), _ptr(w_up), _ptr(image), _stream(stream)))


def pack_weights_fp8(cfg, w_gate, w_up, device="cuda", stream=None):
    """The FP8 gate/up image of the weights (a load-time layout)."""
    image = torch.empty(fp8_weight_bytes(cfg), dtype=torch.uint8, device=device)
    moe_pack_weights_fp8(cfg, w_gate, w_up, image, stream)
    return image


def moe_ffn_gate_up_fp8_gather(cfg, x_codes, scale_zero, src_of, expert_offsets, image, h,
                               stream=None):
    _check("moe_ffn_gate_up_fp8_gather", lib().moe_ffn_gate_up_fp8_gather(
        ctypes.byref(cfg), _ptr(x_codes), _ptr(scale_zero), _ptr(src_of), _ptr(expert_offsets),
        _ptr(image), _ptr(h), _stream(stream)))


def moe_route_stats(cfg, logits, bias, expert_offsets, rank_offsets, hist, rank_load, stats,
                    ws=None, stream=None):
    wp, wn = _ws(ws)
    _check("moe_route_stats",
           lib().moe_route_stats(ctypes.byref(cfg), _ptr(logits), _ptr(bias), _ptr(expert_offsets),
                                 _ptr(rank_offsets), _ptr(hist), _ptr(rank_load), _ptr(stats), wp,
                                 wn, _stream(stream)))


def moe_quantize_fp8(cfg, x, codes, scale_zero, stream=None):
    _check("moe_quantize_fp8", lib().moe_quantize_fp8(ctypes.byref(cfg), _ptr(x), _ptr(codes),
                                                      _ptr(scale_zero), _stream(stream)))


def moe_dequantize_fp8(cfg, codes, src_of, scale_zero, x_perm, stream=None):
    _check("moe_dequantize_fp8",
           lib().moe_dequantize_fp8(ctypes.byref(cfg), _ptr(codes), _ptr(src_of), _ptr(scale_zero),
                                    _ptr(x_perm), _stream(stream)))


def moe_combine_backward(cfg, d_out, y_perm, slot_of, topk_w, d_y_perm, d_topk_w, stream=None):
    _check("moe_combine_backward",
           lib().moe_combine_backward(ctypes.byref(cfg), _ptr(d_out), _ptr(y_perm), _ptr(slot_of),
                                      _ptr(topk_w), _ptr(d_y_perm), _ptr(d_topk_w),
                                      _stream(stream)))


def moe_ffn_gate_up_packed_train(cfg, act, src_of, expert_offsets, packed_gate_up, h, a, u,
                                 stream=None):
    _check("moe_ffn_gate_up_packed_train",
           lib().moe_ffn_gate_up_packed_train(ctypes.byref(cfg), _ptr(act), _ptr(src_of),
                                              _ptr(expert_offsets), _ptr(packed_gate_up), _ptr(h),
                                              _ptr(a), _ptr(u), _stream(stream)))


def moe_ffn_backward(cfg, x_perm, expert_offsets, w_gate, w_up, w_down, d_y_perm, d_x_perm,
                     d_w_gate, d_w_up, d_w_down, ws=None, stream=None, a=None, u=None,
                     packed_dh=None, packed_dx=None):
    wp, wn = _ws(ws)
    _check("moe_ffn_backward",
           lib().moe_ffn_backward(ctypes.byref(cfg), _ptr(x_perm), _ptr(expert_offsets),
                                  _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(a), _ptr(u),
                                  _ptr(packed_dh), _ptr(packed_dx), _ptr(d_y_perm),
                                  _ptr(d_x_perm), _ptr(d_w_gate), _ptr(d_w_up), _ptr(d_w_down),
                                  wp, wn, _stream(stream)))


def packed_weight_bytes_backward(cfg) -> tuple[int, int]:
    dh, dx = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check("moe_packed_weight_bytes_backward",
           lib().moe_packed_weight_bytes_backward(ctypes.byref(cfg), ctypes.byref(dh),
                                                  ctypes.byref(dx)))
    return dh.value, dx.value


def moe_pack_weights_backward(cfg, w_gate, w_up, w_down, packed_dh, packed_dx, stream=None):
    _check("moe_pack_weights_backward",
           lib().moe_pack_weights_backward(ctypes.byref(cfg), _ptr(w_gate), _ptr(w_up),
                                           _ptr(w_down), _ptr(packed_dh), _ptr(packed_dx),
                                           _stream(stream)))


def pack_weights_backward(cfg, w_gate, w_up, w_down, device="cuda", stream=None):
    """Allocates and fills the two transposed images the FFN backward's
    activation-gradient products can run on (uint8 device tensors)."""
    dh, dx = packed_weight_bytes_backward(cfg)
    pdh = torch.empty(dh, dtype=torch.uint8, device=device)
    pdx = torch.empty(dx, dtype=torch.uint8, device=device)
    moe_pack_weights_backward(cfg, w_gate, w_up, w_down, pdh, pdx, stream)
    return pdh, pdx


def moe_route_backward(cfg, x, w_router, logits, bias, topk_idx, d_topk_w, d_logits, d_x_router,
                       d_w_router, d_bias, ws=None, stream=None):
    wp, wn = _ws(ws)
    _check("moe_route_backward",
           lib().moe_route_backward(ctypes.byref(cfg), _ptr(x), _ptr(w_router), _ptr(logits),
                                    _ptr(bias), _ptr(topk_idx), _ptr(d_topk_w), _ptr(d_logits),
                                    _ptr(d_x_router), _ptr(d_w_router), _ptr(d_bias), wp, wn,
                                    _stream(stream)))


def moe_unpermute_backward(cfg, d_x_perm, slot_of, d_x_router, d_x, stream=None):
    _check("moe_unpermute_backward",
           lib().moe_unpermute_backward(ctypes.byref(cfg), _ptr(d_x_perm), _ptr(slot_of),
                                        _ptr(d_x_router), _ptr(d_x), _stream(stream)))


def moe_ffn_down_packed(cfg, h, expert_offsets, packed_down, y_perm, stream=None):
    _check("moe_ffn_down_packed",
           lib().moe_ffn_down_packed(ctypes.byref(cfg), _ptr(h), _ptr(expert_offsets),
                                     _ptr(packed_down), _ptr(y_perm), _stream(stream)))


def moe_layer_fwd_packed(cfg, x, w_router, bias, packed_gate_up, packed_down, out,
                         bufs: dict | None = None, ws=None, stream=None):
    b = None
    if bufs:
        b = MoELayerBufs(**{n: _ptr(bufs.get(n)) for n in LAYER_BUF_FIELDS})
    wp, wn = _ws(ws)
    _check("moe_layer_fwd_packed",
           lib().moe_layer_fwd_packed(ctypes.byref(cfg), _ptr(x), _ptr(w_router), _ptr(bias),
                                      _ptr(packed_gate_up), _ptr(packed_down), _ptr(out),
                                      ctypes.byref(b) if b else None, wp, wn, _stream(stream)))


# ------------------------------------------------------------ device tensors
def moe_layer_fwd_packed_waved(cfg, x, w_router, bias, packed_gate_up, packed_down, out,
                               bufs: dict | None = None, ws=None, n_waves=2, stream=None,
                               aux_stream=None):
    b = None
    if bufs is not None:
        b = MoELayerBufs(**{n: _ptr(bufs.get(n)) for n in LAYER_BUF_FIELDS})
    wp, wn = _ws(ws)
    aux = None if aux_stream is None else (aux_stream if isinstance(aux_stream, int)
                                           else aux_stream.cuda_stream)
    _check("moe_layer_fwd_packed_waved", lib().moe_layer_fwd_packed_waved(
        ctypes.byref(cfg), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(packed_gate_up),
        _ptr(packed_down), _ptr(out), ctypes.byref(b) if b is not None else None, wp, wn,
        int(n_waves), _stream(stream), aux))


def to_device(a, device="cuda") -> torch.Tensor:
    """numpy array -> device tensor; uint16 arrays are bf16 bit patterns."""
    import numpy as np
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def to_host_bits(t: torch.Tensor):
    """device tensor -> numpy (bf16 as uint16 bit patterns)."""
    import numpy as np
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
