"""ctypes binding of libmoe.so (include/moe.h).  Argument marshalling only.

Each function takes torch tensors that already live on the GPU, passes their
data pointers and the current HIP stream to the C entry point of the same
name, and raises MoeError on a non-OK status.  Every step of the layer runs
in the library's HIP kernels; there is no fallback of any kind -- if the
library is not built, loading it raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16, MOE_FP8_E4M3 = range(3)
(MOE_KID_ROUTER_LOGITS, MOE_KID_ROUTER_TOPK, MOE_KID_PERMUTE, MOE_KID_TILES, MOE_KID_GATHER,
 MOE_KID_ACT_QUANT, MOE_KID_GATE_UP, MOE_KID_DOWN, MOE_KID_COMBINE, MOE_KID_NORM, MOE_KID_COUNT) = range(11)

(MOE_WS_H, MOE_WS_H_CODES, MOE_WS_H_SCALES, MOE_WS_H_SHARED, MOE_WS_H_SHARED_CODES, MOE_WS_H_SHARED_SCALES,
 MOE_WS_Y, MOE_WS_Y_SHARED, MOE_WS_COUNT) = range(9)

DTYPES = {"f32": MOE_F32, "bf16": MOE_BF16, "fp8_e4m3": MOE_FP8_E4M3}


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({detail})")
        self.status = status


class MoeConfig(ctypes.Structure):
    _fields_ = [("hidden_size", ctypes.c_int32), ("moe_intermediate_size", ctypes.c_int32),
                ("n_routed_experts", ctypes.c_int32), ("num_experts_per_tok", ctypes.c_int32),
                ("n_shared_experts", ctypes.c_int32), ("n_group", ctypes.c_int32),
                ("topk_group", ctypes.c_int32), ("norm_topk_prob", ctypes.c_int32),
                ("routed_scaling_factor", ctypes.c_float), ("scoring_func", ctypes.c_int32),
                ("topk_method", ctypes.c_int32), ("act_dtype", ctypes.c_int32),
                ("weight_dtype", ctypes.c_int32), ("weight_block_size", ctypes.c_int32 * 2)]

    @classmethod
    def from_fields(cls, f: Dict) -> "MoeConfig":
        """Build from the model-config field names (hidden_size, ...)."""
        wdt = DTYPES[f["weight_dtype"]]
        c = cls()
        for name in ("hidden_size", "moe_intermediate_size", "n_routed_experts", "num_experts_per_tok",
                     "n_shared_experts", "n_group", "topk_group"):
            setattr(c, name, int(f[name]))
        c.norm_topk_prob = 1 if f.get("norm_topk_prob", True) else 0
        c.routed_scaling_factor = float(f["routed_scaling_factor"])
        c.scoring_func = {"sigmoid": 0}.get(f.get("scoring_func", "sigmoid"), 99)
        c.topk_method = {"noaux_tc": 0}.get(f.get("topk_method", "noaux_tc"), 99)
        c.act_dtype = DTYPES[f["act_dtype"]]
        c.weight_dtype = wdt
        c.weight_block_size[0] = c.weight_block_size[1] = 128 if wdt == MOE_FP8_E4M3 else 0
        return c


_P = ctypes.c_void_p
_W_FIELDS = ["w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down", "sh_gate", "sh_up", "sh_down",
             "sh_s_gate", "sh_s_up", "sh_s_down"]


class MoeWeights(ctypes.Structure):
    _fields_ = [(n, _P) for n in _W_FIELDS]

    @classmethod
    def from_tensors(cls, d: Dict[str, torch.Tensor]) -> "MoeWeights":
        w = cls()
        for n in _W_FIELDS:
            t = d.get(n)
            setattr(w, n, _ptr(t) if t is not None else None)
        return w


_lib = None


def load() -> ctypes.CDLL:
    """Load libmoe.so (built by build.py); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run `python -m sparse_moe_transformer_sigmoid_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    CP = ctypes.POINTER(MoeConfig)
    WP = ctypes.POINTER(MoeWeights)
    i64, sz, st = ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
    sigs = {
        "moe_workspace_size": (sz, [CP, i64]),
        "moe_route": (st, [CP, _P, _P, _P, i64, _P, _P, _P, sz, _P]),
        "moe_permute": (st, [CP, _P, _P, i64, _P, _P, _P, _P, _P, _P, sz, _P]),
        "moe_expert_ffn": (st, [CP, WP, _P, _P, _P, _P, i64, _P, _P, _P, sz, _P]),
        "moe_combine": (st, [CP, _P, _P, _P, _P, i64, _P, _P]),
        "moe_layer_forward": (st, [CP, WP, _P, _P, _P, i64, _P, _P, _P, _P, sz, _P]),
        "moe_layer_forward_static": (st, [CP, WP, _P, _P, _P, i64, _P, _P, _P, _P]),
        "moe_block_forward": (st, [CP, WP, _P, _P, ctypes.c_float, _P, _P, i64, _P, _P, _P, _P, sz, _P]),
        "moe_status_string": (ctypes.c_char_p, [st]),
        "moe_last_error": (ctypes.c_char_p, []),
        "moe_abi_version": (ctypes.c_int, []),
        "moe_profile_arm": (st, [ctypes.c_int32, _P, _P]),
        "moe_workspace_region": (st, [CP, i64, ctypes.c_int32, ctypes.POINTER(sz), ctypes.POINTER(sz)]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    _lib = lib
    return lib


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmoe must be contiguous")
    return t.data_ptr()


def _stream(stream=None):
    if stream is not None:
        return stream
    return torch.cuda.current_stream().cuda_stream


def _check(status: int, where: str):
    if status != MOE_OK:
        lib = load()
        raise MoeError(status, where, lib.moe_last_error().decode())


def _nbytes(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def moe_workspace_size(cfg: MoeConfig, num_tokens: int) -> int:
    return load().moe_workspace_size(ctypes.byref(cfg), int(num_tokens))


def alloc_workspace(cfg: MoeConfig, num_tokens: int, device="cuda") -> torch.Tensor:
    n = moe_workspace_size(cfg, num_tokens)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def moe_route(cfg, x, router_w, router_bias, topk_ids, topk_weights, ws, stream=None):
    _check(load().moe_route(ctypes.byref(cfg), _ptr(x), _ptr(router_w), _ptr(router_bias), x.shape[0],
                            _ptr(topk_ids), _ptr(topk_weights), _ptr(ws), _nbytes(ws), _stream(stream)),
           "moe_route")


def moe_permute(cfg, x, topk_ids, expert_offsets, sorted_token_ids, inv_perm, x_perm, x_perm_scales, ws,
                stream=None):
    _check(load().moe_permute(ctypes.byref(cfg), _ptr(x), _ptr(topk_ids), topk_ids.shape[0],
                              _ptr(expert_offsets), _ptr(sorted_token_ids), _ptr(inv_perm), _ptr(x_perm),
                              _ptr(x_perm_scales), _ptr(ws), _nbytes(ws), _stream(stream)),
           "moe_permute")


def moe_expert_ffn(cfg, weights: MoeWeights, x, x_perm, x_perm_scales, expert_offsets, y_perm, y_shared, ws,
                   stream=None):
    _check(load().moe_expert_ffn(ctypes.byref(cfg), ctypes.byref(weights), _ptr(x), _ptr(x_perm),
                                 _ptr(x_perm_scales), _ptr(expert_offsets), x.shape[0], _ptr(y_perm),
                                 _ptr(y_shared), _ptr(ws), _nbytes(ws), _stream(stream)),
           "moe_expert_ffn")


def moe_combine(cfg, y_perm, y_shared, topk_weights, inv_perm, out, stream=None):
    _check(load().moe_combine(ctypes.byref(cfg), _ptr(y_perm), _ptr(y_shared), _ptr(topk_weights),
                              _ptr(inv_perm), out.shape[0], _ptr(out), _stream(stream)),
           "moe_combine")


def moe_layer_forward(cfg, weights: MoeWeights, x, router_w, router_bias, out, ws, topk_ids=None,
                      topk_weights=None, stream=None):
    _check(load().moe_layer_forward(ctypes.byref(cfg), ctypes.byref(weights), _ptr(x), _ptr(router_w),
                                    _ptr(router_bias), x.shape[0], _ptr(out), _ptr(topk_ids),
                                    _ptr(topk_weights), _ptr(ws), _nbytes(ws), _stream(stream)),
           "moe_layer_forward")


MOE_STATIC_SCRATCH_BYTES = 64 << 20


def moe_layer_forward_static(cfg, weights: MoeWeights, x, router_w, router_bias, out, topk_ids=None,
                             topk_weights=None, stream=None):
    """moe_layer_forward on the library's fixed per-GPU scratch (no workspace
    argument, nothing allocated)."""
    _check(load().moe_layer_forward_static(ctypes.byref(cfg), ctypes.byref(weights), _ptr(x), _ptr(router_w),
                                           _ptr(router_bias), x.shape[0], _ptr(out), _ptr(topk_ids),
                                           _ptr(topk_weights), _stream(stream)),
           "moe_layer_forward_static")


def moe_block_forward(cfg, weights: MoeWeights, x, norm_weight, rms_norm_eps, router_w, router_bias, out, ws,
                      topk_ids=None, topk_weights=None, stream=None):
    _check(load().moe_block_forward(ctypes.byref(cfg), ctypes.byref(weights), _ptr(x), _ptr(norm_weight),
                                    float(rms_norm_eps), _ptr(router_w), _ptr(router_bias), x.shape[0], _ptr(out),
                                    _ptr(topk_ids), _ptr(topk_weights), _ptr(ws), _nbytes(ws), _stream(stream)),
           "moe_block_forward")


def moe_profile_arm(kernel_id: int, ev_start: Optional[int] = None, ev_stop: Optional[int] = None):
    """Arm a one-shot pair of raw hipEvent_t handles (ints) around the next
    launch of kernel `kernel_id` (MOE_KID_*); None/None disarms."""
    _check(load().moe_profile_arm(int(kernel_id), ev_start, ev_stop), "moe_profile_arm")


def moe_workspace_region(cfg: MoeConfig, num_tokens: int, region: int):
    """(byte offset, bytes) of workspace region `region` (MOE_WS_*) for num_tokens."""
    off, n = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load().moe_workspace_region(ctypes.byref(cfg), int(num_tokens), int(region), ctypes.byref(off),
                                       ctypes.byref(n)), "moe_workspace_region")
    return off.value, n.value


def workspace_view(ws: torch.Tensor, cfg: MoeConfig, num_tokens: int, region: int, dtype: torch.dtype,
                   shape) -> torch.Tensor:
    """A tensor view of one workspace region (no copy)."""
    off, n = moe_workspace_region(cfg, num_tokens, region)
    esz = torch.empty((), dtype=dtype).element_size()
    count = 1
    for d in shape:
        count *= d
    if count * esz > n:
        raise ValueError(f"region {region} holds {n} bytes, {count * esz} asked for")
    return ws[off:off + count * esz].view(dtype).view(*shape)


def moe_status_string(status: int) -> str:
    return load().moe_status_string(int(status)).decode()


def moe_last_error() -> str:
    return load().moe_last_error().decode()
