"""Helpers of the GPU tests: run the HIP path through the C ABI and compare
with the oracle at the stated tolerances (TOL: relative error of the layer
output per weight dtype; W_RTOL: routing weights)."""
from __future__ import annotations

import sys

import numpy as np
import torch

from sparse_moe_transformer_sigmoid_amd import binding as B
from sparse_moe_transformer_sigmoid_amd import inputs as gen

# max-abs-err / max|ref| bounds of the outputs, by weight dtype
TOL = {gen.F32: 1e-4, gen.BF16: 1e-2, gen.FP8: 5e-2}
# Routing weights, relative.  The logits are fp32 dot products of length H
# (7168): with partial sums of size ~0.02*sqrt(k) the accumulated rounding is
# ~2^-24 * 0.02 * H / sqrt(2) ~ 6e-6 absolute; a weight s/sum(s) inherits
# (1 - s) times that (up to ~0.5 for bias-favoured low scores) plus a few ulp
# from the sigmoid and the renormalisation, so 1e-5 bounds it.
W_RTOL = 1e-5


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def cfg_of(wl: gen.Workload) -> B.MoeConfig:
    return B.MoeConfig.from_fields(wl.fields())


def act_dtype(wl):
    return gen.torch_dtype(wl.act_dtype)


def run_layer(wl: gen.Workload, case: dict, ws=None):
    """moe_layer_forward on `case` (device tensors); returns out, ids, weights."""
    cfg = cfg_of(wl)
    x = case["x"]
    T = x.shape[0]
    k = wl.num_experts_per_tok
    out = torch.empty((T, wl.hidden_size), dtype=act_dtype(wl), device=x.device)
    ids = torch.empty((T, k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = B.alloc_workspace(cfg, T)
    B.moe_layer_forward(cfg, B.MoeWeights.from_tensors(case), x, case["router_w"], case["router_bias"], out,
                        ws, ids, w)
    torch.cuda.synchronize()
    return out, ids, w


def run_stages(wl: gen.Workload, case: dict):
    """route -> permute -> expert_ffn -> combine, returning every intermediate."""
    cfg = cfg_of(wl)
    x = case["x"]
    dev = x.device
    T, H, E, k = x.shape[0], wl.hidden_size, wl.n_routed_experts, wl.num_experts_per_tok
    ws = B.alloc_workspace(cfg, T)
    r = {"ids": torch.empty((T, k), dtype=torch.int32, device=dev),
         "w": torch.empty((T, k), dtype=torch.float32, device=dev)}
    B.moe_route(cfg, x, case["router_w"], case["router_bias"], r["ids"], r["w"], ws)
    fp8 = wl.weight_dtype == gen.FP8
    r["offsets"] = torch.empty(E + 1, dtype=torch.int32, device=dev)
    r["sorted"] = torch.empty(T * k, dtype=torch.int32, device=dev)
    r["inv"] = torch.empty(T * k, dtype=torch.int32, device=dev)
    if fp8:
        r["x_perm"] = torch.empty((T * k, H), dtype=torch.uint8, device=dev)
        r["x_perm_scales"] = torch.empty((T * k, H // 128), dtype=torch.float32, device=dev)
    else:
        r["x_perm"] = torch.empty((T * k, H), dtype=act_dtype(wl), device=dev)
        r["x_perm_scales"] = None
    B.moe_permute(cfg, x, r["ids"], r["offsets"], r["sorted"], r["inv"], r["x_perm"], r["x_perm_scales"], ws)
    r["y_perm"] = torch.empty((T * k, H), dtype=act_dtype(wl), device=dev)
    r["y_sh"] = torch.empty((T, H), dtype=act_dtype(wl), device=dev)
    B.moe_expert_ffn(cfg, B.MoeWeights.from_tensors(case), x, r["x_perm"], r["x_perm_scales"], r["offsets"],
                     r["y_perm"], r["y_sh"], ws)
    r["out"] = torch.empty((T, H), dtype=act_dtype(wl), device=dev)
    B.moe_combine(cfg, r["y_perm"], r["y_sh"], r["w"], r["inv"], r["out"])
    torch.cuda.synchronize()
    return r


def rel_err(got: torch.Tensor, ref: np.ndarray) -> float:
    g = got.detach().to("cpu", torch.float64).numpy()
    scale = np.abs(ref).max()
    return float(np.abs(g - ref).max() / scale) if scale > 0 else float(np.abs(g).max())


def check_route(ids: torch.Tensor, w: torch.Tensor, route, rows=None):
    ids_np = ids.cpu().numpy()
    w_np = w.cpu().numpy().astype(np.float64)
    if rows is not None:
        ids_np, w_np = ids_np[rows], w_np[rows]
    bad = np.nonzero((ids_np != route.ids).any(axis=1))[0]
    assert len(bad) == 0, f"routing differs on {len(bad)} tokens, first {bad[:5]}"
    rel = np.abs(w_np - route.weights) / np.abs(route.weights)
    assert rel.max() <= W_RTOL, f"routing weights rel err {rel.max():.3g}"


def run_block(wl: gen.Workload, case: dict):
    """moe_block_forward on `case`; returns out, ids, weights."""
    cfg = cfg_of(wl)
    x = case["x"]
    T, k = x.shape[0], wl.num_experts_per_tok
    out = torch.empty((T, wl.hidden_size), dtype=act_dtype(wl), device=x.device)
    ids = torch.empty((T, k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    ws = B.alloc_workspace(cfg, T)
    B.moe_block_forward(cfg, B.MoeWeights.from_tensors(case), x, case["norm_weight"], float(np.float32(wl.rms_norm_eps)),
                        case["router_w"], case["router_bias"], out, ws, ids, w)
    torch.cuda.synchronize()
    return out, ids, w


def block_err(got: torch.Tensor, ref: np.ndarray, x: np.ndarray, act: str) -> float:
    """Error of a sub-block output in units of max|layer part|, after allowing
    one unit in the last place of the output's rounding (bf16: 2^-8 |ref|,
    fp32: 2^-22 |ref|): the layer part ref - x carries the layer tolerance,
    the residual only the final rounding."""
    g = got.detach().to("cpu", torch.float64).numpy()
    ulp = 2.0 ** -8 if act == gen.BF16 else 2.0 ** -22
    excess = np.maximum(np.abs(g - ref) - ulp * np.abs(ref), 0.0)
    scale = np.abs(ref - x).max()
    return float(excess.max() / scale)
