"""Helpers of the GPU tests: run the HIP path through the C ABI and compare
with the oracle at the stated tolerances (TOL: relative error of the layer
output per weight dtype; W_RTOL: routing weights), and the full-size oracle
helpers (every grouped row, the fp8 codes of the SwiGLU output)."""
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
    r["ws"] = ws
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


# ------------------------------------------------ full-size oracle helpers --
class Experts:
    """Oracle callback over a case's expert weights that prepares the fp64
    weights of the experts in `order` ahead of use on worker threads (the
    per-expert conversion, not the products, is what dominates at full
    size).  Call with an expert id in `order`'s order."""

    def __init__(self, wl, case, order, workers: int = 4, ahead: int = 8):
        import concurrent.futures
        import cases
        self.fn = cases.expert_fn(wl, case)
        self.order = [int(e) for e in order]
        self.pool = concurrent.futures.ThreadPoolExecutor(workers)
        self.ahead = ahead
        self.futs = {}
        self.pos = 0
        self._fill()

    def _fill(self):
        while len(self.futs) < self.ahead and self.pos < len(self.order):
            e = self.order[self.pos]
            self.futs[e] = self.pool.submit(self.fn, e)
            self.pos += 1

    def __call__(self, e):
        e = int(e)
        fut = self.futs.pop(e, None)
        w = fut.result() if fut is not None else self.fn(e)
        self._fill()
        return w

    def close(self):
        self.pool.shutdown(wait=False, cancel_futures=True)


def rows_err(got: torch.Tensor, ref: np.ndarray, chunk: int = 4096) -> np.ndarray:
    """Per row: max |got - ref| / max |ref| (got on any device)."""
    out = np.empty(ref.shape[0])
    for a in range(0, ref.shape[0], chunk):
        g = got[a:a + chunk].detach().to("cpu", torch.float64).numpy()
        r = ref[a:a + chunk]
        out[a:a + chunk] = np.abs(g - r).max(axis=1) / np.maximum(np.abs(r).max(axis=1), 1e-300)
    return out


def grouped_oracle(wl, x64: np.ndarray, sorted_ids: np.ndarray, offsets: np.ndarray, case, experts=None,
                   hidden: bool = False):
    """The oracle on the grouped rows of `experts` (default: all non-empty):
    for expert e and every row p of its segment, y[p] = swiglu_expert of
    x[sorted_ids[p]] with e's weights; with `hidden`, also h[p] (the SwiGLU
    output ahead of the down projection).  Returns (rows, y, h or None) with
    the rows ascending."""
    import oracle
    fp8 = wl.weight_dtype == gen.FP8
    E = wl.n_routed_experts
    counts = np.diff(offsets)
    order = [e for e in (range(E) if experts is None else experts) if counts[e] > 0]
    fetch = Experts(wl, case, order)
    rows, ys, hs = [], [], []
    try:
        for e in order:
            wg, wu, wd = fetch(e)
            p = np.arange(offsets[e], offsets[e + 1])
            a = x64[sorted_ids[p]]
            h = oracle.swiglu_hidden(a, wg, wu, fp8_act=fp8)
            hq = oracle.act_quant(h)[0] if fp8 else h
            rows.append(p)
            ys.append(hq @ wd.T)
            if hidden:
                hs.append(h)
    finally:
        fetch.close()
    rows = np.concatenate(rows)
    return rows, np.concatenate(ys), (np.concatenate(hs) if hidden else None)


def check_h_codes(codes: torch.Tensor, scales: torch.Tensor, h_ref: np.ndarray, what: str):
    """e4m3 codes and per-128 scales of the SwiGLU output against the oracle's
    activation quantisation of its fp64 h (the same fp32 scale and division).
    The kernel's h is fp32: gate and up are sums of H = 7168 products in fp32,
    whose cancellation (|sum| ~ sum|terms| / sqrt(H)) leaves relative errors
    up to ~1e-4 of a group's largest h (measured 9.6e-5 on the scales).  So a
    scale may differ by that (bound 1e-3), and h / s (at most 448) by up to
    448 * 2e-4 ~ 0.09: every code must be the e4m3 rounding of some value
    within DELTA = 0.25 of the oracle's h / s, i.e. lie between
    e4m3(r - DELTA) and e4m3(r + DELTA) (the rounding is monotone), and at
    most 1 % of the codes may differ from the oracle's (measured 0.15 % at K2
    size, fp8, T=4096: the scale differences move whole groups).  A wrong
    group maximum, channel or division fails both."""
    import oracle
    DELTA = 0.25
    _, q_ref, s_ref = oracle.act_quant(h_ref)
    s_got = scales.detach().cpu().numpy()
    rel = np.abs(s_got.astype(np.float64) - s_ref) / s_ref
    assert rel.max() <= 1e-3, f"{what}: scales differ by {rel.max():.3g} relative"
    q_got = oracle.e4m3_decode(codes.detach().cpu().numpy())
    diff = np.argwhere(q_got != q_ref)
    say(f"  {what}: {q_ref.size} codes, {len(diff)} differ, scale rel diff {rel.max():.2e}")
    if len(diff) == 0:
        return
    assert len(diff) <= 1e-2 * q_ref.size, f"{what}: {len(diff)} codes differ"
    r, c = diff[:, 0], diff[:, 1]
    ratio = h_ref[r, c] / s_ref[r, c // 128].astype(np.float64)
    v = q_got[r, c]
    ok = (oracle.e4m3_round(ratio - DELTA) <= v) & (v <= oracle.e4m3_round(ratio + DELTA))
    # the smallest shift of r that reaches the kernel's code: distance to the
    # rounding midpoint between the two codes
    mid = (v + q_ref[r, c]) / 2
    say(f"  {what}: differing codes at {np.median(np.abs(ratio - mid)):.2g} (median), "
        f"{np.abs(ratio - mid).max():.3g} (max) from the midpoint")
    assert ok.all(), f"{what}: {int((~ok).sum())} codes are no rounding of h / s +- {DELTA}"
