"""fp64 CPU oracle of the Kimi-K2 routed MoE FFN layer.

TEST INFRASTRUCTURE ONLY.  This is the plain, slow, obviously-correct
definition that the HIP path is checked against.  Only the test suite, the
smoke check and the CPU-baseline leg of the benchmark may import it; the
library and its Python binding never do.  It shares no code with the HIP
path (neither imports the other; both only consume the seeded inputs).

What it computes, with where the pages fix each step:

1. Router scores.  logits = x W_r^T, s = sigmoid(logits).
   ["Kimi K2 Base" / "Kimi K2 0905" raw config fields: scoring_func sigmoid,
   n_routed_experts 384, hidden_size 7168.]
2. Selection with a correction bias (topk_method noaux_tc).  sel = s + b is
   used only to choose experts; the pages give only the method's name, so the
   reading taken is: the bias is added for selection and the weights come from
   the unbiased s.  [raw config fields: topk_method noaux_tc]
3. Optional group restriction (n_group > 1, topk_group).  Experts are split
   into n_group contiguous groups; a group's score is the sum of its two
   largest sel values; only the topk_group best groups stay eligible.  K2 uses
   n_group 1 (identity).  The pages state only why grouping exists ("Behind
   Kimi-K2's Config", section 2.4); the top-2-sum rule is the reading taken
   for the DeepSeek-V3-shaped comparison workload.
4. Top-k (num_experts_per_tok 8) of sel among eligible experts; ties go to the
   lower index; the chosen ids are reported in ascending order.
5. Weights w = s[ids] / sum(s[ids]) (norm_topk_prob true), times
   routed_scaling_factor 2.827.  [raw config fields]
6. Expert: y = W_down (silu(W_gate x) * (W_up x)), weights stored [out][in],
   no bias.  ["Kimi K2 . Down projection": the down_proj(act_fn(gate_proj(x))
   * up_proj(x)) expression, the "[out, in]" note and the no-bias note;
   hidden_act silu, moe_intermediate_size 2048.]
7. Shared expert (n_shared_experts 1): same form with intermediate width
   n_shared * moe_intermediate_size, weight 1, added to the routed sum.
8. out[t] = shared(x_t) + sum_j w_j expert_{id_j}(x_t).
9. fp8 mode ("Kimi K2 . Down projection", config.json quantization_config:
   fmt e4m3, weight_block_size [128, 128], activation_scheme dynamic):
   weights are q * s_block; activations entering each expert GEMM (x before
   gate/up, h before down) are quantised per token per 128 channels with
   s = fp32(amax) / 448 (fp32 divide; s = 1 for an all-zero group),
   q = RNE-saturate-e4m3fn(fp32(v) / s), and used as q * s.  The router stays
   unquantised.
10. The sub-block around the layer (block_forward): the pre-MoE RMSNorm
   u = x / sqrt(mean(x^2) + eps) * g, rounded once to the activation dtype
   (the layer's input, as in a plain norm-then-linear model), and the residual
   add out = x + layer(u).  ["Kimi K2 Base" architecture table: RMSNorm;
   raw config fields: rms_norm_eps 1e-06.]  The norm and the rounding
   decision are fp64 here and in the kernel, so both sides round the same
   value.

Everything is float64 except the two places where the method itself fixes
fp32 (the fp8 scale and the division feeding the e4m3 rounding) and the one
rounding of the normalised activations to the activation dtype (step 10).

Pins: each function is checked by tests against page-printed values, closed
forms, library routines or brute force (tests/test_oracle_pins.py).  Parity
unpinned: the numeric value of a full K2-sized layer output has no printed
example on the pages; it is pinned only through the special cases listed
there (identical experts, E=1, x=0, permutation/batch invariance).
"""
from __future__ import annotations

import dataclasses
from typing import Callable, Optional, Sequence, Tuple

import numpy as np

E4M3_MAX = 448.0


# --------------------------------------------------------------------------
# parameter accounting ("Kimi K2 . Down projection", Parameters table)
# --------------------------------------------------------------------------
def linear_params(n_out: int, n_in: int) -> int:
    """Parameters of one bias-free [out, in] linear."""
    return n_out * n_in


def expert_params(hidden_size: int, intermediate: int) -> int:
    """gate_proj + up_proj ([F, H] each) + down_proj ([H, F])."""
    return 2 * linear_params(intermediate, hidden_size) + linear_params(hidden_size, intermediate)


def fp8_expert_bytes(hidden_size: int, intermediate: int, block: int = 128) -> Tuple[int, int]:
    """(weight bytes at 1 B/param, fp32 block-scale bytes) of one fp8 expert."""
    w = expert_params(hidden_size, intermediate)
    nscale = 3 * (intermediate // block) * (hidden_size // block)
    return w, 4 * nscale


def layer_flops(num_tokens: int, hidden_size: int, intermediate: int, n_routed: int,
                top_k: int, n_shared: int) -> int:
    """Multiply-add flops (x2) of one layer: router GEMV plus k routed and the
    shared expert per token (each expert = three H x F products)."""
    per_expert = 2 * 3 * hidden_size * intermediate
    return num_tokens * (top_k * per_expert + n_shared * per_expert + 2 * hidden_size * n_routed)


# --------------------------------------------------------------------------
# e4m3fn (OCP FP8, max 448, no infinities) round-to-nearest-even, saturating
# --------------------------------------------------------------------------
def e4m3_round(v) -> np.ndarray:
    """Round values to the nearest e4m3fn value (ties to even), saturating at
    +-448.  Input is exactly representable in fp64; output is fp64.

    e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits; normals
    2^-6 .. 448 (= 1.75 * 2^8), subnormal spacing 2^-9.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, e = np.frexp(np.where(a > 0, a, 1.0))      # a = m * 2^e, m in [0.5, 1)
    exp = e - 1                                   # a in [2^exp, 2^(exp+1))
    exp = np.maximum(exp, -6)                     # subnormal range shares 2^-6's spacing
    quantum = np.ldexp(1.0, exp - 3)              # 3 mantissa bits
    r = np.rint(a / quantum) * quantum            # exact scaling; rint = ties-to-even
    r = np.minimum(r, E4M3_MAX)
    return np.copysign(r, v)


def e4m3_decode(codes) -> np.ndarray:
    """uint8 e4m3fn codes -> fp64 values (0x7f / 0xff are NaN)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ex = (c >> 3) & 0xF
    man = c & 0x7
    val = np.where(ex == 0, np.ldexp(man / 8.0, -6), np.ldexp(1.0 + man / 8.0, ex - 7))
    val = np.where((ex == 0xF) & (man == 0x7), np.nan, val)
    return sign * val


def act_quant(v: np.ndarray, block: int = 128) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Dynamic activation quantisation per row and per `block` channels.

    Returns (dequantised fp64, e4m3 values fp64, fp32 scales [rows, C/block]).
    s = fp32(amax) / 448 in fp32, 1 for an all-zero group; q = e4m3(fp32(v)/s).
    """
    v32 = np.asarray(v, dtype=np.float64).astype(np.float32)
    R, C = v32.shape
    g = v32.reshape(R, C // block, block)
    amax = np.abs(g).max(axis=2)
    s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    ratio = (g / s[:, :, None]).astype(np.float32)          # IEEE fp32 division
    q = e4m3_round(ratio)
    deq = q * s[:, :, None].astype(np.float64)
    return deq.reshape(R, C), q.reshape(R, C), s


def dequant_weight(q_codes: np.ndarray, scales: np.ndarray, block: int = 128) -> np.ndarray:
    """Block-quantised weight [O][I] (e4m3 codes, fp32 scales [O/b][I/b]) -> fp64:
    code value times its block's scale.  (The code values come from a
    256-entry table of e4m3_decode, which is e4m3_decode of each code.)"""
    table = e4m3_decode(np.arange(256, dtype=np.uint8))
    q = np.asarray(q_codes, dtype=np.uint8)
    O, I = q.shape
    w = table[q].reshape(O // block, block, I // block, block)
    s = np.asarray(scales, np.float64)[:, None, :, None]
    return (w * s).reshape(O, I)


# --------------------------------------------------------------------------
# routing
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Route:
    ids: np.ndarray          # [T, k] int64, ascending per token
    weights: np.ndarray      # [T, k] float64, aligned with ids
    scores: np.ndarray       # [T, E] sigmoid scores
    sel: np.ndarray          # [T, E] selection scores (scores + bias)
    eligible: np.ndarray     # [T, E] bool, after group restriction


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def _top_indices(vals: np.ndarray, n: int) -> np.ndarray:
    """Indices of the n largest entries per row; equal values -> lower index."""
    order = np.argsort(-vals, axis=1, kind="stable")
    return order[:, :n]


def group_scores(sel: np.ndarray, n_group: int) -> np.ndarray:
    """Sum of the two largest selection scores in each contiguous group."""
    T, E = sel.shape
    g = np.sort(sel.reshape(T, n_group, E // n_group), axis=2)
    return g[:, :, -1] + (g[:, :, -2] if E // n_group > 1 else 0.0)


def route(x, router_w, router_bias, *, num_experts_per_tok: int, n_group: int = 1,
          topk_group: int = 1, norm_topk_prob: bool = True,
          routed_scaling_factor: float = 2.827) -> Route:
    x = np.asarray(x, np.float64)
    W = np.asarray(router_w, np.float64)
    b = np.asarray(router_bias, np.float64)
    T, E = x.shape[0], W.shape[0]
    k = num_experts_per_tok
    scores = sigmoid(x @ W.T)
    sel = scores + b[None, :]
    eligible = np.ones((T, E), bool)
    if n_group > 1:
        gs = group_scores(sel, n_group)
        keep = _top_indices(gs, topk_group)
        gmask = np.zeros((T, n_group), bool)
        np.put_along_axis(gmask, keep, True, axis=1)
        eligible = np.repeat(gmask, E // n_group, axis=1)
    masked = np.where(eligible, sel, -np.inf)
    ids = np.sort(_top_indices(masked, k), axis=1)
    w = np.take_along_axis(scores, ids, axis=1)
    if norm_topk_prob:
        w = w / w.sum(axis=1, keepdims=True)
    w = w * routed_scaling_factor
    return Route(ids=ids, weights=w, scores=scores, sel=sel, eligible=eligible)


def selection_gap(r: Route, k: int) -> np.ndarray:
    """Per token: (k-th largest eligible sel) - ((k+1)-th largest eligible sel);
    infinite when every expert is chosen (no (k+1)-th)."""
    if k >= r.sel.shape[1]:
        return np.full(r.sel.shape[0], np.inf)
    masked = np.where(r.eligible, r.sel, -np.inf)
    srt = -np.sort(-masked, axis=1)
    return srt[:, k - 1] - srt[:, k]


def group_gap(r: Route, n_group: int, topk_group: int) -> np.ndarray:
    """Per token: gap between the topk_group-th and next group score."""
    if n_group <= 1:
        return np.full(r.sel.shape[0], np.inf)
    gs = -np.sort(-group_scores(r.sel, n_group), axis=1)
    return gs[:, topk_group - 1] - gs[:, topk_group]


# --------------------------------------------------------------------------
# grouping tokens by expert (stable)
# --------------------------------------------------------------------------
def permute(ids: np.ndarray, n_experts: int):
    """(offsets [E+1], sorted_token_ids [n], inv_perm [T*k]).

    Entry (t, j) goes to segment ids[t, j]; inside a segment entries keep
    ascending flat order t*k + j (ascending t; a token that names one expert
    twice keeps its slots in order); inv_perm[t*k+j] is its row in the grouped
    order.  An entry whose id lies outside [0, E) is not grouped (no row,
    inv_perm -1), so offsets[E] = n, the number of grouped entries (T*k when
    every id is valid).  (The pages route every token to k of the E experts;
    the out-of-range case is a reading for ids from other sources, e.g. an
    expert held by another expert-parallel rank.)
    """
    T, k = ids.shape
    flat = np.asarray(ids, np.int64).reshape(-1)
    valid = (flat >= 0) & (flat < n_experts)
    counts = np.bincount(flat[valid], minlength=n_experts)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    order = np.flatnonzero(valid)[np.argsort(flat[valid], kind="stable")]
    inv = np.full(T * k, -1, np.int64)
    inv[order] = np.arange(len(order))
    return offsets.astype(np.int64), (order // k).astype(np.int64), inv


def combine(y_perm, y_shared, weights, inv_perm) -> np.ndarray:
    """out[t] = y_shared[t] + sum_j weights[t, j] * y_perm[inv_perm[t*k + j]]
    (step 8 above, on grouped expert outputs), skipping entries whose row
    lies outside y_perm's T*k rows (not grouped: -1).  y_shared may be None
    (no shared expert)."""
    w = np.asarray(weights, np.float64)
    T, k = w.shape
    y = np.asarray(y_perm, np.float64)
    out = np.zeros((T, y.shape[1])) if y_shared is None else np.array(y_shared, np.float64)
    inv = np.asarray(inv_perm, np.int64).reshape(T, k)
    for t in range(T):
        for j in range(k):
            r = inv[t, j]
            if 0 <= r < T * k:
                out[t] += w[t, j] * y[r]
    return out


# --------------------------------------------------------------------------
# experts
# --------------------------------------------------------------------------
def silu(z):
    return z * sigmoid(z)


def swiglu_hidden(x, w_gate, w_up, fp8_act: bool = False) -> np.ndarray:
    """h = silu(W_gate x) * (W_up x), the input of the down projection (before
    its fp8 quantisation); rows of x are tokens; [out][in]."""
    a = np.asarray(x, np.float64)
    if fp8_act:
        a = act_quant(a)[0]
    g = a @ np.asarray(w_gate, np.float64).T
    u = a @ np.asarray(w_up, np.float64).T
    return silu(g) * u


def swiglu_expert(x, w_gate, w_up, w_down, fp8_act: bool = False) -> np.ndarray:
    """y = W_down (silu(W_gate x) * (W_up x)); rows of x are tokens; [out][in]."""
    h = swiglu_hidden(x, w_gate, w_up, fp8_act)
    if fp8_act:
        h = act_quant(h)[0]
    return h @ np.asarray(w_down, np.float64).T


ExpertFn = Callable[[int], Tuple[np.ndarray, np.ndarray, np.ndarray]]


def layer_forward(x, router_w, router_bias, expert: ExpertFn, shared: Optional[Sequence[np.ndarray]],
                  *, num_experts_per_tok: int, n_group: int = 1, topk_group: int = 1,
                  norm_topk_prob: bool = True, routed_scaling_factor: float = 2.827,
                  fp8_act: bool = False, tokens: Optional[np.ndarray] = None,
                  route_result: Optional[Route] = None):
    """Full layer.  `expert(e)` returns (w_gate, w_up, w_down) of routed expert
    e as fp64-convertible arrays (fetched one at a time); `shared` is the
    shared expert's triple or None.  `tokens` restricts the output to a subset
    of rows (routing is still computed for those rows only).

    Returns (out [len(tokens), H] fp64, Route of the computed rows).
    """
    x = np.asarray(x, np.float64)
    if tokens is not None:
        x = x[np.asarray(tokens)]
    r = route_result if route_result is not None else route(
        x, router_w, router_bias, num_experts_per_tok=num_experts_per_tok, n_group=n_group,
        topk_group=topk_group, norm_topk_prob=norm_topk_prob,
        routed_scaling_factor=routed_scaling_factor)
    T, H = x.shape
    out = np.zeros((T, H), np.float64)
    if shared is not None:
        out += swiglu_expert(x, *shared, fp8_act=fp8_act)
    for e in np.unique(r.ids):
        rows, slot = np.nonzero(r.ids == e)
        y = swiglu_expert(x[rows], *expert(int(e)), fp8_act=fp8_act)
        out[rows] += r.weights[rows, slot][:, None] * y
    return out, r


# --------------------------------------------------------------------------
# the sub-block around the layer: pre-MoE RMSNorm and residual add
# ("Kimi K2 Base" architecture table: RMSNorm; raw config fields:
# rms_norm_eps 1e-06)
# --------------------------------------------------------------------------
def round_bf16(v) -> np.ndarray:
    """Nearest bfloat16 value (ties to even) of fp64 values, returned as fp64.

    bfloat16 keeps 7 of the 52 fp64 mantissa bits: the 45 dropped bits are
    rounded half-to-even straight from fp64 (no detour through fp32, which
    would round twice).  Defined for zero and for magnitudes in the normal
    bfloat16 range [2^-126, 2^128)."""
    a = np.ascontiguousarray(np.asarray(v, np.float64))
    bits = a.view(np.uint64)
    sign = bits & np.uint64(1 << 63)
    mag = bits & np.uint64((1 << 63) - 1)
    low = mag & np.uint64((1 << 45) - 1)
    kept = mag >> np.uint64(45)
    half = np.uint64(1 << 44)
    up = (low > half) | ((low == half) & ((kept & np.uint64(1)) == np.uint64(1)))
    kept = kept + up.astype(np.uint64)
    out = ((kept << np.uint64(45)) | sign).view(np.float64)
    m = np.abs(out)
    if not np.all((a == 0) | ((np.abs(a) >= 2.0 ** -126) & (m < 2.0 ** 128))):
        raise ValueError("round_bf16: value outside the normal bfloat16 range")
    return out


def round_act(v, act_dtype: str) -> np.ndarray:
    """Round to the activation dtype: "bf16" (round_bf16) or "f32" (IEEE
    round-to-nearest-even of the fp64 value)."""
    if act_dtype == "f32":
        return np.asarray(v, np.float64).astype(np.float32).astype(np.float64)
    return round_bf16(v)


def rms_norm(x, weight, eps: float) -> np.ndarray:
    """u = x / sqrt(mean_h x^2 + eps) * weight, per row, in fp64."""
    x = np.asarray(x, np.float64)
    ms = np.mean(x * x, axis=1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(weight, np.float64)


def block_forward(x, norm_weight, eps: float, router_w, router_bias, expert: ExpertFn,
                  shared: Optional[Sequence[np.ndarray]], *, act_dtype: str = "bf16",
                  tokens: Optional[np.ndarray] = None, **layer_kw):
    """out = x + layer(u), u = the activation-dtype rounding of rms_norm(x).

    Returns (out [rows, H] fp64, Route of the computed rows, u [rows, H])."""
    x = np.asarray(x, np.float64)
    if tokens is not None:
        x = x[np.asarray(tokens)]
    u = round_act(rms_norm(x, norm_weight, eps), act_dtype)
    y, r = layer_forward(u, router_w, router_bias, expert, shared, **layer_kw)
    return x + y, r, u
