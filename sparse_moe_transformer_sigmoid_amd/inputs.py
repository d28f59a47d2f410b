"""Seeded synthetic inputs for the routed MoE FFN layer.

This module only draws random numbers and lays them out; it holds none of the
layer's arithmetic (no scoring, no selection, no expert math).  Both the HIP
path and the fp64 oracle consume exactly the tensors produced here.

Workload recipe (shapes and distributions follow the Kimi-K2 config tables:
"Kimi K2 Base" raw config fields and "Kimi K2 0905" raw config fields;
initializer_range 0.02 is read as a standard deviation):

* x ~ N(0, 1) drawn in fp32, then rounded (RNE) to the activation dtype.
  The layer input is taken to be post-RMSNorm, so unit variance.
* router weight [E][H], expert weights ~ N(0, 0.02) drawn in fp32, rounded.
* router correction bias [E] fp32 ~ N(0, 0.01), or, for the skewed prefill
  workload, a Zipf-like log profile b_e = -1.1 * beta * ln(r_e) over a seeded
  random ranking r of 1..E (beta = 0.1, no other noise).
* fp8 weights: per 128x128 block of the fp32 draw, s = u * amax / 448 with
  u ~ U(0.5, 2); q = e4m3fn(clamp(W / s, +-448)) using torch's cast.  This is
  the checkpoint layout of the "Kimi K2 . Down projection" page's
  quantization_config (fmt e4m3, weight_block_size [128, 128]).

Every tensor has its own stream: numpy PCG64 seeded by SeedSequence([seed,
tensor_id, index]).  Expert weights that live on a GPU are drawn there with a
torch generator seeded from the same SeedSequence, so a single expert can be
regenerated without the others; the oracle then reads the same device bytes
back, never a second draw.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np
import torch

# tensor ids of the independent random streams
TID_X = 1
TID_X_RESAMPLE = 2
TID_ROUTER = 3
TID_BIAS = 4
TID_GATE = 5
TID_UP = 6
TID_DOWN = 7
TID_SH_GATE = 8
TID_SH_UP = 9
TID_SH_DOWN = 10
TID_FP8_U = 11
TID_ZIPF_RANK = 12
TID_DISPATCH_COUNT = 13
TID_DISPATCH_ROWS = 14
TID_NORM = 15

F32, BF16, FP8 = "f32", "bf16", "fp8_e4m3"


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shapes, config fields and input distributions of one synthetic workload.

    Field names follow the model config tables on the pages (hidden_size,
    moe_intermediate_size, n_routed_experts, num_experts_per_tok, ...).
    """
    name: str
    num_tokens: int
    hidden_size: int
    moe_intermediate_size: int
    n_routed_experts: int
    num_experts_per_tok: int
    n_shared_experts: int = 1
    n_group: int = 1
    topk_group: int = 1
    norm_topk_prob: bool = True
    routed_scaling_factor: float = 2.827
    act_dtype: str = BF16          # x, router weight, output
    weight_dtype: str = BF16       # expert weights
    weight_std: float = 0.02
    bias: str = "normal"           # "normal" | "zipf" | "zero" | "hot"
    rms_norm_eps: float = 1e-6     # pre-MoE RMSNorm ("Kimi K2 Base" raw config fields)
    norm_weight_std: float = 0.1   # RMSNorm weight ~ 1 + N(0, std)
    bias_std: float = 0.01
    zipf_beta: float = 0.1
    zipf_s: float = 1.1
    seed: int = 0
    # > 1: the workload is one expert-parallel rank's share of a model with
    # n_routed_experts * ep_size experts; num_tokens is the rank's own batch
    # (which its shared expert serves) and the routed rows arrive dispatched
    # from a global batch of num_tokens * ep_size tokens
    ep_size: int = 1
    # True: the workload is the sub-block around the layer (pre-MoE RMSNorm,
    # the layer, the residual add); x is then the residual stream
    block: bool = False

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def shared_intermediate_size(self) -> int:
        return self.n_shared_experts * self.moe_intermediate_size

    def fields(self) -> Dict:
        """The config fields as a plain dict (what the oracle and binding take)."""
        return dict(
            hidden_size=self.hidden_size,
            moe_intermediate_size=self.moe_intermediate_size,
            n_routed_experts=self.n_routed_experts,
            num_experts_per_tok=self.num_experts_per_tok,
            n_shared_experts=self.n_shared_experts,
            n_group=self.n_group,
            topk_group=self.topk_group,
            norm_topk_prob=self.norm_topk_prob,
            routed_scaling_factor=self.routed_scaling_factor,
            act_dtype=self.act_dtype,
            weight_dtype=self.weight_dtype,
        )


def _k2(name, T, **kw) -> Workload:
    base = dict(hidden_size=7168, moe_intermediate_size=2048, n_routed_experts=384,
                num_experts_per_tok=8, n_shared_experts=1)
    base.update(kw)
    return Workload(name=name, num_tokens=T, **base)


# The Kimi-K2 layer workloads (decode, Zipf prefill, fp8, the DeepSeek-V3 and
# Moonlight shapes, the sub-block, the dense layer, expert-parallel rank
# shares), plus small parity shapes.
WORKLOADS: Dict[str, Workload] = {
    "tiny_fp32": Workload("tiny_fp32", 16, 256, 128, 16, 4, act_dtype=F32, weight_dtype=F32),
    "k2_decode_bf16": _k2("k2_decode_bf16", 128),
    "k2_prefill_bf16_zipf": _k2("k2_prefill_bf16_zipf", 8192, bias="zipf"),
    "k2_fp8": _k2("k2_fp8", 4096, weight_dtype=FP8),
    "dsv3_decode_bf16": _k2("dsv3_decode_bf16", 128, n_routed_experts=256, n_group=8, topk_group=4),
    # Moonlight-16B MoE shape ("Kimi K2 Base" comparison table): hidden 2048,
    # 64 routed experts top-6, 2 shared, moe_intermediate 1408
    "moonlight_bf16": Workload("moonlight_bf16", 256, 2048, 1408, 64, 6, n_shared_experts=2),
    # the dense first layer (first_k_dense_replace 1, intermediate_size 18432)
    # as one always-selected expert of weight 1: E = 1, k = 1, no shared
    # the same decode batch through the sub-block (RMSNorm + layer + residual)
    "k2_block_decode_bf16": _k2("k2_block_decode_bf16", 128, block=True),
    "k2_dense_layer_bf16": _k2("k2_dense_layer_bf16", 128, moe_intermediate_size=18432, n_routed_experts=1,
                               num_experts_per_tok=1, n_shared_experts=0, routed_scaling_factor=1.0,
                               bias="zero"),
    # one expert-parallel rank's share of the Kimi-K2 layer at decode: 384
    # experts over 128 ranks (3 routed + the shared expert per rank) or over
    # 8 ranks (48 routed + shared), 128 tokens per rank
    "k2_ep128_rank_bf16": _k2("k2_ep128_rank_bf16", 128, n_routed_experts=3, ep_size=128),
    "k2_ep8_rank_bf16": _k2("k2_ep8_rank_bf16", 128, n_routed_experts=48, ep_size=8),
    # small shapes that still span several tiles and a ragged tail
    "small_bf16": Workload("small_bf16", 100, 512, 256, 32, 8),
    "small_fp8": Workload("small_fp8", 100, 512, 256, 32, 8, weight_dtype=FP8),
    "small_grouped_bf16": Workload("small_grouped_bf16", 100, 512, 256, 32, 8, n_group=8, topk_group=4),
}


def _rng(seed: int, tid: int, *idx: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid, *idx])))


def _torch_seed(seed: int, tid: int, *idx: int) -> int:
    st = np.random.SeedSequence([seed, tid, *idx]).generate_state(2, np.uint32)
    return int(st[0]) | (int(st[1] & 0x7FFFFFFF) << 32)


def torch_dtype(name: str) -> torch.dtype:
    return {F32: torch.float32, BF16: torch.bfloat16}[name]


def round_to(a: np.ndarray, dtype: str) -> torch.Tensor:
    """fp32 numpy -> torch tensor in `dtype` (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t if dtype == F32 else t.to(torch_dtype(dtype))


def gen_x_rows(wl: Workload, rows: np.ndarray, attempt: int) -> torch.Tensor:
    """Redraw the given token rows (used to enforce a routing-score gap)."""
    out = np.empty((len(rows), wl.hidden_size), np.float32)
    for i, t in enumerate(rows):
        out[i] = _rng(wl.seed, TID_X_RESAMPLE, int(t), attempt).standard_normal(wl.hidden_size, np.float32)
    return round_to(out, wl.act_dtype)


def gen_x(wl: Workload, num_tokens: Optional[int] = None, batch: int = 0) -> torch.Tensor:
    """Token rows x ~ N(0, 1); batch b > 0 draws an independent batch of the
    same shape (a benchmark rotates among several)."""
    T = wl.num_tokens if num_tokens is None else num_tokens
    rng = _rng(wl.seed, TID_X) if batch == 0 else _rng(wl.seed, TID_X, batch)
    a = rng.standard_normal((T, wl.hidden_size), np.float32)
    return round_to(a, wl.act_dtype)


def gen_router(wl: Workload) -> torch.Tensor:
    a = _rng(wl.seed, TID_ROUTER).standard_normal((wl.n_routed_experts, wl.hidden_size), np.float32)
    return round_to(a * np.float32(wl.weight_std), wl.act_dtype)


def gen_bias(wl: Workload) -> torch.Tensor:
    E = wl.n_routed_experts
    if wl.bias == "zero":
        b = np.zeros(E, np.float32)
    elif wl.bias == "normal":
        b = _rng(wl.seed, TID_BIAS).standard_normal(E, np.float32) * np.float32(wl.bias_std)
    elif wl.bias == "hot":
        # two experts (the first and the last) favoured by every token
        b = _rng(wl.seed, TID_BIAS).standard_normal(E, np.float32) * np.float32(wl.bias_std)
        b[0] += 5.0
        b[E - 1] += 5.0
    elif wl.bias == "zipf":
        ranks = _rng(wl.seed, TID_ZIPF_RANK).permutation(E) + 1
        b = (-wl.zipf_s * wl.zipf_beta * np.log(ranks.astype(np.float64))).astype(np.float32)
    else:
        raise ValueError(wl.bias)
    return torch.from_numpy(b)


def _draw(shape, seed, tid, idx, std, device) -> torch.Tensor:
    """fp32 N(0, std) draw of one expert's matrix, on `device`."""
    if torch.device(device).type == "cpu":
        a = _rng(seed, tid, idx).standard_normal(shape, np.float32) * np.float32(std)
        return torch.from_numpy(a)
    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(seed, tid, idx))
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


def _uniform(shape, seed, tid, idx, lo, hi, device) -> torch.Tensor:
    a = _rng(seed, tid, idx).uniform(lo, hi, shape).astype(np.float32)
    return torch.from_numpy(a).to(device)


def quantize_fp8_blocks(w: torch.Tensor, u: torch.Tensor):
    """fp32 [O][I] -> (e4m3fn bytes [O][I] uint8, fp32 scales [O/128][I/128]).

    Checkpoint layout of the "Kimi K2 . Down projection" page, config.json
    quantization_config: e4m3 with one fp32 scale per 128x128 block.
    """
    O, I = w.shape
    blk = w.reshape(O // 128, 128, I // 128, 128)
    amax = blk.abs().amax(dim=(1, 3))
    s = (u * amax / 448.0).to(torch.float32)
    s = torch.where(s > 0, s, torch.ones_like(s))
    q = (blk / s[:, None, :, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q.reshape(O, I).view(torch.uint8), s.contiguous()


def _matrix(wl, shape, tid, idx, device):
    w = _draw(shape, wl.seed, tid, idx, wl.weight_std, device)
    if wl.weight_dtype == FP8:
        u = _uniform((shape[0] // 128, shape[1] // 128), wl.seed, TID_FP8_U, tid * 1_000_003 + idx,
                     0.5, 2.0, w.device)
        return quantize_fp8_blocks(w, u)
    return w.to(torch_dtype(wl.weight_dtype)), None


def gen_expert_weights(wl: Workload, device="cpu", experts: Optional[range] = None) -> Dict[str, torch.Tensor]:
    """Routed + shared expert weights, [out][in] layout, no bias.

    Returns w_gate, w_up [E][F][H]; w_down [E][H][F]; sh_gate, sh_up [Fs][H];
    sh_down [H][Fs]; for fp8 also s_* scale grids [.][out/128][in/128].
    """
    E, H, F, Fs = wl.n_routed_experts, wl.hidden_size, wl.moe_intermediate_size, wl.shared_intermediate_size
    experts = range(E) if experts is None else experts
    wdt = torch.uint8 if wl.weight_dtype == FP8 else torch_dtype(wl.weight_dtype)
    n = len(experts)
    out = {
        "w_gate": torch.empty((n, F, H), dtype=wdt, device=device),
        "w_up": torch.empty((n, F, H), dtype=wdt, device=device),
        "w_down": torch.empty((n, H, F), dtype=wdt, device=device),
    }
    if wl.weight_dtype == FP8:
        out["s_gate"] = torch.empty((n, F // 128, H // 128), dtype=torch.float32, device=device)
        out["s_up"] = torch.empty((n, F // 128, H // 128), dtype=torch.float32, device=device)
        out["s_down"] = torch.empty((n, H // 128, F // 128), dtype=torch.float32, device=device)
    for i, e in enumerate(experts):
        for name, tid, shape in (("gate", TID_GATE, (F, H)), ("up", TID_UP, (F, H)), ("down", TID_DOWN, (H, F))):
            q, s = _matrix(wl, shape, tid, e, device)
            out["w_" + name][i].copy_(q)
            if s is not None:
                out["s_" + name][i].copy_(s)
    if wl.n_shared_experts > 0:
        for name, tid, shape in (("gate", TID_SH_GATE, (Fs, H)), ("up", TID_SH_UP, (Fs, H)), ("down", TID_SH_DOWN, (H, Fs))):
            q, s = _matrix(wl, shape, tid, 0, device)
            out["sh_" + name] = q.contiguous()
            if s is not None:
                out["sh_s_" + name] = s
    return out


def gen_norm_weight(wl: Workload) -> torch.Tensor:
    """RMSNorm weight [H] in the activation dtype: 1 + N(0, norm_weight_std)."""
    a = 1.0 + _rng(wl.seed, TID_NORM).standard_normal(wl.hidden_size, np.float32) * np.float32(wl.norm_weight_std)
    return round_to(a, wl.act_dtype)


def gen_dispatch_counts(wl: Workload, num_tokens: Optional[int] = None) -> np.ndarray:
    """Rows each local expert of an expert-parallel rank receives: every token
    of the global batch (num_tokens * ep_size) picks num_experts_per_tok of
    the n_routed_experts * ep_size experts, so a given expert's count is
    Binomial(global tokens, k / global experts), drawn independently here."""
    T = wl.num_tokens if num_tokens is None else num_tokens
    n_global = T * wl.ep_size
    p = wl.num_experts_per_tok / (wl.n_routed_experts * wl.ep_size)
    return _rng(wl.seed, TID_DISPATCH_COUNT, T).binomial(n_global, p, wl.n_routed_experts).astype(np.int64)


def gen_dispatched_rows(wl: Workload, n_rows: int) -> torch.Tensor:
    """Token rows as they arrive from the dispatch exchange (grouped by local
    expert; each one is some token's layer input, so the same N(0, 1) law)."""
    a = _rng(wl.seed, TID_DISPATCH_ROWS, n_rows).standard_normal((n_rows, wl.hidden_size), np.float32)
    return round_to(a, wl.act_dtype)


def gen_inputs(wl: Workload, device="cpu", num_tokens: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """All inputs of one workload: x, router_w, router_bias and expert weights."""
    d = {"x": gen_x(wl, num_tokens), "router_w": gen_router(wl), "router_bias": gen_bias(wl)}
    d = {k: v.to(device) for k, v in d.items()}
    d.update(gen_expert_weights(wl, device))
    return d
