"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Small shapes (several tiles, ragged tails) are compared element by element.
The full Kimi-K2 shapes are compared on routing and grouping for every token
and on every output row: the decode batches and the DeepSeek-V3 shape through
the oracle's layer; the Zipf prefill (T=8192) and the fp8 layer (T=4096)
stage by stage, every grouped row of every expert against the oracle's
expert, the fp8 SwiGLU output's e4m3 codes and scales against the oracle's
activation quantisation, and every token through the oracle's combine.  Bars:
routing ids and grouping bit-exact, routing weights within 1e-5 relative,
outputs within max-abs-err <= tol * max|ref| (fp32 1e-4, bf16 1e-2,
fp8 5e-2), and each grouped row within tol of its own max|ref|.
"""
import numpy as np
import pytest
import torch

import cases
import oracle
from gpu_util import (TOL, Experts, block_err, check_h_codes, check_route, grouped_oracle, rel_err, rows_err,
                      run_block, run_layer, run_stages, say)
from sparse_moe_transformer_sigmoid_amd import binding as B
from sparse_moe_transformer_sigmoid_amd import inputs as gen

pytestmark = pytest.mark.gpu

W = gen.WORKLOADS


def small_case(wl, T):
    say(f"[case] {wl.name} T={T} seed={wl.seed} bias={wl.bias}")
    return cases.make_case(wl, device="cuda", num_tokens=T)


SMALL = [
    (W["tiny_fp32"], 16), (W["tiny_fp32"], 1), (W["tiny_fp32"], 37),
    # 1, 7, 28 tokens: streamed work items of 16, 16, 32 rows; 40 .. 1100
    # tokens: the LDS-tiled kernels with the K loop split over 2-4 blocks (few
    # work items, ragged last tiles); 4096: tiled, no split; intermediate
    # size 384 (not a multiple of the 256-feature gate_up slab) at 100 and 40
    # tokens and hidden size 640 (not a multiple of the 512-row down slab) at
    # 100 tokens: streamed items of 64 and 32 rows
    (W["small_bf16"], 1), (W["small_bf16"], 7), (W["small_bf16"], 28), (W["small_bf16"], 40),
    (W["small_bf16"], 100), (W["small_bf16"], 256), (W["small_bf16"], 257), (W["small_bf16"], 300),
    (W["small_bf16"], 1024), (W["small_bf16"], 4096),
    (W["small_bf16"].replace(name="small_bf16_f384", moe_intermediate_size=384), 100),
    (W["small_bf16"].replace(name="small_bf16_f384", moe_intermediate_size=384), 40),
    (W["small_bf16"].replace(name="small_bf16_h640", hidden_size=640), 100),
    # hidden size 2560 (40 K steps of 64) at 100 tokens: gate_up split over 7
    # K parts of 6, 6, 6, 6, 6, 6 and 4 steps
    (W["small_bf16"].replace(name="small_bf16_h2560", hidden_size=2560), 100),
    # the tiled kernels at 10 and 16 rows per expert (few work items: K
    # splits of both GEMMs)
    (W["small_bf16"].replace(name="small_bf16_h2560", hidden_size=2560), 40),
    (W["small_bf16"], 64),
    # 6.5 rows per expert: the streamed 32-row items (tiled from 7)
    (W["small_bf16"], 26),
    (W["small_bf16"].replace(name="small_bf16_e64", n_routed_experts=64), 1100),
    (W["small_grouped_bf16"], 100),
    (W["small_bf16"].replace(name="small_bf16_hot", bias="hot"), 300),
    (W["small_bf16"].replace(name="small_bf16_noshared", n_shared_experts=0), 50),
    (W["small_bf16"].replace(name="small_bf16_shared2", n_shared_experts=2), 50),
    # 64 experts and >= 512 tokens: the LDS-tiled router (128-token tiles, ragged tail)
    (W["small_bf16"].replace(name="small_bf16_e64", n_routed_experts=64), 600),
    (W["small_grouped_bf16"].replace(name="small_grouped_bf16_e64", n_routed_experts=64), 520),
    # fp8: streamed items of 16 rows (1, 7 tokens) and 32 rows (28, 44), tiled
    # from 12 rows per expert on; hidden size 640 does not fit the fp8 tiles, so 100
    # tokens stream in 64-row items and 40 in 32-row items
    (W["small_fp8"], 1), (W["small_fp8"], 7), (W["small_fp8"], 28), (W["small_fp8"], 44), (W["small_fp8"], 100),
    (W["small_fp8"], 300),
    (W["small_fp8"].replace(name="small_fp8_h640", hidden_size=640), 100),
    (W["small_fp8"].replace(name="small_fp8_h640", hidden_size=640), 40),
    (W["small_fp8"].replace(name="small_fp8_hot", bias="hot"), 200),
    # routing extremes: k = 32 (the largest supported), E = 1023 (the largest:
    # 16 experts per lane in top-k, 1024 groups in the single-block
    # grouping), 64 groups of 2 experts keeping 3, weights not renormalised
    (W["small_bf16"].replace(name="small_bf16_k32", n_routed_experts=64, num_experts_per_tok=32), 50),
    (W["small_bf16"].replace(name="small_bf16_e1023", n_routed_experts=1023, hidden_size=256,
                             moe_intermediate_size=128), 64),
    (W["small_bf16"].replace(name="small_bf16_g64", n_routed_experts=128, n_group=64, topk_group=3,
                             num_experts_per_tok=6), 100),
    (W["small_bf16"].replace(name="small_bf16_nonorm", norm_topk_prob=False, routed_scaling_factor=1.0), 100),
    (W["small_fp8"].replace(name="small_fp8_noshared", n_shared_experts=0), 50),
    # routing variants at decode sizes (the single-block grouping and work
    # list): grouped routing, k = 32, E = 1023 (16 experts per lane), no
    # renormalisation, fp8 with and without the shared expert
    (W["small_grouped_bf16"], 16),
    (W["small_bf16"].replace(name="small_bf16_g64", n_routed_experts=128, n_group=64, topk_group=3,
                             num_experts_per_tok=6), 3),
    (W["small_bf16"].replace(name="small_bf16_k32", n_routed_experts=64, num_experts_per_tok=32), 16),
    (W["small_bf16"].replace(name="small_bf16_e1023", n_routed_experts=1023, hidden_size=256,
                             moe_intermediate_size=128), 9),
    (W["small_bf16"].replace(name="small_bf16_nonorm", norm_topk_prob=False, routed_scaling_factor=1.0), 2),
    (W["small_fp8"], 16),
    (W["small_fp8"].replace(name="small_fp8_noshared", n_shared_experts=0), 5),
]


@pytest.mark.parametrize("wl,T", SMALL, ids=[f"{w.name}-T{t}" for w, t in SMALL])
def test_layer_matches_oracle_small(wl, T):
    case = small_case(wl, T)
    out, ids, w = run_layer(wl, case)
    ref, route = cases.oracle_forward(wl, case)
    check_route(ids, w, route)
    err = rel_err(out, ref)
    say(f"  rel err {err:.3e} (tol {TOL[wl.weight_dtype]})")
    assert err <= TOL[wl.weight_dtype]


def check_fp8_codes(x: torch.Tensor, sorted_ids: np.ndarray, codes: torch.Tensor, scales: torch.Tensor):
    """x_perm codes/scales are the oracle's activation quantisation of the
    gathered rows, bit for bit (same fp32 divide, RNE-saturating e4m3)."""
    _, q, s = oracle.act_quant(cases.to64(x)[sorted_ids])
    got_q = oracle.e4m3_decode(codes.cpu().numpy())
    assert np.array_equal(scales.cpu().numpy(), s), "activation scales differ"
    bad = np.argwhere(got_q != q)
    assert len(bad) == 0, f"{len(bad)} activation codes differ, first {bad[:3].tolist()}"


# up to 256 tokens the grouping (and, in the layer, the work list) is one
# single-block kernel; from 257 on, per-chunk histograms, a scan and a
# scatter over 256-token chunks (1024: four chunks)
@pytest.mark.parametrize("name,T", [("tiny_fp32", 16), ("small_bf16", 100), ("small_grouped_bf16", 100),
                                    ("small_fp8", 100), ("small_bf16", 256), ("small_bf16", 257),
                                    ("small_bf16", 1024), ("small_fp8", 257)])
def test_stages_match_oracle_and_layer(name, T):
    wl = W[name]
    case = small_case(wl, T)
    r = run_stages(wl, case)
    ref, route = cases.oracle_forward(wl, case)
    check_route(r["ids"], r["w"], route)
    offsets, sorted_ids, inv = oracle.permute(route.ids, wl.n_routed_experts)
    assert np.array_equal(r["offsets"].cpu().numpy(), offsets)
    assert np.array_equal(r["sorted"].cpu().numpy(), sorted_ids)
    assert np.array_equal(r["inv"].cpu().numpy(), inv)
    if wl.weight_dtype == gen.FP8:
        check_fp8_codes(case["x"], sorted_ids, r["x_perm"], r["x_perm_scales"])
    else:
        # the gathered rows are byte copies of x
        assert torch.equal(r["x_perm"], case["x"][r["sorted"].long()])
    assert rel_err(r["out"], ref) <= TOL[wl.weight_dtype]
    out, _, _ = run_layer(wl, case)
    assert torch.equal(out, r["out"]), "stage chain and fused layer differ"


@pytest.mark.parametrize("name,T", [("small_bf16", 300), ("small_bf16", 7), ("small_fp8", 300),
                                    ("small_grouped_bf16", 100), ("tiny_fp32", 37)])
def test_every_stage_is_deterministic(name, T):
    """Each stage run twice gives the same bits (fixed-order reductions, stable
    grouping, K-split partials added in part order), and so does the layer."""
    wl = W[name]
    case = small_case(wl, T)
    r1, r2 = run_stages(wl, case), run_stages(wl, case)
    for key, v in r1.items():
        if v is not None and key != "ws":   # (the workspace's unused bytes are arbitrary)
            assert torch.equal(v, r2[key]), f"stage output {key} differs between runs"
    a, ia, wa = run_layer(wl, case)
    b, ib, wb = run_layer(wl, case)
    assert torch.equal(a, b) and torch.equal(ia, ib) and torch.equal(wa, wb)


def test_zero_tokens_is_a_noop():
    wl = W["small_bf16"]
    case = small_case(wl, 4)
    case["x"] = case["x"][:0]
    out, ids, w = run_layer(wl, case)
    assert out.shape == (0, wl.hidden_size)


def test_zero_input_gives_zero_output():
    wl = W["small_bf16"]
    case = small_case(wl, 20)
    case["x"] = torch.zeros_like(case["x"])
    out, _, _ = run_layer(wl, case)
    assert torch.count_nonzero(out) == 0


# ---------------------------------------------------------------- full size --
@pytest.fixture(scope="module")
def k2_weights():
    wl = W["k2_decode_bf16"]
    say("[fixture] generating Kimi-K2 bf16 expert weights on the GPU")
    w = gen.gen_expert_weights(wl, device="cuda")
    torch.cuda.synchronize()
    return w


def full_case(wl, weights, T=None, experts=None):
    T = wl.num_tokens if T is None else T
    say(f"[case] {wl.name} T={T}")
    x = gen.gen_x(wl, T)
    rw, b = gen.gen_router(wl), gen.gen_bias(wl)
    x = cases.enforce_gap(wl, x, rw, b)
    d = {"x": x.cuda(), "router_w": rw.cuda(), "router_bias": b.cuda()}
    for k, v in weights.items():
        # the DeepSeek-V3-shaped workload uses the first 256 experts: the
        # generator draws expert e from the same stream for any E, so this is
        # the tensor it would generate for E = 256
        d[k] = v[:experts] if (experts is not None and k in ("w_gate", "w_up", "w_down")) else v
    return d


def check_sampled(wl, case, out, tokens):
    ref, _ = cases.oracle_forward(wl, case, tokens=np.asarray(tokens))
    err = rel_err(out[torch.as_tensor(tokens, device=out.device)], ref)
    say(f"  sampled tokens {list(tokens)}: rel err {err:.3e}")
    assert err <= TOL[wl.weight_dtype]


def full_route(wl, case):
    return oracle.route(cases.to64(case["x"]), cases.to64(case["router_w"]), cases.to64(case["router_bias"]),
                        **cases.route_kwargs(wl))


def check_every_row(wl, case, out, ids, w):
    """Routing of every token exact; every output row against the oracle's
    layer (the experts' fp64 weights prepared ahead on worker threads)."""
    route = full_route(wl, case)
    check_route(ids, w, route)
    fetch = Experts(wl, case, np.unique(route.ids))
    try:
        ref, _ = oracle.layer_forward(
            cases.to64(case["x"]), cases.to64(case["router_w"]), cases.to64(case["router_bias"]), fetch,
            cases.shared_weights(wl, case), fp8_act=(wl.weight_dtype == gen.FP8), route_result=route,
            **cases.route_kwargs(wl))
    finally:
        fetch.close()
    err = rel_err(out, ref)
    per_row = rows_err(out, ref)
    say(f"  active experts {len(np.unique(route.ids))}; every row: rel err {err:.3e}, worst row {per_row.max():.3e}")
    assert err <= TOL[wl.weight_dtype] and per_row.max() <= TOL[wl.weight_dtype]
    return route


@pytest.mark.timeout(600)
@pytest.mark.parametrize("T", [128, 1, 8, 300, 384, 512])
def test_k2_decode_full_size(k2_weights, T):
    """Every output row of the K2 decode layer at T tokens (streamed work
    items of 16 / 32 rows up to 300 tokens, tiled from 384)."""
    wl = W["k2_decode_bf16"]
    case = full_case(wl, k2_weights, T)
    out, ids, w = run_layer(wl, case)
    check_every_row(wl, case, out, ids, w)


def test_k2_one_token_layer_equals_stage_chain(k2_weights):
    """One token (T = 1, the smallest decode batch): for four different
    tokens the fused layer equals route -> permute -> expert FFN -> combine
    bit for bit and matches the oracle; so does the sub-block (RMSNorm,
    layer, residual)."""
    wl = W["k2_decode_bf16"]
    for b in range(4):
        x = cases.enforce_gap(wl, gen.gen_x(wl, 1, batch=10 + b), gen.gen_router(wl), gen.gen_bias(wl))
        case = full_case(wl, k2_weights, 1)
        case["x"] = x.cuda()
        out, ids, w = run_layer(wl, case)
        r = run_stages(wl, case)
        same = torch.equal(out, r["out"]) and torch.equal(ids, r["ids"])
        ref, route = cases.oracle_forward(wl, case)
        say(f"  token {b}: layer == stage chain: {same}, rel err {rel_err(out, ref):.3e}")
        assert same
        check_route(ids, w, route)
        assert rel_err(out, ref) <= TOL[wl.weight_dtype]
    case = full_block_case(wl, k2_weights, 1)
    out, ids, w = run_block(wl, case)
    ref, route, _ = cases.oracle_block(wl, case)
    check_route(ids, w, route)
    err = block_err(out, ref, cases.to64(case["x"]), wl.act_dtype)
    say(f"  sub-block, one token: err {err:.3e}")
    assert err <= TOL[wl.weight_dtype]


def check_grouped_rows(wl, case, r, route, hidden=None):
    """Stage chain at full size: grouping exact; every grouped row of every
    expert (y_perm) against the oracle's expert on that row; every shared row;
    every token's output through the oracle's combine of the oracle's rows.
    `hidden` (fp8): (codes, scales, shared codes, shared scales) of the
    SwiGLU output, checked against the oracle's quantisation of its h."""
    x64 = cases.to64(case["x"])
    offsets, sorted_ids, inv = oracle.permute(route.ids, wl.n_routed_experts)
    assert np.array_equal(r["offsets"].cpu().numpy(), offsets)
    assert np.array_equal(r["sorted"].cpu().numpy(), sorted_ids)
    assert np.array_equal(r["inv"].cpu().numpy(), inv)
    counts = np.diff(offsets)
    say(f"  active {int((counts > 0).sum())} empty {int((counts == 0).sum())} hottest {int(counts.max())}; "
        f"{int(np.sum((counts + 127) // 128))} work items of 128 rows")
    rows, y_ref, h_ref = grouped_oracle(wl, x64, sorted_ids, offsets, case, hidden=hidden is not None)
    assert np.array_equal(rows, np.arange(len(sorted_ids)))
    tol = TOL[wl.weight_dtype]
    per_row = rows_err(r["y_perm"], y_ref)
    worst = int(np.argmax(per_row))
    say(f"  every grouped row ({len(rows)}): worst row {worst} err {per_row[worst]:.3e}")
    assert per_row.max() <= tol
    sh = cases.shared_weights(wl, case)
    fp8 = wl.weight_dtype == gen.FP8
    h_sh = oracle.swiglu_hidden(x64, sh[0], sh[1], fp8_act=fp8)
    y_sh = (oracle.act_quant(h_sh)[0] if fp8 else h_sh) @ sh[2].T
    per_sh = rows_err(r["y_sh"], y_sh)
    say(f"  every shared row: worst {per_sh.max():.3e}")
    assert per_sh.max() <= tol
    if hidden is not None:
        check_h_codes(hidden[0], hidden[1], h_ref, "routed h codes")
        check_h_codes(hidden[2], hidden[3], h_sh, "shared h codes")
    ref_out = oracle.combine(y_ref, y_sh, route.weights, inv)
    err = rel_err(r["out"], ref_out)
    per_tok = rows_err(r["out"], ref_out)
    say(f"  every token: rel err {err:.3e}, worst token {per_tok.max():.3e}")
    assert err <= tol and per_tok.max() <= tol


def test_k2_prefill_zipf_full_size(k2_weights):
    """The Zipf-skewed prefill (T=8192, ~137 active experts, the hottest
    spanning ~31 work items of 128 rows): every grouped row, shared row and
    token against the oracle; the fused layer equal to the stage chain."""
    wl = W["k2_prefill_bf16_zipf"]
    case = full_case(wl, k2_weights)
    r = run_stages(wl, case)
    route = full_route(wl, case)
    check_route(r["ids"], r["w"], route)
    out, _, _ = run_layer(wl, case)
    assert torch.equal(out, r["out"])
    check_grouped_rows(wl, case, r, route)


@pytest.fixture(scope="module")
def k2_fp8_weights():
    wl = W["k2_fp8"]
    say("[fixture] generating Kimi-K2 fp8 expert weights on the GPU")
    w = gen.gen_expert_weights(wl, device="cuda")
    torch.cuda.synchronize()
    return w


def fp8_hidden_views(wl, r, T):
    """The SwiGLU output's e4m3 codes and scales left in the stage chain's
    workspace by moe_expert_ffn (routed and shared)."""
    cfg, ws = B.MoeConfig.from_fields(wl.fields()), r["ws"]
    k, F, Fs = wl.num_experts_per_tok, wl.moe_intermediate_size, wl.shared_intermediate_size
    return (B.workspace_view(ws, cfg, T, B.MOE_WS_H_CODES, torch.uint8, (T * k, F)),
            B.workspace_view(ws, cfg, T, B.MOE_WS_H_SCALES, torch.float32, (T * k, F // 128)),
            B.workspace_view(ws, cfg, T, B.MOE_WS_H_SHARED_CODES, torch.uint8, (T, Fs)),
            B.workspace_view(ws, cfg, T, B.MOE_WS_H_SHARED_SCALES, torch.float32, (T, Fs // 128)))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("T", [4096, 1, 64, 512])
def test_k2_fp8_full_size(k2_fp8_weights, T):
    """fp8 weights at K2 size.  T=4096 (the tiled fp8 kernels, 384 active
    experts): stage by stage, every grouped row, the e4m3 codes and scales of
    every SwiGLU output row, every token.  Smaller T (streamed items): every
    output row through the oracle's layer."""
    wl = W["k2_fp8"]
    case = full_case(wl, k2_fp8_weights, T)
    if T == 4096:
        r = run_stages(wl, case)
        route = full_route(wl, case)
        check_route(r["ids"], r["w"], route)
        _, sorted_ids, _ = oracle.permute(route.ids, wl.n_routed_experts)
        check_fp8_codes(case["x"], sorted_ids[:4096], r["x_perm"][:4096], r["x_perm_scales"][:4096])
        check_grouped_rows(wl, case, r, route, hidden=fp8_hidden_views(wl, r, T))
        out, _, _ = run_layer(wl, case)
        assert torch.equal(out, r["out"])
    else:
        out, ids, w = run_layer(wl, case)
        check_every_row(wl, case, out, ids, w)


@pytest.mark.parametrize("T", [64, 256, 7])
def test_moonlight_shape_full_size(T):
    """Second MoE shape on the pages (Moonlight-16B: hidden 2048, 64 experts
    top-6, 2 shared, d_ff 1408), compared element by element."""
    wl = W["moonlight_bf16"]
    case = small_case(wl, T)
    out, ids, w = run_layer(wl, case)
    ref, route = cases.oracle_forward(wl, case)
    check_route(ids, w, route)
    err = rel_err(out, ref)
    say(f"  rel err {err:.3e}")
    assert err <= TOL[wl.weight_dtype]


@pytest.mark.parametrize("T", [1, 16, 32, 128, 1024])
def test_dense_first_layer_full_size(T):
    """The dense first layer (SwiGLU 7168 -> 18432 -> 7168) as E = 1, k = 1,
    scale 1 through the same entry point; every row compared (streamed up to
    31 rows, tiled from 32, with the nontemporal weight DMA up to 128)."""
    wl = W["k2_dense_layer_bf16"]
    case = small_case(wl, T)
    out, ids, w = run_layer(wl, case)
    assert torch.all(ids == 0) and torch.all(w == 1.0)
    ref, _ = cases.oracle_forward(wl, case)
    err = rel_err(out, ref)
    say(f"  rel err {err:.3e}")
    assert err <= TOL[wl.weight_dtype]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("T", [1, 8, 32, 128, 512])
def test_dsv3_grouped_decode_full_size(k2_weights, T):
    """The DeepSeek-V3 shape (256 experts, 8 groups keeping 4): routing of
    every token and every output row."""
    wl = W["dsv3_decode_bf16"]
    case = full_case(wl, k2_weights, T, experts=256)
    out, ids, w = run_layer(wl, case)
    check_every_row(wl, case, out, ids, w)


@pytest.mark.parametrize("name", ["k2_ep128_rank_bf16", "k2_ep8_rank_bf16"])
def test_ep_rank_share_full_size(name):
    """One expert-parallel rank's share of the Kimi-K2 layer at decode (3 or
    48 local experts + shared, rows dispatched from 128 tokens per rank):
    moe_expert_ffn with k as the row capacity.  Every dispatched row and every
    shared row is compared with the oracle; the capacity rows past the last
    segment keep their sentinel."""
    wl = W[name]
    say(f"[case] {name} T={wl.num_tokens} ep_size={wl.ep_size}")
    case, cap = cases.make_rank_case(wl)
    cfg = B.MoeConfig.from_fields(dict(wl.fields(), num_experts_per_tok=cap))
    T, H = wl.num_tokens, wl.hidden_size
    R = int(case["offsets"][-1])
    say(f"  rows {R} (capacity {T * cap}), per expert {case['offsets'].diff().tolist()[:8]}...")
    sentinel = torch.tensor(1234.0, dtype=torch.bfloat16)
    y = torch.full((T * cap, H), sentinel.item(), dtype=torch.bfloat16, device="cuda")
    y_sh = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ws = B.alloc_workspace(cfg, T)
    B.moe_expert_ffn(cfg, B.MoeWeights.from_tensors(case), case["x"], case["x_rows"], None, case["offsets"],
                     y, y_sh, ws)
    torch.cuda.synchronize()
    assert torch.all(y[R:] == sentinel.to("cuda"))
    ref, ref_sh = cases.oracle_rank_share(wl, case)
    err, err_sh = rel_err(y[:R], ref), rel_err(y_sh, ref_sh)
    say(f"  rel err routed {err:.3e} shared {err_sh:.3e}")
    assert err <= TOL[wl.weight_dtype] and err_sh <= TOL[wl.weight_dtype]


# ------------------------------------------- the sub-block around the layer --
BLOCK = [
    (W["tiny_fp32"], 16), (W["small_bf16"], 1), (W["small_bf16"], 40), (W["small_bf16"], 300),
    (W["small_bf16"], 1024), (W["small_grouped_bf16"], 100), (W["small_fp8"], 100), (W["small_fp8"], 300),
]


@pytest.mark.parametrize("wl,T", BLOCK, ids=[f"{w.name}-T{t}" for w, t in BLOCK])
def test_block_matches_oracle_small(wl, T):
    """moe_block_forward = RMSNorm (fp64, one rounding) -> layer -> residual
    add, against the oracle's block_forward on every row."""
    say(f"[case] block {wl.name} T={T}")
    case = cases.make_block_case(wl, device="cuda", num_tokens=T)
    out, ids, w = run_block(wl, case)
    ref, route, _ = cases.oracle_block(wl, case)
    check_route(ids, w, route)
    err = block_err(out, ref, cases.to64(case["x"]), wl.act_dtype)
    say(f"  err {err:.3e} of max|layer part| (tol {TOL[wl.weight_dtype]})")
    assert err <= TOL[wl.weight_dtype]


def test_block_with_zero_experts_is_the_residual():
    """All expert weights zero: the output is the residual stream, bit for bit."""
    wl = W["small_bf16"]
    case = cases.make_block_case(wl, device="cuda", num_tokens=50)
    for k in ("w_gate", "w_up", "w_down", "sh_gate", "sh_up", "sh_down"):
        case[k] = torch.zeros_like(case[k])
    out, _, _ = run_block(wl, case)
    assert torch.equal(out, case["x"])


def full_block_case(wl, weights, T):
    say(f"[case] block {wl.name} T={T}")
    x = gen.gen_x(wl, T)
    g, rw, b = gen.gen_norm_weight(wl), gen.gen_router(wl), gen.gen_bias(wl)
    sc = cases.row_scales(T)
    g64, eps = cases.to64(g), cases.eps32(wl)
    x = cases.enforce_gap(wl, x, rw, b, transform=lambda x64, rows: oracle.round_act(
        oracle.rms_norm(x64 * sc[rows, None], g64, eps), wl.act_dtype))
    x = x * torch.from_numpy(sc).to(x.dtype)[:, None]
    d = {"x": x.cuda(), "norm_weight": g.cuda(), "router_w": rw.cuda(), "router_bias": b.cuda()}
    d.update(weights)
    return d


@pytest.mark.timeout(600)
@pytest.mark.parametrize("T", [128, 8])
def test_k2_block_decode_full_size(k2_weights, T):
    """The sub-block at K2 decode size: routing of every token and every
    output row."""
    wl = W["k2_decode_bf16"]
    case = full_block_case(wl, k2_weights, T)
    out, ids, w = run_block(wl, case)
    ref, route, _ = cases.oracle_block(wl, case)
    check_route(ids, w, route)
    err = block_err(out, ref, cases.to64(case["x"]), wl.act_dtype)
    say(f"  every row: err {err:.3e}")
    assert err <= TOL[wl.weight_dtype]


def test_k2_block_fp8_full_size(k2_fp8_weights):
    wl = W["k2_fp8"]
    T = 64
    case = full_block_case(wl, k2_fp8_weights, T)
    out, ids, w = run_block(wl, case)
    tokens = np.array([0, T - 1])
    ref, route, _ = cases.oracle_block(wl, case, tokens=tokens)
    check_route(ids, w, route, rows=tokens)
    err = block_err(out[torch.as_tensor(tokens, device="cuda")], ref, cases.to64(case["x"])[tokens], wl.act_dtype)
    say(f"  sampled tokens {list(tokens)}: err {err:.3e}")
    assert err <= TOL[wl.weight_dtype]


# ----------------------------------------------------------- graph capture --
# 100 tokens: the tiled kernels; 8 tokens: the streaming kernels, bf16 and
# fp8 (x quantised by the top-k launch, or by the norm pass of the block)
@pytest.mark.parametrize("name,block,T", [("small_bf16", False, 100), ("small_fp8", False, 100),
                                          ("small_bf16", True, 100), ("small_bf16", False, 8),
                                          ("small_fp8", False, 8), ("small_bf16", True, 8),
                                          ("small_fp8", True, 8)])
def test_layer_replays_from_a_graph(name, block, T):
    """The entry points launch kernels only (no memset, no host sync), so a
    call can be captured in a HIP graph: every replay -- with eager library
    calls and a change of input between replays -- equals the eager result
    on the same input, bit for bit."""
    wl = W[name]
    case = cases.make_block_case(wl, device="cuda", num_tokens=T) if block else small_case(wl, T)
    cfg = B.MoeConfig.from_fields(wl.fields())
    weights = B.MoeWeights.from_tensors(case)
    eps = float(np.float32(wl.rms_norm_eps))
    x = case["x"].clone()
    out = torch.empty((T, wl.hidden_size), dtype=gen.torch_dtype(wl.act_dtype), device="cuda")
    ids = torch.empty((T, wl.num_experts_per_tok), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, wl.num_experts_per_tok), dtype=torch.float32, device="cuda")
    ws = B.alloc_workspace(cfg, T)

    def call():
        if block:
            B.moe_block_forward(cfg, weights, x, case["norm_weight"], eps, case["router_w"], case["router_bias"],
                                out, ws, ids, wts)
        else:
            B.moe_layer_forward(cfg, weights, x, case["router_w"], case["router_bias"], out, ws, ids, wts)

    def eager(xin):
        c = dict(case)
        c["x"] = xin
        return (run_block if block else run_layer)(wl, c)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        call()
    torch.cuda.synchronize()
    inputs = [case["x"], case["x"].flip(0).contiguous(), case["x"]]
    for i, xin in enumerate(inputs + inputs):
        x.copy_(xin)
        out.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref_out, ref_ids, ref_w = eager(xin.clone())   # eager work between replays
        say(f"  replay {i}: equal={torch.equal(out, ref_out)}")
        assert torch.equal(out, ref_out) and torch.equal(ids, ref_ids) and torch.equal(wts, ref_w)


@pytest.mark.parametrize("name", ["k2_decode_bf16", "k2_prefill_bf16_zipf"])
def test_full_size_graph_replay_rotating_batches(k2_weights, name):
    """The launch configuration the benchmark times, at full size: one layer
    call per token batch captured in its own HIP graph (shared workspace),
    the graphs replayed in turn with eager calls in between.  Every replay
    equals the eager call on the same batch bit for bit, and sampled rows of
    each batch match the oracle."""
    wl = W[name]
    T = wl.num_tokens
    cfg = B.MoeConfig.from_fields(wl.fields())
    k = wl.num_experts_per_tok
    batches = []
    for b in range(2):
        case = full_case(wl, k2_weights, T)
        if b:
            x = cases.enforce_gap(wl, gen.gen_x(wl, T, batch=b), case["router_w"].cpu(), case["router_bias"].cpu())
            case["x"] = x.cuda()
        batches.append(case)
    weights = B.MoeWeights.from_tensors(batches[0])
    ws = B.alloc_workspace(cfg, T)
    bufs = [(torch.empty((T, wl.hidden_size), dtype=gen.torch_dtype(wl.act_dtype), device="cuda"),
             torch.empty((T, k), dtype=torch.int32, device="cuda"),
             torch.empty((T, k), dtype=torch.float32, device="cuda")) for _ in batches]

    def call(i):
        c = batches[i]
        B.moe_layer_forward(cfg, weights, c["x"], c["router_w"], c["router_bias"], bufs[i][0], ws, bufs[i][1],
                            bufs[i][2])

    side = torch.cuda.Stream()
    graphs = []
    for i in range(2):
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            call(i)
        torch.cuda.synchronize()
        graphs.append(g)
    refs = [run_layer(wl, c) for c in batches]
    for rep in range(4):
        i = rep % 2
        for o in bufs[i]:
            o.fill_(0)
        torch.cuda.synchronize()
        graphs[i].replay()
        torch.cuda.synchronize()
        run_layer(wl, batches[1 - i])   # eager work between replays
        same = all(torch.equal(a, r) for a, r in zip(bufs[i], refs[i]))
        say(f"  replay {rep} (batch {i}): equal={same}")
        assert same
    for i in range(2):
        check_sampled(wl, batches[i], bufs[i][0], [0, T // 2, T - 1])


@pytest.mark.parametrize("name,T", [("small_bf16", 300), ("small_bf16", 7), ("small_fp8", 100)])
def test_concurrent_calls_on_two_streams(name, T):
    """The library keeps no state between calls beyond the caller's buffers:
    two layer calls in flight at once on two streams, each with its own
    workspace and a different input, give the same bits as each call alone."""
    wl = W[name]
    case = small_case(wl, T)
    cfg = B.MoeConfig.from_fields(wl.fields())
    weights = B.MoeWeights.from_tensors(case)
    xs = [case["x"], case["x"].flip(0).contiguous()]
    refs = []
    for xin in xs:
        c = dict(case)
        c["x"] = xin
        refs.append(run_layer(wl, c))
    k = wl.num_experts_per_tok
    outs = [(torch.empty((T, wl.hidden_size), dtype=gen.torch_dtype(wl.act_dtype), device="cuda"),
             torch.empty((T, k), dtype=torch.int32, device="cuda"),
             torch.empty((T, k), dtype=torch.float32, device="cuda")) for _ in xs]
    wss = [B.alloc_workspace(cfg, T) for _ in xs]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]   # default priority
    torch.cuda.synchronize()
    for rep in range(3):
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                o, ids, w = outs[i]
                B.moe_layer_forward(cfg, weights, xs[i], case["router_w"], case["router_bias"], o, wss[i], ids, w)
        torch.cuda.synchronize()
        for i in range(2):
            assert all(torch.equal(a, b) for a, b in zip(outs[i], refs[i])), f"stream {i}, pass {rep}"


def test_k2_max_tokens_full_size(k2_weights):
    """The largest batch the ABI takes (65536 tokens, 524288 grouped rows:
    row offsets past 2^31 elements): routing of every token and the
    grouping are exact; sampled rows match the oracle."""
    wl = W["k2_prefill_bf16_zipf"]
    T = 65536
    case = full_case(wl, k2_weights, T)
    out, ids, w = run_layer(wl, case)
    route = full_route(wl, case)
    check_route(ids, w, route)
    check_sampled(wl, case, out, [0, T // 2 - 1, T - 1])
