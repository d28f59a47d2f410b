"""Pins of the fp64 oracle against what the pages and mathematics fix.

Each test names the passage (page title + table/section) or the closed form it
checks.  No expected value here comes from the HIP path or from the oracle
itself: they are page-printed numbers, hand-derived closed forms, brute force
over all subsets, or independent library routines (torch fp64, torch's e4m3
cast).  test_planted_mistakes_are_caught plants plausible bugs in the oracle
and checks that some pin fails for each.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import moe_oracle as om
from sparse_moe_transformer_sigmoid_amd import inputs as gen
import cases

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- P1 / P2 --
def check_param_counts():
    g = gold("down_proj_params.json")
    assert om.linear_params(g["out_features"], g["in_features"]) == g["per_instance"]
    assert om.linear_params(g["out_features"], g["in_features"]) * g["n_experts"] == g["per_layer_384_experts"]
    assert (om.linear_params(g["out_features"], g["in_features"]) * g["n_experts"] * g["moe_blocks"]
            == g["all_60_moe_blocks"])
    c = gold("k2_config_fields.json")
    # gate/up are [F, H], down is [H, F]: three equal-size linears per expert
    assert om.expert_params(c["hidden_size"], c["moe_intermediate_size"]) == 3 * g["per_instance"]


def test_p1_param_counts_match_down_projection_page():
    check_param_counts()


def test_p1_k2_workload_fields_match_config_table():
    c = gold("k2_config_fields.json")
    for name in ("k2_decode_bf16", "k2_prefill_bf16_zipf", "k2_fp8"):
        f = gen.WORKLOADS[name].fields()
        for key in ("hidden_size", "moe_intermediate_size", "n_routed_experts", "num_experts_per_tok",
                    "n_shared_experts", "n_group", "topk_group", "norm_topk_prob", "routed_scaling_factor"):
            assert f[key] == c[key], (name, key)
        assert gen.WORKLOADS[name].weight_std == c["initializer_range"]


def check_ep128_footprint():
    g = gold("ep128_footprint.json")
    c = gold("k2_config_fields.json")
    wbytes, sbytes = om.fp8_expert_bytes(c["hidden_size"], c["moe_intermediate_size"])
    assert wbytes == 44_040_192 and sbytes == 10_752
    dsv3 = g["dsv3_experts_per_rank"] * (g["num_hidden_layers"] - g["dsv3_dense_layers"]) * wbytes / 1e9
    k2 = g["k2_experts_per_rank"] * (g["num_hidden_layers"] - g["k2_dense_layers"]) * wbytes / 1e9
    # the page's figures are rounded ("about"); 1 B/param fp8 and a shared
    # expert as large as a routed one land within 10 % of both
    assert abs(dsv3 - g["dsv3_gb_approx"]) / g["dsv3_gb_approx"] < 0.10
    assert abs(k2 - g["k2_gb_approx"]) / g["k2_gb_approx"] < 0.10
    assert abs((k2 - dsv3) - g["extra_gb_approx"]) / g["extra_gb_approx"] < 0.25


def test_p2_ep128_footprints_match_section_2_1():
    check_ep128_footprint()


def test_dense_layer_params_match_a_few_hundred_mb():
    # first_k_dense_replace 1 with intermediate_size 18432 ("Kimi K2 Base" raw
    # config fields): one SwiGLU of 3 x 7168 x 18432 parameters, which at the
    # fp8 checkpoint's 1 B/param is "a few hundred MB" ("Behind Kimi-K2's
    # Config", section 2.3)
    n = om.expert_params(7168, 18432)
    assert n == 396_361_728
    assert 100e6 < n * 1 < 1e9
    wl = gen.WORKLOADS["k2_dense_layer_bf16"]
    assert (wl.n_routed_experts, wl.num_experts_per_tok, wl.n_shared_experts) == (1, 1, 0)
    assert wl.routed_scaling_factor == 1.0


def test_dense_layer_as_single_expert_is_plain_swiglu():
    # E = 1, k = 1, scale 1: the routed layer reduces to the expert itself
    rng = np.random.default_rng(11)
    x = rng.standard_normal((5, 24))
    ex, _ = small_weights(11, 1, 24, F=40)
    out, r = oracle.layer_forward(x, rng.standard_normal((1, 24)), np.zeros(1), lambda e: ex[0], None,
                                  num_experts_per_tok=1, routed_scaling_factor=1.0)
    assert np.all(r.weights == 1.0)
    np.testing.assert_allclose(out, torch_swiglu(x, *ex[0]), rtol=1e-12, atol=1e-12)


def test_moonlight_workload_matches_comparison_table():
    # "Kimi K2 Base" field comparison vs Moonlight 16B
    wl = gen.WORKLOADS["moonlight_bf16"]
    assert (wl.hidden_size, wl.n_routed_experts, wl.num_experts_per_tok, wl.n_shared_experts,
            wl.moe_intermediate_size) == (2048, 64, 6, 2, 1408)


def test_p12_prefill_flop_ratio_closed_form():
    # activated flops per token barely change between 256 and 384 experts
    # ("Behind Kimi-K2's Config", section 2.1, Prefill bullet)
    k2 = om.layer_flops(1, 7168, 2048, 384, 8, 1)
    ds = om.layer_flops(1, 7168, 2048, 256, 8, 1)
    assert k2 == 9 * 2 * 3 * 7168 * 2048 + 2 * 7168 * 384
    assert abs(k2 / ds - 1.0023) < 1e-4


# --------------------------------------------------------- worked examples --
def check_routing_worked_example():
    """Hand-derived: sigmoid(ln a) = a / (1 + a).

    logits = [0, ln 3, -ln 3, ln 9] -> scores [1/2, 3/4, 1/4, 9/10].
    bias   = [0.5, 0, 0.3, -0.5]    -> sel    [1.0, 0.75, 0.55, 0.4].
    top-2 by sel = {0, 1} (without the bias it would be {1, 3}); weights use
    the unbiased scores: [0.5, 0.75] / 1.25 * 2.827 = [1.1308, 1.6962].
    """
    x = np.array([[1.0]])
    w = np.array([[0.0], [math.log(3)], [-math.log(3)], [math.log(9)]])
    b = np.array([0.5, 0.0, 0.3, -0.5])
    r = oracle.route(x, w, b, num_experts_per_tok=2, routed_scaling_factor=2.827)
    assert r.ids.tolist() == [[0, 1]]
    np.testing.assert_allclose(r.weights, [[0.4 * 2.827, 0.6 * 2.827]], rtol=1e-14)
    r0 = oracle.route(x, w, np.zeros(4), num_experts_per_tok=2, routed_scaling_factor=2.827)
    assert r0.ids.tolist() == [[1, 3]]
    np.testing.assert_allclose(r0.weights, [[0.75 / 1.65 * 2.827, 0.9 / 1.65 * 2.827]], rtol=1e-14)
    # norm_topk_prob false: the scaled raw scores
    r1 = oracle.route(x, w, b, num_experts_per_tok=2, norm_topk_prob=False, routed_scaling_factor=2.0)
    np.testing.assert_allclose(r1.weights, [[1.0, 1.5]], rtol=1e-14)


def test_routing_worked_example():
    check_routing_worked_example()


def check_swiglu_worked_example():
    """Hand-derived: x = [2, 0]; W_gate = [[ln3 / 2, 5]] -> g = ln 3;
    W_up = [[1, 7]] -> u = 2; silu(ln 3) = ln 3 * 3/4; h = 1.5 ln 3;
    W_down = [[1], [-2]] -> y = [1.5 ln 3, -3 ln 3]."""
    x = np.array([[2.0, 0.0]])
    y = om.swiglu_expert(x, np.array([[math.log(3) / 2, 5.0]]), np.array([[1.0, 7.0]]),
                         np.array([[1.0], [-2.0]]))
    np.testing.assert_allclose(y, [[1.5 * math.log(3), -3 * math.log(3)]], rtol=1e-14)


def test_swiglu_worked_example():
    check_swiglu_worked_example()


# ---------------------------------------------------------------- P3 / P4 --
def tiny_router(seed=0, T=64, E=16, H=32, bias_std=0.01):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((T, H)), rng.standard_normal((E, H)) * 0.3, rng.standard_normal(E) * bias_std


def check_routing_invariants(x, w, b, k, **kw):
    r = oracle.route(x, w, b, num_experts_per_tok=k, **kw)
    T, E = r.scores.shape
    assert r.ids.shape == (T, k)
    for t in range(T):
        assert len(set(r.ids[t].tolist())) == k
        assert np.all(np.diff(r.ids[t]) > 0)
    np.testing.assert_allclose(r.weights.sum(1), kw.get("routed_scaling_factor", 2.827), rtol=1e-12)
    assert np.all(r.weights > 0)
    offsets, sorted_ids, inv = oracle.permute(r.ids, E)
    assert offsets[-1] == k * T and np.bincount(r.ids.ravel(), minlength=E).sum() == k * T
    # chosen experts' sel dominate the unchosen eligible ones
    for t in range(T):
        chosen = np.zeros(E, bool)
        chosen[r.ids[t]] = True
        others = r.sel[t][~chosen & r.eligible[t]]
        if len(others):
            assert r.sel[t][chosen].min() >= others.max()
    return r


def test_p3_routing_invariants_tiny_and_k2_router():
    x, w, b = tiny_router()
    check_routing_invariants(x, w, b, 4)
    wl = gen.WORKLOADS["k2_decode_bf16"]
    xr = cases.to64(gen.gen_x(wl, 64))
    check_routing_invariants(xr, cases.to64(gen.gen_router(wl)), cases.to64(gen.gen_bias(wl)), 8)


def check_bruteforce_topk(seed=1, k=4):
    x, w, b = tiny_router(seed, T=24)
    r = oracle.route(x, w, b, num_experts_per_tok=k)
    E = w.shape[0]
    for t in range(x.shape[0]):
        best = max(itertools.combinations(range(E), k), key=lambda s: r.sel[t, list(s)].sum())
        assert list(best) == r.ids[t].tolist()
        # weights: unbiased scores of the chosen set, renormalised, scaled
        s = 1.0 / (1.0 + np.exp(-(w[list(best)] @ x[t])))
        np.testing.assert_allclose(r.weights[t], s / s.sum() * 2.827, rtol=1e-12)


def test_p4_bruteforce_topk_all_subsets():
    check_bruteforce_topk()


def check_bruteforce_grouped(seed=2, E=16, n_group=4, topk_group=2, k=4):
    x, w, b = tiny_router(seed, T=24, E=E, bias_std=0.3)
    r = oracle.route(x, w, b, num_experts_per_tok=k, n_group=n_group, topk_group=topk_group)
    gsz = E // n_group
    for t in range(x.shape[0]):
        sel = r.sel[t]
        # a group's score: the best pair of sel values inside it
        gscore = [max(sel[g * gsz + i] + sel[g * gsz + j] for i in range(gsz) for j in range(i + 1, gsz))
                  for g in range(n_group)]
        gbest = max(itertools.combinations(range(n_group), topk_group), key=lambda s: sum(gscore[i] for i in s))
        allowed = [e for g in gbest for e in range(g * gsz, (g + 1) * gsz)]
        best = max(itertools.combinations(allowed, k), key=lambda s: sel[list(s)].sum())
        assert sorted(best) == r.ids[t].tolist()


def test_p4_bruteforce_grouped_topk():
    check_bruteforce_grouped()


# --------------------------------------------------------------------- P5 --
def test_p5_grouping_that_keeps_every_group_is_ungrouped():
    x, w, b = tiny_router(3)
    r0 = oracle.route(x, w, b, num_experts_per_tok=4)
    for ng in (2, 4, 16):
        r = oracle.route(x, w, b, num_experts_per_tok=4, n_group=ng, topk_group=ng)
        assert np.array_equal(r.ids, r0.ids)
        np.testing.assert_array_equal(r.weights, r0.weights)


def test_p5_zero_bias_selects_topk_logits():
    x, w, _ = tiny_router(4)
    r = oracle.route(x, w, np.zeros(w.shape[0]), num_experts_per_tok=4)
    logits = x @ w.T
    expect = np.sort(np.argsort(logits, axis=1)[:, -4:], axis=1)
    assert np.array_equal(r.ids, expect)


# ------------------------------------------------------------- P6 / P7 / P8 --
def torch_swiglu(x, wg, wu, wd):
    """Independent fp64 SwiGLU via torch library routines."""
    X = torch.from_numpy(np.asarray(x, np.float64))
    g = torch.matmul(X, torch.from_numpy(wg).T)
    u = torch.matmul(X, torch.from_numpy(wu).T)
    return torch.matmul(torch.nn.functional.silu(g) * u, torch.from_numpy(wd).T).numpy()


def small_weights(seed, E, H=24, F=16, Fs=16):
    rng = np.random.default_rng(seed)
    ex = [tuple(rng.standard_normal(s) * 0.2 for s in ((F, H), (F, H), (H, F))) for _ in range(E)]
    sh = tuple(rng.standard_normal(s) * 0.2 for s in ((Fs, H), (Fs, H), (H, Fs)))
    return ex, sh


def check_identical_experts(seed=5):
    rng = np.random.default_rng(seed)
    T, H, E, k = 20, 24, 8, 3
    x = rng.standard_normal((T, H))
    rw, b = rng.standard_normal((E, H)) * 0.3, rng.standard_normal(E) * 0.1
    ex, sh = small_weights(seed, 1, H)
    out, _ = oracle.layer_forward(x, rw, b, lambda e: ex[0], sh, num_experts_per_tok=k)
    expect = torch_swiglu(x, *sh) + 2.827 * torch_swiglu(x, *ex[0])
    np.testing.assert_allclose(out, expect, rtol=1e-12, atol=1e-12)


def test_p6_identical_experts_closed_form():
    check_identical_experts()


def check_single_expert(seed=6):
    rng = np.random.default_rng(seed)
    T, H = 9, 24
    x = rng.standard_normal((T, H))
    ex, sh = small_weights(seed, 1, H, F=16, Fs=32)
    out, r = oracle.layer_forward(x, rng.standard_normal((1, H)), np.zeros(1), lambda e: ex[0], sh,
                                  num_experts_per_tok=1)
    assert np.all(r.ids == 0) and np.allclose(r.weights, 2.827)
    np.testing.assert_allclose(out, torch_swiglu(x, *sh) + 2.827 * torch_swiglu(x, *ex[0]),
                               rtol=1e-12, atol=1e-12)


def test_p7_single_expert_is_textbook_swiglu():
    check_single_expert()


def test_p8_zero_input_and_invariances():
    rng = np.random.default_rng(7)
    T, H, E, k = 12, 24, 8, 3
    rw, b = rng.standard_normal((E, H)) * 0.3, rng.standard_normal(E) * 0.1
    ex, sh = small_weights(7, E, H)
    fwd = lambda xx: oracle.layer_forward(xx, rw, b, lambda e: ex[e], sh, num_experts_per_tok=k)[0]
    assert np.all(fwd(np.zeros((3, H))) == 0.0)
    x = rng.standard_normal((T, H))
    full = fwd(x)
    perm = rng.permutation(T)
    np.testing.assert_allclose(fwd(x[perm]), full[perm], rtol=1e-12, atol=1e-13)
    for t in range(T):
        np.testing.assert_allclose(fwd(x[t:t + 1])[0], full[t], rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------- P9 --
def all_e4m3_values():
    codes = np.arange(256, dtype=np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return codes, vals


def check_e4m3():
    codes, tv = all_e4m3_values()
    ov = om.e4m3_decode(codes)
    finite = ~np.isnan(tv)
    assert np.array_equal(np.isnan(ov), ~finite)
    np.testing.assert_array_equal(ov[finite], tv[finite])
    assert np.nanmax(tv) == 448.0
    # every representable value round-trips exactly
    np.testing.assert_array_equal(om.e4m3_round(tv[finite]), tv[finite])
    # midpoints (ties) and random values vs torch's RNE cast after clamping
    pos = np.unique(np.abs(tv[finite]))
    mids = (pos[1:] + pos[:-1]) / 2
    rng = np.random.default_rng(0)
    rnd = np.concatenate([rng.uniform(-500, 500, 20000), rng.standard_normal(20000) * 0.01,
                          rng.standard_normal(2000) * 1e-3, mids, -mids, [0.0, 447.9, 448.0, 460.0, 470.0, 1e6]])
    rnd = rnd.astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(np.clip(rnd, -448, 448)).to(torch.float32).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(om.e4m3_round(rnd), ref)


def test_p9_e4m3_matches_torch_cast():
    check_e4m3()


def test_p9_activation_quant_properties():
    rng = np.random.default_rng(8)
    v = (rng.standard_normal((5, 256)) * np.array([1.0, 1e-3, 10.0, 0.0, 1.0])[:, None]).astype(np.float32)
    deq, q, s = om.act_quant(v)
    assert s.dtype == np.float32 and s.shape == (5, 2)
    assert np.all(s[3] == 1.0) and np.all(deq[3] == 0.0)
    # each group's largest magnitude maps to +-448 and nothing exceeds it
    g = np.abs(q.reshape(5, 2, 128))
    assert np.all(g.max(axis=2)[[0, 1, 2, 4]] == 448.0) and g.max() <= 448.0
    # reconstruction error <= half an e4m3 step (relative 2^-4) plus subnormal floor
    err = np.abs(deq - v.astype(np.float64))
    bound = np.abs(v) * 2.0 ** -4 + np.repeat(s.astype(np.float64), 128, axis=1) * 2.0 ** -10
    assert np.all(err <= bound * (1 + 1e-6))


def test_p9_block_dequant_matches_decode_times_scale():
    rng = np.random.default_rng(9)
    codes = rng.integers(0, 256, (256, 384)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0
    scales = rng.uniform(0.5, 2, (2, 3)).astype(np.float32)
    w = om.dequant_weight(codes, scales)
    tv = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for i in range(2):
        for j in range(3):
            np.testing.assert_array_equal(w[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128],
                                          tv[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128] * float(scales[i, j]))


# -------------------------------------------------------------------- P10 --
def check_permutation(seed=10):
    x, w, b = tiny_router(seed, T=40)
    r = oracle.route(x, w, b, num_experts_per_tok=4)
    E, (T, k) = w.shape[0], r.ids.shape
    offsets, sorted_ids, inv = oracle.permute(r.ids, E)
    # brute force: walk experts in order, tokens in order
    pos, want_sorted, want_inv = 0, [], np.zeros(T * k, int)
    for e in range(E):
        assert offsets[e] == pos
        for t in range(T):
            for j in range(k):
                if r.ids[t, j] == e:
                    want_sorted.append(t)
                    want_inv[t * k + j] = pos
                    pos += 1
    assert offsets[E] == pos == T * k
    assert sorted_ids.tolist() == want_sorted
    assert inv.tolist() == want_inv.tolist()


def test_p10_stable_permutation_bruteforce():
    check_permutation()


def check_permutation_worked_example():
    """Hand-derived: E = 3, k = 2, ids [[2, 0], [2, 2], [-1, 1]] (token 1
    names expert 2 twice, token 2 names no expert in slot 0).  Expert 0 gets
    pair (0,1); expert 1 pair (2,1); expert 2 pairs (0,0), (1,0), (1,1) in
    flat order; pair (2,0) is not grouped."""
    offsets, sorted_ids, inv = oracle.permute(np.array([[2, 0], [2, 2], [-1, 1]]), 3)
    assert offsets.tolist() == [0, 1, 2, 5]
    assert sorted_ids.tolist() == [0, 2, 0, 1, 1]
    assert inv.tolist() == [2, 0, 3, 4, -1, 1]


def check_permutation_general(seed=11):
    """Loop definition on random ids with repeats and out-of-range values:
    walk experts in order, pairs in flat order; out-of-range pairs get -1."""
    rng = np.random.default_rng(seed)
    T, k, E = 50, 4, 7
    ids = rng.integers(-2, E + 2, (T, k))
    offsets, sorted_ids, inv = oracle.permute(ids, E)
    pos, want_sorted, want_inv = 0, [], [-1] * (T * k)
    for e in range(E):
        assert offsets[e] == pos
        for f in range(T * k):
            if ids[f // k, f % k] == e:
                want_sorted.append(f // k)
                want_inv[f] = pos
                pos += 1
    assert offsets[E] == pos == int(((ids >= 0) & (ids < E)).sum())
    assert sorted_ids.tolist() == want_sorted and inv.tolist() == want_inv


def test_p10_permutation_with_repeats_and_foreign_ids():
    check_permutation_worked_example()
    check_permutation_general()


def check_combine():
    """Hand-derived: y_perm rows [1,2], [3,4], [5,6], [7,8]; shared [[10,0],
    [0,10]]; weights [[0.5, 2], [1, -1]]; inv [3, 0, -1, 2]:
    out[0] = [10,0] + 0.5 [7,8] + 2 [1,2] = [15.5, 8];
    out[1] = [0,10] + (slot 0 not grouped) - [5,6] = [-5, 4]."""
    y = np.array([[1.0, 2], [3, 4], [5, 6], [7, 8]])
    out = oracle.combine(y, np.array([[10.0, 0], [0, 10]]), np.array([[0.5, 2], [1, -1]]), np.array([3, 0, -1, 2]))
    np.testing.assert_array_equal(out, [[15.5, 8], [-5, 4]])
    out0 = oracle.combine(y, None, np.array([[0.5, 2], [1, -1]]), np.array([3, 0, -1, 2]))
    np.testing.assert_array_equal(out0, [[5.5, 8], [-5, -6]])


def check_combine_is_the_layer_sum(seed=12):
    """The layer (step 8, each expert applied to its own tokens) equals the
    combine of the grouped expert outputs: permute, one SwiGLU per segment,
    combine (every slot grouped)."""
    rng = np.random.default_rng(seed)
    T, H, F, E, k = 12, 8, 6, 5, 2
    x, rw, b = rng.standard_normal((T, H)), rng.standard_normal((E, H)), rng.standard_normal(E) * 0.01
    ws = [tuple(rng.standard_normal(s) * 0.3 for s in ((F, H), (F, H), (H, F))) for _ in range(E + 1)]
    ref, r = oracle.layer_forward(x, rw, b, lambda e: ws[e], ws[E], num_experts_per_tok=k)
    offsets, sorted_ids, inv = oracle.permute(r.ids, E)
    y = np.zeros((T * k, H))
    for e in range(E):
        a, c = offsets[e], offsets[e + 1]
        if c > a:
            y[a:c] = om.swiglu_expert(x[sorted_ids[a:c]], *ws[e])
    out = oracle.combine(y, om.swiglu_expert(x, *ws[E]), r.weights, inv)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)


def test_combine_worked_example_and_layer_identity():
    check_combine()
    check_combine_is_the_layer_sum()


def check_gaps(seed=13):
    """selection_gap and group_gap by brute force on tiny inputs: the chosen
    set's smallest sel minus the largest eligible unchosen one; the kept
    groups' smallest score (top-2 sums taken by a loop) minus the largest
    dropped one, the kept set being the best of all C(4, 2) subsets."""
    x, w, b = tiny_router(seed, T=20, E=16, bias_std=0.3)
    r = oracle.route(x, w, b, num_experts_per_tok=4)
    gap = oracle.selection_gap(r, 4)
    for t in range(20):
        chosen = np.zeros(16, bool)
        chosen[r.ids[t]] = True
        assert math.isclose(gap[t], r.sel[t][chosen].min() - r.sel[t][~chosen].max(), rel_tol=0, abs_tol=1e-15)
    rg = oracle.route(x, w, b, num_experts_per_tok=4, n_group=4, topk_group=2)
    ggap = oracle.group_gap(rg, 4, 2)
    for t in range(20):
        sc = []
        for g in range(4):
            v = sorted(rg.sel[t, 4 * g:4 * g + 4].tolist(), reverse=True)
            sc.append(v[0] + v[1])
        kept = max(itertools.combinations(range(4), 2), key=lambda s: sum(sc[i] for i in s))
        dropped = [sc[i] for i in range(4) if i not in kept]
        assert math.isclose(ggap[t], min(sc[i] for i in kept) - max(dropped), rel_tol=0, abs_tol=1e-15)
    assert np.all(oracle.group_gap(r, 1, 1) == np.inf)
    assert np.all(oracle.selection_gap(r, 16) == np.inf)


def test_selection_and_group_gaps_bruteforce():
    check_gaps()


# -------------------------------------------------------------------- P11 --
def test_p11_active_expert_count_matches_expectation():
    # decode bytes scale with the number of distinct experts touched,
    # E (1 - (1 - k/E)^T) for independent uniform picks ("Behind Kimi-K2's
    # Config", section 2.1, Decode bullet: time follows parameters read).
    # With a zero correction bias the random router is close to uniform; the
    # N(0, 0.01) bias of the workloads skews it (fewer experts touched), which
    # is why measured bytes use the realised count.
    wl = gen.WORKLOADS["k2_decode_bf16"].replace(bias="zero")
    rw, b = cases.to64(gen.gen_router(wl)), cases.to64(gen.gen_bias(wl))
    for T in (32, 128):
        x = cases.to64(gen.gen_x(wl, T))
        r = oracle.route(x, rw, b, num_experts_per_tok=8)
        active = len(np.unique(r.ids))
        expect = 384 * (1 - (1 - 8 / 384) ** T)
        assert abs(active - expect) < 0.04 * expect, (T, active, expect)


# ------------------------------------------------------------ fp8 layer ----
def test_fp8_layer_matches_dequantised_reference():
    """fp8 mode = the same layer on q*s weights and q*s activations: with
    activation quantisation switched on, every expert sees act_quant(x) and
    act_quant(h).  Checked against torch fp64 on those dequantised inputs."""
    wl = gen.WORKLOADS["small_fp8"].replace(num_tokens=6)
    case = cases.make_case(wl)
    out, r = cases.oracle_forward(wl, case)
    ex, sh = cases.expert_fn(wl, case), cases.shared_weights(wl, case)
    xq = om.act_quant(cases.to64(case["x"]))[0]

    def f(xx, wg, wu, wd):
        X = torch.from_numpy(xx)
        h = torch.nn.functional.silu(X @ torch.from_numpy(wg).T) * (X @ torch.from_numpy(wu).T)
        h = torch.from_numpy(om.act_quant(h.numpy())[0])
        return (h @ torch.from_numpy(wd).T).numpy()

    expect = f(xq, *sh)
    for t in range(6):
        for j, e in enumerate(r.ids[t]):
            expect[t] += r.weights[t, j] * f(xq[t:t + 1], *ex(int(e)))[0]
    np.testing.assert_allclose(out, expect, rtol=1e-12, atol=1e-12)


# ------------------------------- the sub-block: RMSNorm + residual add ----
# ("Kimi K2 Base" architecture table: RMSNorm; raw config fields: rms_norm_eps)
def _bf16_neighbours(r):
    """The bf16 values just below and above a bf16 value r > 0 (one unit in
    the last of its 8 significant bits)."""
    _, e = np.frexp(r)             # r = m 2^e, m in [0.5, 1)
    ulp = np.ldexp(1.0, e - 8)
    return r - ulp, r + ulp


def check_round_bf16(seed=11):
    # library routine: torch's fp32 -> bf16 cast (round to nearest even) on
    # values that fp32 holds exactly
    v = np.random.default_rng(seed).standard_normal(20000).astype(np.float32).astype(np.float64)
    assert np.array_equal(om.round_bf16(v), torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).double().numpy())
    # the nearest value by definition, on fp64 values fp32 cannot hold
    w = np.abs(np.random.default_rng(seed + 1).standard_normal(2000)) + 1e-3
    r = om.round_bf16(w)
    lo, hi = _bf16_neighbours(r)
    assert np.all(np.abs(w - r) <= np.abs(w - lo)) and np.all(np.abs(w - r) <= np.abs(w - hi))
    # just above the midpoint 1 + 2^-8 of 1 and 1 + 2^-7: rounds up (a detour
    # through fp32 would land on the midpoint and round to even, i.e. down)
    assert om.round_bf16(np.array([1.0 + 2.0 ** -8 + 2.0 ** -40]))[0] == 1.0 + 2.0 ** -7
    # exact midpoints go to the even neighbour
    assert om.round_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    assert om.round_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6


def test_round_bf16_nearest_even_from_fp64():
    check_round_bf16()


def check_rms_norm(seed=12):
    rng = np.random.default_rng(seed)
    x, g = rng.standard_normal((5, 64)), 1.0 + 0.1 * rng.standard_normal(64)
    # library routine: torch's RMSNorm in fp64
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(g), 1e-6).numpy()
    np.testing.assert_allclose(om.rms_norm(x, g, 1e-6), ref, rtol=1e-14, atol=1e-14)
    # closed form: a constant row c gives g * c / sqrt(c^2 + eps)
    c, eps = -3.0, 0.25
    np.testing.assert_allclose(om.rms_norm(np.full((1, 8), c), np.ones(8), eps), c / math.sqrt(c * c + eps),
                               rtol=1e-15)
    # eps = 0: scale-free and of unit mean square
    u = om.rms_norm(x, np.ones(64), 0.0)
    np.testing.assert_allclose(om.rms_norm(7.5 * x, np.ones(64), 0.0), u, rtol=1e-14)
    np.testing.assert_allclose(np.mean(u * u, axis=1), 1.0, rtol=1e-14)


def test_rms_norm_matches_torch_and_closed_forms():
    check_rms_norm()


def check_block(seed=13):
    wl = gen.WORKLOADS["small_bf16"].replace(num_tokens=5, rms_norm_eps=0.0)
    case = cases.make_case(wl)
    x = cases.to64(case["x"]) * 3.0
    g = cases.to64(gen.gen_norm_weight(wl))
    kw = dict(cases.route_kwargs(wl))
    ex, sh = cases.expert_fn(wl, case), cases.shared_weights(wl, case)
    rw, b = cases.to64(case["router_w"]), cases.to64(case["router_bias"])
    out, r, u = om.block_forward(x, g, 0.0, rw, b, ex, sh, **kw)
    # the residual: out - x is the layer applied to u, u the bf16 rounding of the norm
    np.testing.assert_array_equal(u, om.round_bf16(om.rms_norm(x, g, 0.0)))
    y, _ = om.layer_forward(u, rw, b, ex, sh, **kw)
    np.testing.assert_allclose(out - x, y, rtol=0, atol=1e-12)
    # eps = 0: the layer part does not depend on the scale of x
    out2, _, _ = om.block_forward(0.25 * x, g, 0.0, rw, b, ex, sh, **kw)
    np.testing.assert_allclose(out2 - 0.25 * x, out - x, rtol=0, atol=1e-12)
    # all-zero expert weights: only the residual is left
    zero = tuple(np.zeros_like(m) for m in sh)
    out3, _, _ = om.block_forward(x, g, 0.0, rw, b, lambda e: zero, zero, **kw)
    np.testing.assert_array_equal(out3, x)


def test_block_is_residual_plus_layer_on_rounded_norm():
    check_block()


# ------------------------------------------------------ planted mistakes ---
PINS = [check_param_counts, check_routing_worked_example, check_swiglu_worked_example,
        check_bruteforce_topk, check_bruteforce_grouped, check_identical_experts,
        check_single_expert, check_e4m3, check_permutation, check_permutation_worked_example,
        check_permutation_general, check_combine, check_combine_is_the_layer_sum, check_gaps,
        check_round_bf16, check_rms_norm, check_block]


def _any_pin_fails():
    for p in PINS:
        try:
            p()
        except AssertionError:
            return True
    return False


MUTANTS = {
    "weights_from_biased_scores": ("route", lambda orig: (
        lambda x, w, b, **kw: _weights_from(orig(x, w, b, **kw), "sel", kw))),
    "no_renormalisation": ("route", lambda orig: (
        lambda x, w, b, **kw: orig(x, w, b, **{**kw, "norm_topk_prob": False}))),
    "bottom_k": ("_top_indices", lambda orig: (lambda v, n: orig(-v, n))),
    "silu_sign": ("silu", lambda orig: (lambda z: z / (1.0 + np.exp(z)))),
    "drop_shared": ("swiglu_expert", None),
    "gate_up_swapped": ("swiglu_expert", lambda orig: (
        lambda x, wg, wu, wd, fp8_act=False: orig(x, wu, wg, wd, fp8_act))),
    "group_max_not_top2": ("group_scores", lambda orig: (
        lambda sel, ng: np.sort(sel.reshape(sel.shape[0], ng, -1), axis=2)[:, :, -1])),
    "e4m3_truncate": ("e4m3_round", lambda orig: (lambda v: _trunc_e4m3(v))),
    "permute_unstable": ("permute", lambda orig: (lambda ids, E: _unstable_permute(orig, ids, E))),
    "permute_clips_foreign_ids": ("permute", lambda orig: (lambda ids, E: orig(np.clip(ids, 0, E - 1), E))),
    "combine_wraps_minus_one": ("combine", lambda orig: (
        lambda y, ysh, w, inv: orig(y, ysh, w, np.where(np.asarray(inv) < 0, np.asarray(inv) + len(y), inv)))),
    "combine_drops_shared": ("combine", lambda orig: (lambda y, ysh, w, inv: orig(y, None, w, inv))),
    "selection_gap_next_pair": ("selection_gap", lambda orig: (
        lambda r, k: orig(r, k + 1) if k + 1 < r.sel.shape[1] else orig(r, k))),
    "group_gap_next_pair": ("group_gap", lambda orig: (
        lambda r, ng, tg: orig(r, ng, tg + 1) if 1 < tg + 1 < ng else orig(r, ng, tg))),
    "expert_params_two_linears": ("expert_params", lambda orig: (lambda h, f: 2 * h * f)),
    "bf16_via_fp32": ("round_bf16", lambda orig: (
        lambda v: torch.from_numpy(np.asarray(v, np.float64).astype(np.float32)).to(torch.bfloat16).double().numpy())),
    "norm_mean_abs": ("rms_norm", lambda orig: (
        lambda x, g, eps: np.asarray(x) / (np.mean(np.abs(x), axis=1, keepdims=True) + eps) * g)),
    "norm_eps_outside_sqrt": ("rms_norm", lambda orig: (
        lambda x, g, eps: np.asarray(x) / (np.sqrt(np.mean(np.asarray(x) ** 2, axis=1, keepdims=True)) + eps) * g)),
    "block_no_residual": ("block_forward", lambda orig: (
        lambda x, *a, **kw: (lambda o: (o[0] - (np.asarray(x, np.float64) if kw.get("tokens") is None
                                               else np.asarray(x, np.float64)[kw["tokens"]]), o[1], o[2]))(
            orig(x, *a, **kw)))),
}


def _weights_from(r, field, kw):
    w = np.take_along_axis(getattr(r, field), r.ids, axis=1)
    r.weights = w / w.sum(1, keepdims=True) * kw.get("routed_scaling_factor", 2.827)
    return r


def _trunc_e4m3(v):
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    _, e = np.frexp(np.where(a > 0, a, 1.0))
    q = np.ldexp(1.0, np.maximum(e - 1, -6) - 3)
    return np.copysign(np.minimum(np.floor(a / q) * q, 448.0), v)


def _unstable_permute(orig, ids, E):
    offsets, s, inv = orig(ids, E)
    for e in range(E):
        a, b = offsets[e], offsets[e + 1]
        s[a:b] = s[a:b][::-1]
    return offsets, s, inv


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_planted_mistakes_are_caught(mutant, monkeypatch):
    assert not _any_pin_fails()
    fname, make = MUTANTS[mutant]
    orig = getattr(om, fname)
    if mutant == "drop_shared":
        calls = {"n": 0}

        def patched(x, wg, wu, wd, fp8_act=False):
            calls["n"] += 1
            y = orig(x, wg, wu, wd, fp8_act)
            return 0 * y if calls["n"] == 1 else y
        # the first expert evaluated in layer_forward is the shared one
        monkeypatch.setattr(om, "layer_forward", _fresh_counter(om.layer_forward, calls))
        monkeypatch.setattr(om, fname, patched)
    else:
        monkeypatch.setattr(om, fname, make(orig))
    monkeypatch.setattr(oracle, fname, getattr(om, fname), raising=False)
    if hasattr(oracle, "layer_forward"):
        monkeypatch.setattr(oracle, "layer_forward", om.layer_forward)
    assert _any_pin_fails(), f"planted mistake {mutant} went unnoticed"


def _fresh_counter(fn, calls):
    def wrapped(*a, **kw):
        calls["n"] = 0
        return fn(*a, **kw)
    return wrapped
