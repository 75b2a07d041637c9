"""Pins of the CPU oracle against facts the pages and the mathematics fix (no GPU).

Every pin here uses something other than the oracle's own formula: numbers printed on the pages,
closed forms derived by hand, a library routine the method reduces to in a special case, an
independent second formulation, or invariants that a plausible mistake breaks.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import (OracleDims, cache_counts, decode_step_absorbed, decode_step_explicit, decode_step_precombined,
                    head_slices, load_rows, precombined_heads, precombined_weights, prefill_chunk, rope,
                    rope_frequencies, softmax, store_rows)
from synth import RUNNING_DIMS, V2_DIMS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_weights(dims, rng, sw=0.3, kappa=1.0):
    from synth.gen import weight_shapes
    W = {k: rng.standard_normal(s) * sw for k, s in weight_shapes(dims).items()}
    W["W_uq"] *= kappa
    W["W_qr"] *= kappa
    return W


SMALL = OracleDims(d=24, n_h=3, d_h=4, d_c=6, d_cq=5, d_r=4)
SMALL6 = OracleDims(d=24, n_h=3, d_h=4, d_c=8, d_cq=5, d_r=4)   # rows of whole 6-bit groups (12 codes)


# ---------------------------------------------------------------- printed values on the pages
def test_softmax_matches_pages_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "softmax_gate_example.json")))
    z = np.array(g["logits"])
    p = softmax(z)
    np.testing.assert_allclose(np.round(np.exp(z), 3), g["exps"], atol=0)
    assert round(float(np.exp(z).sum()), 3) == g["sum"]
    # the page divides its 3-decimal exponentials by its 3-decimal sum, then prints 3 decimals;
    # the exact probabilities therefore agree with the printed ones to within 1e-3
    np.testing.assert_allclose(np.round(np.array(g["exps"]) / g["sum"], 3), g["probs"], atol=0)
    assert np.max(np.abs(p - np.array(g["probs"]))) <= 1e-3
    assert abs(round(float(p.sum()), 3) - 1.0) == 0
    assert abs(p.sum() - 1.0) < 1e-15
    # shift invariance and no overflow at large logits
    np.testing.assert_allclose(softmax(z + 1000.0), p, rtol=1e-13)


def test_cache_counts_match_pages():
    g = json.load(open(os.path.join(GOLDEN, "cache_counts.json")))
    r = g["running_model"]
    d = r["dims"]
    c = cache_counts(d["n_h"], d["d_h"], d["d_c"], d["d_r"], d["layers"], d["bytes_per_elem"])
    for k in ("mha_per_layer", "mha_total", "mha_bytes", "mla_latent_only_per_layer",
              "mla_latent_only_total", "mla_latent_only_bytes", "mla_per_layer", "mla_total",
              "mla_bytes", "gqa_per_layer", "gqa_total", "mqa_per_layer", "mqa_total"):
        assert c[k] == r[k], k
    assert c["gqa_bytes"] / 1024 == r["gqa_bytes_kb"]
    assert c["mqa_bytes"] / 1024 == r["mqa_bytes_kb"]
    assert c["mla_bytes"] / 1024 == r["mla_kb"] and c["mha_bytes"] / 1024 == r["mha_kb"]
    assert c["gqa_equivalent_groups"] == r["gqa_equivalent_groups"]
    assert c["mla_bytes"] / c["mha_bytes"] == r["mla_over_mha_printed"]
    # the latent-only first attempt is 8x smaller than MHA
    assert c["mha_per_layer"] / c["mla_latent_only_per_layer"] == 8

    v = g["v2"]
    d = v["dims"]
    c = cache_counts(d["n_h"], d["d_h"], d["d_c"], d["d_r"], d["layers"])
    assert c["mha_per_layer"] == v["mha_per_layer"] and c["mla_per_layer"] == v["mla_per_layer"]
    assert c["mha_total"] == v["mha_total"] and c["mla_total"] == v["mla_total"]
    assert round(c["mla_over_mha"], 4) == v["ratio_printed"]
    assert round(1 / c["mla_over_mha"], 1) == v["reduction_printed"]
    assert round(1 / c["mla_over_mha"]) == v["about_times_fewer_printed"]
    assert c["gqa_equivalent_groups"] == v["gqa_equivalent_groups"]

    rules = g["dims_rules"]
    for dims in (V2_DIMS,):
        assert dims.d_c / dims.d_h == rules["d_c_over_d_h"]
        assert dims.d_r / dims.d_h == rules["d_r_over_d_h"]
        assert dims.row / dims.d_h == rules["row_over_d_h"]
    t = g["toy"]
    assert t["full_numbers"] * t["bytes_per_number"] == t["full_bytes"]
    assert t["latent_numbers"] * t["bytes_per_number"] == t["latent_bytes"]
    assert t["latent_bytes"] / t["full_bytes"] == t["ratio"]
    # the build's dims tables agree with the pages' dims
    assert RUNNING_DIMS.row == r["mla_per_layer"]
    assert V2_DIMS.row == v["mla_per_layer"]


def test_softmax_scale_constants():
    # 1/sqrt(d_h + d_h^R): sqrt(96) for the running model, sqrt(192) at the V2 shape
    assert RUNNING_DIMS.d_h + RUNNING_DIMS.d_r == 96
    assert V2_DIMS.d_h + V2_DIMS.d_r == 192


# ---------------------------------------------------------------- rotary embedding
def _rope_complex(x, pos, base):
    """Same rotation written with complex numbers: pair m is z_m = x_2m + i x_2m+1, multiplied by
    exp(i pos base^(-2m/n))."""
    n = x.shape[-1]
    z = x[..., 0::2] + 1j * x[..., 1::2]
    w = np.exp(1j * pos * base ** (-2.0 * np.arange(n // 2) / n))
    r = z * w
    out = np.empty(x.shape)
    out[..., 0::2] = r.real
    out[..., 1::2] = r.imag
    return out


@pytest.mark.parametrize("n", [2, 32, 64])
def test_rope_invariants(n):
    rng = np.random.default_rng(n)
    q, k = rng.standard_normal(n), rng.standard_normal(n)
    np.testing.assert_array_equal(rope(q, 0), q)                       # identity at position 0
    for pos in (1, 17, 4095, 131071):
        np.testing.assert_allclose(np.linalg.norm(rope(q, pos)), np.linalg.norm(q), rtol=1e-13)
        np.testing.assert_allclose(rope(q, pos), _rope_complex(q, pos, 10000.0), atol=1e-12)
    # the dot product depends on the position difference only
    for (t, j, dlt) in [(5, 2, 7), (100, 0, 1000), (131071, 3, -3)]:
        a = rope(q, t) @ rope(k, j)
        b = rope(q, t + dlt) @ rope(k, j + dlt)
        assert abs(a - b) < 1e-10 * (1 + abs(a))
    # composition: rotating by t then by s equals rotating by t + s
    np.testing.assert_allclose(rope(rope(q, 3), 5), rope(q, 8), atol=1e-12)


def test_rope_does_not_commute_with_projection():
    # the reason the rotary key is decoupled: RoPE(W c, t) != W RoPE(c, t) for a general W
    rng = np.random.default_rng(1)
    W = rng.standard_normal((8, 8))
    c = rng.standard_normal(8)
    assert np.linalg.norm(rope(W @ c, 5) - W @ rope(c, 5)) > 1e-3


# ---------------------------------------------------------------- absorption algebra
def test_absorption_identity_both_ways():
    rng = np.random.default_rng(2)
    for dims in (SMALL, OracleDims.of(RUNNING_DIMS)):
        W = _rand_weights(dims, rng)
        _, _, Wuk, Wuv, Wo = head_slices(W, dims)
        for i in range(dims.n_h):
            q = rng.standard_normal(dims.d_h)
            c = rng.standard_normal(dims.d_c)
            lhs = q @ (Wuk[i] @ c)                       # q^T (U c)
            rhs = (Wuk[i].T @ q) @ c                     # (U^T q)^T c
            assert abs(lhs - rhs) <= 1e-12 * (1 + abs(lhs))
            # value side: sum_j a_j W x_j = W sum_j a_j x_j, and W^O_i (W^UV_i x) = (W^O_i W^UV_i) x
            X = rng.standard_normal((7, dims.d_c))
            a = softmax(rng.standard_normal(7))
            np.testing.assert_allclose(sum(a[j] * (Wuv[i] @ X[j]) for j in range(7)), Wuv[i] @ (a @ X),
                                       rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(Wo[i] @ (Wuv[i] @ c), (Wo[i] @ Wuv[i]) @ c, rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("dims,T,cdtype", [
    (SMALL, 1, "f32"), (SMALL, 9, "f32"), (SMALL, 9, "bf16"), (SMALL, 9, "fp8_e4m3"),
    (OracleDims.of(RUNNING_DIMS), 33, "f16"), (OracleDims.of(RUNNING_DIMS), 64, "f32"),
    (OracleDims.of(V2_DIMS), 5, "bf16"), (OracleDims.of(V2_DIMS), 3, "fp8_e4m3"),
    (SMALL6, 9, "fp6_e2m3"), (OracleDims.of(V2_DIMS), 4, "fp6_e2m3"),
])
def test_explicit_equals_absorbed(dims, T, cdtype):
    """An independent formulation (scores against the latent with W^UK absorbed into the query,
    latent-weighted sum up-projected afterwards) agrees to 1e-10 relative."""
    rng = np.random.default_rng(T + dims.d)
    W = _rand_weights(dims, rng, sw=1.0 / math.sqrt(dims.d), kappa=3.0)
    h = rng.standard_normal(dims.d)
    stored, sc = store_rows(rng.standard_normal((T - 1, dims.d_c + dims.d_r)), cdtype)
    prefix = load_rows(stored, cdtype, sc)
    e = decode_step_explicit(W, h, prefix, dims, cdtype)
    a = decode_step_absorbed(W, h, prefix, dims, cdtype)
    for k in ("u", "o_lat", "lse"):
        err = np.linalg.norm(e[k] - a[k]) / np.linalg.norm(a[k])
        assert err < 1e-10, (k, err)


@pytest.mark.parametrize("dims,T,cdtype", [
    (SMALL, 1, "f32"), (SMALL, 9, "bf16"), (OracleDims.of(RUNNING_DIMS), 33, "f16"),
    (OracleDims.of(V2_DIMS), 4, "bf16"),
])
def test_precombined_equals_explicit(dims, T, cdtype):
    """The pre-combined form ([Scratch] sections 5.1-5.2: W~^Q_i = (W^UK_i)^T W^UQ_i and
    W~^O_i = W^O_i W^UV_i, stacked by head) with exact float64 matrices gives the explicit step's
    u, o_lat and lse to 1e-10: a transposed factor, a head block out of place or a wrong stacking
    axis breaks it."""
    rng = np.random.default_rng(3 * T + dims.d)
    W = _rand_weights(dims, rng, sw=1.0 / math.sqrt(dims.d), kappa=3.0)
    h = rng.standard_normal(dims.d)
    stored, sc = store_rows(rng.standard_normal((T - 1, dims.d_c + dims.d_r)), cdtype)
    prefix = load_rows(stored, cdtype, sc)
    if dims.d <= 512:
        Wq_pre, Wo_pre = precombined_weights(W, dims)
        assert Wq_pre.shape == (dims.n_h * dims.d_c, dims.d_cq) and Wo_pre.shape == (dims.d, dims.n_h * dims.d_c)
        # the stacked layout: row block i of Wq_pre is W~^Q_i, column block i of Wo_pre is W~^O_i
        _, _, Wuk, Wuv, Wo = head_slices(W, dims)
        Wuq = W["W_uq"].reshape(dims.n_h, dims.d_h, dims.d_cq)
        i = dims.n_h - 1
        np.testing.assert_allclose(Wq_pre[i * dims.d_c:(i + 1) * dims.d_c], Wuk[i].T @ Wuq[i], rtol=1e-12)
        np.testing.assert_allclose(Wo_pre[:, i * dims.d_c:(i + 1) * dims.d_c], Wo[i] @ Wuv[i], rtol=1e-12)
    e = decode_step_explicit(W, h, prefix, dims, cdtype)
    p = decode_step_precombined(W, precombined_heads(W, dims), h, prefix, dims, cdtype)
    for k in ("u", "o_lat", "lse"):
        err = np.linalg.norm(e[k] - p[k]) / np.linalg.norm(e[k])
        assert err < 1e-10, (k, err)


def test_precombined_weight_sizes():
    """Element counts of the pre-combined matrices against the factors they replace, from the
    pages' two shapes: at DeepSeek-V2 W~^Q is 3x and W~^O 3.6x the factors' elements; at the
    running model W~^Q is the smaller one."""
    def counts(D):
        wq = D.n_h * D.d_c * D.d_cq
        wo = D.d * D.n_h * D.d_c
        two_q = D.n_h * D.d_h * D.d_cq + D.n_h * D.d_h * D.d_c      # W^UQ + W^UK
        two_o = D.d * D.n_h * D.d_h + D.n_h * D.d_h * D.d_c         # W^O + W^UV
        return wq, wo, two_q, two_o
    wq, wo, tq, to = counts(V2_DIMS)
    assert (wq, tq) == (100_663_296, 33_554_432) and wq == 3 * tq
    assert (wo, to) == (335_544_320, 92_274_688) and abs(wo / to - 3.636) < 1e-3
    wq, wo, tq, to = counts(RUNNING_DIMS)
    assert (wq, tq) == (98_304, 114_688) and wq < tq
    assert (wo, to) == (524_288, 327_680) and wo > to


# ---------------------------------------------------------------- closed forms
def test_single_token_closed_form():
    """T = 1: the only weight is 1, so u = sum_i W^O_i W^UV_i c_0 and the query has no effect."""
    rng = np.random.default_rng(3)
    dims = SMALL
    W = _rand_weights(dims, rng)
    h = rng.standard_normal(dims.d)
    e = decode_step_explicit(W, h, np.zeros((0, dims.d_c + dims.d_r)), dims, "f32")
    c0 = e["read_new"][: dims.d_c]
    np.testing.assert_allclose(c0, (W["W_dkv"] @ h).astype(np.float32), rtol=0)
    ref = W["W_o"] @ (W["W_uv"] @ c0)          # u = W^O W^UV c_0 with full (unsliced) matrices
    np.testing.assert_allclose(e["u"], ref, rtol=1e-12)
    W2 = dict(W, W_uq=W["W_uq"] * -7.0, W_qr=W["W_qr"] * 5.0, W_dq=W["W_dq"] + 1.0)
    np.testing.assert_allclose(decode_step_explicit(W2, h, np.zeros((0, 10)), dims, "f32")["u"], ref, rtol=1e-12)
    assert np.allclose(e["lse"], e["lse"]) and np.all(e["alpha_max"] == 1.0)


def _hand_dims():
    return OracleDims(d=2, n_h=1, d_h=1, d_c=1, d_cq=1, d_r=2)


def test_hand_case_rotary_scores():
    """Tiny case solvable by hand; it pins the rotation direction, the pair layout, the position
    of the current token, the scale 1/sqrt(d_h + d_r) and the value sum.

    d=2, n_h=1, d_h=1, d_c=1, d_c'=1, d_r=2. h = (1, 1).
      W^DQ=[[1,0]] -> c^Q = 1;  W^UQ=[[1]] -> q^C = 1;  W^QR=[[1],[0]] -> raw q^R = (1, 0)
      W^DKV=[[0,1]] -> c_1 = 1;  W^KR=[[1,0],[0,0]] -> raw k^R = (1, 0);  W^UK=[[0]] (no content score)
      W^UV=[[1]], W^O=[[1],[0]].
    Prefix row (position 0): c_0 = 2, k^R_0 = (0, 1). Current token at position 1, angle 1 rad.
      q^R = (cos 1, sin 1), k^R_1 = (cos 1, sin 1)
      s_0 = q^R . k^R_0 / sqrt(3) = sin(1)/sqrt(3);   s_1 = 1/sqrt(3)
      alpha_0 = 1 / (1 + exp(s_1 - s_0));  u = (2 alpha_0 + 1 (1 - alpha_0), 0).
    """
    dims = _hand_dims()
    W = {"W_dq": np.array([[1.0, 0.0]]), "W_uq": np.array([[1.0]]), "W_qr": np.array([[1.0], [0.0]]),
         "W_dkv": np.array([[0.0, 1.0]]), "W_kr": np.array([[1.0, 0.0], [0.0, 0.0]]),
         "W_uk": np.array([[0.0]]), "W_uv": np.array([[1.0]]), "W_o": np.array([[1.0], [0.0]])}
    h = np.array([1.0, 1.0])
    prefix = np.array([[2.0, 0.0, 1.0]])
    e = decode_step_explicit(W, h, prefix, dims, "f32")
    s0, s1 = math.sin(1.0) / math.sqrt(3.0), 1.0 / math.sqrt(3.0)
    a0 = 1.0 / (1.0 + math.exp(s1 - s0))
    assert abs(e["u"][0] - (2 * a0 + (1 - a0))) < 1e-7 and e["u"][1] == 0.0
    assert abs(e["lse"][0] - math.log(math.exp(s0) + math.exp(s1))) < 1e-7
    # rotary key of the appended row, rotated by +1 rad (stored as float32)
    np.testing.assert_allclose(e["read_new"], [1.0, math.cos(1.0), math.sin(1.0)], atol=1e-7)


def test_hand_case_content_scores_two_heads():
    """Two heads, content scores only (W^QR = 0). Pins head slicing of W^UQ/W^UK/W^UV (row
    blocks) and of W^O (column blocks).

    d=2, n_h=2, d_h=1, d_c=2, d_c'=1, d_r=2; h=(1,0); W^DQ=[[1,0]] -> c^Q = 1.
      W^UQ = [[a],[b]] -> q^C_1 = a, q^C_2 = b.  W^UK = [[1,0],[0,1]]: head 1 sees c[0], head 2 c[1].
      W^UV = [[0,1],[1,0]]: head 1 values c[1], head 2 values c[0].
      W^O = [[1,0],[0,3]]: u_0 = o_1, u_1 = 3 o_2.  W^DKV = 0 -> the current row's latent is 0.
    Prefix: c_0 = (1, 2). Scores (scale 1/sqrt(3)): head 1 s = (a*1, 0)/sqrt3, head 2 s = (2b, 0)/sqrt3.
    """
    a, b = 0.7, -1.3
    dims = OracleDims(d=2, n_h=2, d_h=1, d_c=2, d_cq=1, d_r=2)
    W = {"W_dq": np.array([[1.0, 0.0]]), "W_uq": np.array([[a], [b]]), "W_qr": np.zeros((4, 1)),
         "W_dkv": np.zeros((2, 2)), "W_kr": np.zeros((2, 2)),
         "W_uk": np.array([[1.0, 0.0], [0.0, 1.0]]), "W_uv": np.array([[0.0, 1.0], [1.0, 0.0]]),
         "W_o": np.array([[1.0, 0.0], [0.0, 3.0]])}
    e = decode_step_explicit(W, np.array([1.0, 0.0]), np.array([[1.0, 2.0, 0.0, 0.0]]), dims, "f32")
    r3 = math.sqrt(3.0)
    a1 = 1.0 / (1.0 + math.exp(-a / r3))          # weight of row 0 in head 1
    a2 = 1.0 / (1.0 + math.exp(-2.0 * b / r3))    # weight of row 0 in head 2
    o1 = a1 * 2.0                                 # head 1 values c[1]: row0 -> 2, row1 -> 0
    o2 = a2 * 1.0                                 # head 2 values c[0]: row0 -> 1, row1 -> 0
    np.testing.assert_allclose(e["u"], [o1, 3.0 * o2], rtol=1e-12)


# ---------------------------------------------------------------- reduction to a library routine
def test_reduces_to_torch_sdpa():
    """With d_c = n_h d_h and W^UK = W^UV = I, the keys/values of head i are the i-th block of the
    latent (plus the shared rotary key), so the step is ordinary attention that torch's
    scaled_dot_product_attention computes (float64, explicit scale)."""
    rng = np.random.default_rng(5)
    n_h, d_h, d_r, T = 4, 8, 6, 37
    dims = OracleDims(d=20, n_h=n_h, d_h=d_h, d_c=n_h * d_h, d_cq=11, d_r=d_r)
    W = _rand_weights(dims, rng, sw=0.5)
    W["W_uk"] = np.eye(n_h * d_h)
    W["W_uv"] = np.eye(n_h * d_h)
    h = rng.standard_normal(dims.d)
    prefix = rng.standard_normal((T - 1, dims.d_c + d_r))
    e = decode_step_explicit(W, h, prefix, dims, "f32")

    # independent construction of q, K, V
    cQ = W["W_dq"] @ h
    qC = (W["W_uq"] @ cQ).reshape(n_h, d_h)
    qR = _rope_complex((W["W_qr"] @ cQ).reshape(n_h, d_r), T - 1, 10000.0)
    new = np.concatenate([W["W_dkv"] @ h, _rope_complex(W["W_kr"] @ h, T - 1, 10000.0)])
    new = new.astype(np.float32).astype(np.float64)        # f32 storage of the appended row
    rows = np.vstack([prefix, new])
    K = np.stack([np.concatenate([rows[:, i * d_h:(i + 1) * d_h], rows[:, n_h * d_h:]], 1) for i in range(n_h)])
    V = np.stack([rows[:, i * d_h:(i + 1) * d_h] for i in range(n_h)])
    q = np.concatenate([qC, qR], 1)[:, None, :]
    o = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(K), torch.from_numpy(V), scale=1.0 / math.sqrt(d_h + d_r))
    o = o.numpy()[:, 0, :]
    np.testing.assert_allclose(e["o"], o, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(e["u"], W["W_o"] @ o.reshape(-1), rtol=1e-11, atol=1e-13)


def test_stepwise_decode_equals_causal_attention():
    """Decoding tokens one at a time (each step appends its row) equals causal attention over the
    whole sequence computed at once (torch SDPA with a causal mask on explicitly built K/V)."""
    rng = np.random.default_rng(6)
    dims = SMALL
    W = _rand_weights(dims, rng, sw=0.6, kappa=2.0)
    N = 12
    H = rng.standard_normal((N, dims.d))
    prefix = np.zeros((0, dims.d_c + dims.d_r))
    us = []
    for t in range(N):
        e = decode_step_explicit(W, H[t], prefix, dims, "f32")
        us.append(e["u"])
        prefix = np.vstack([prefix, e["read_new"]])

    # whole-sequence form
    n_h, d_h, d_r = dims.n_h, dims.d_h, dims.d_r
    cQ = H @ W["W_dq"].T
    qC = (cQ @ W["W_uq"].T).reshape(N, n_h, d_h)
    qR = np.stack([_rope_complex((cQ[t] @ W["W_qr"].T).reshape(n_h, d_r), t, 10000.0) for t in range(N)])
    C = (H @ W["W_dkv"].T).astype(np.float32).astype(np.float64)
    KR = np.stack([_rope_complex(W["W_kr"] @ H[t], t, 10000.0) for t in range(N)]).astype(np.float32).astype(np.float64)
    kC = (C @ W["W_uk"].T).reshape(N, n_h, d_h)
    vC = (C @ W["W_uv"].T).reshape(N, n_h, d_h)
    q = np.concatenate([qC, qR], 2).transpose(1, 0, 2)
    k = np.concatenate([kC, np.repeat(KR[:, None, :], n_h, 1)], 2).transpose(1, 0, 2)
    v = vC.transpose(1, 0, 2)
    o = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=True,
        scale=1.0 / math.sqrt(d_h + d_r)).numpy()
    U = o.transpose(1, 0, 2).reshape(N, -1) @ W["W_o"].T
    np.testing.assert_allclose(np.array(us), U, rtol=1e-10, atol=1e-12)


def test_prefill_chunk_equals_masked_attention():
    """A chunk of C tokens after p0 stored rows equals attention computed at once over [prefix ;
    chunk rows] with an offset causal mask (query t sees keys 0 .. p0 + t): torch SDPA with an
    explicit boolean mask on explicitly built K/V."""
    rng = np.random.default_rng(8)
    dims = SMALL
    W = _rand_weights(dims, rng, sw=0.6, kappa=2.0)
    p0, C = 9, 6
    prefix = rng.standard_normal((p0, dims.d_c + dims.d_r))
    H = rng.standard_normal((C, dims.d))
    outs = prefill_chunk(W, H, prefix, dims, "f32")
    n_h, d_h, d_r = dims.n_h, dims.d_h, dims.d_r
    pos = np.arange(p0, p0 + C)
    cQ = H @ W["W_dq"].T
    qC = (cQ @ W["W_uq"].T).reshape(C, n_h, d_h)
    qR = np.stack([_rope_complex((cQ[t] @ W["W_qr"].T).reshape(n_h, d_r), pos[t], 10000.0) for t in range(C)])
    Cn = (H @ W["W_dkv"].T).astype(np.float32).astype(np.float64)
    KRn = np.stack([_rope_complex(W["W_kr"] @ H[t], pos[t], 10000.0) for t in range(C)]).astype(np.float32).astype(np.float64)
    Call = np.vstack([prefix[:, : dims.d_c], Cn])
    KRall = np.vstack([prefix[:, dims.d_c:], KRn])
    N = p0 + C
    kC = (Call @ W["W_uk"].T).reshape(N, n_h, d_h)
    vC = (Call @ W["W_uv"].T).reshape(N, n_h, d_h)
    q = np.concatenate([qC, qR], 2).transpose(1, 0, 2)                       # [n_h, C, d_h + d_r]
    k = np.concatenate([kC, np.repeat(KRall[:, None, :], n_h, 1)], 2).transpose(1, 0, 2)
    v = vC.transpose(1, 0, 2)
    mask = torch.from_numpy(np.arange(N)[None, :] <= pos[:, None])          # [C, N]
    o = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=mask,
        scale=1.0 / math.sqrt(d_h + d_r)).numpy()
    U = o.transpose(1, 0, 2).reshape(C, -1) @ W["W_o"].T
    np.testing.assert_allclose(np.array([r["u"] for r in outs]), U, rtol=1e-10, atol=1e-12)


def test_appended_row_is_rounded_like_storage():
    rng = np.random.default_rng(7)
    dims = OracleDims.of(RUNNING_DIMS)
    W = _rand_weights(dims, rng, sw=0.05)
    h = rng.standard_normal(dims.d)
    for cdtype, tdt in (("bf16", torch.bfloat16), ("f16", torch.float16)):
        e = decode_step_explicit(W, h, np.zeros((0, dims.d_c + dims.d_r)), dims, cdtype)
        ref = torch.from_numpy(e["row_new"].astype(np.float32)).to(tdt).to(torch.float64).numpy()
        np.testing.assert_array_equal(e["read_new"], ref)


def test_stage_helpers_agree_with_explicit_step():
    """absorbed_query / output_projection (used for stage-level GPU checks) reproduce the explicit
    step: scores from the absorbed query equal the explicit scores, and projecting the explicit
    step's attention-weighted latent gives its u."""
    from oracle import absorbed_query, output_projection
    rng = np.random.default_rng(11)
    dims = SMALL
    W = _rand_weights(dims, rng, sw=0.4, kappa=2.0)
    h = rng.standard_normal(dims.d)
    prefix = rng.standard_normal((6, dims.d_c + dims.d_r))
    e = decode_step_explicit(W, h, prefix, dims, "f32")
    q_lat, qR, row = absorbed_query(W, h, 6, dims)
    np.testing.assert_allclose(row, e["row_new"], rtol=1e-14)
    rows = np.vstack([prefix, e["read_new"]])
    s = (rows[:, :dims.d_c] @ q_lat.T + rows[:, dims.d_c:] @ qR.T) / np.sqrt(dims.d_h + dims.d_r)
    m = s.max(0)
    np.testing.assert_allclose(m + np.log(np.exp(s - m).sum(0)), e["lse"], rtol=1e-12)
    np.testing.assert_allclose(output_projection(W, e["o_lat"], dims), e["u"], rtol=1e-11)


# ---------------------------------------------------------------- YaRN-extended rotary frequencies
YARN = (40.0, 4096, 1.0, 32.0)   # factor s, original context L, ramp bounds alpha < beta (turns)


def test_yarn_factor_one_is_plain_rope():
    """s = 1 leaves every frequency (and so every rotation) as plain RoPE."""
    for n in (32, 64):
        np.testing.assert_array_equal(rope_frequencies(n, 10000.0, (1.0, 4096, 1.0, 32.0)),
                                      rope_frequencies(n, 10000.0))
    rng = np.random.default_rng(7)
    x = rng.standard_normal(64)
    np.testing.assert_array_equal(rope(x, 1234, 10000.0, (1.0, 4096, 1.0, 32.0)), rope(x, 1234, 10000.0))


def test_yarn_interpolates_slow_pairs_and_keeps_fast_ones():
    """Pairs turning fewer than alpha times over the original context are position-interpolated:
    their rotation at position s*p equals plain RoPE's at p. Pairs turning more than beta times are
    untouched. Pairs in between turn at a rate strictly between the two. All three kinds occur at
    d_r = 64 with L = 4096."""
    s, L, a, b = YARN
    n = 64
    plain = rope_frequencies(n, 10000.0)
    turns = L * plain / (2 * np.pi)
    slow, fast = turns < a, turns > b
    mid = ~slow & ~fast
    assert slow.any() and fast.any() and mid.any()
    rng = np.random.default_rng(8)
    x = rng.standard_normal(n)
    for p in (0, 3, 517, 4000):
        y_ext = rope(x, s * p, 10000.0, YARN)
        y_pln = rope(x, p, 10000.0)
        y_now = rope(x, p, 10000.0, YARN)
        for m in np.nonzero(slow)[0]:
            np.testing.assert_allclose(y_ext[2 * m:2 * m + 2], y_pln[2 * m:2 * m + 2], rtol=1e-9, atol=1e-9)
        for m in np.nonzero(fast)[0]:
            np.testing.assert_allclose(y_now[2 * m:2 * m + 2], y_pln[2 * m:2 * m + 2], rtol=1e-12, atol=1e-12)
    ext = rope_frequencies(n, 10000.0, YARN)
    assert np.all(ext[mid] < plain[mid]) and np.all(ext[mid] > plain[mid] / s)


def test_yarn_keeps_relative_position_property():
    """Scores after the extension still depend only on the offset between query and key."""
    rng = np.random.default_rng(9)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    for t, j, delta in ((10, 3, 1000), (4095, 17, 60000), (5, 5, 131000)):
        lhs = rope(q, t, 10000.0, YARN) @ rope(k, j, 10000.0, YARN)
        rhs = rope(q, t + delta, 10000.0, YARN) @ rope(k, j + delta, 10000.0, YARN)
        assert abs(lhs - rhs) <= 1e-9 * (1 + abs(lhs))


def test_yarn_explicit_equals_absorbed():
    """Both formulations agree with the extension on (frequencies and score scale shared)."""
    from dataclasses import replace
    dims = replace(OracleDims.of(V2_DIMS), yarn_factor=YARN[0], yarn_orig_len=YARN[1], yarn_alpha=YARN[2],
                   yarn_beta=YARN[3])
    rng = np.random.default_rng(10)
    W = _rand_weights(dims, rng, sw=1.0 / math.sqrt(dims.d), kappa=3.0)
    h = rng.standard_normal(dims.d)
    stored, sc = store_rows(rng.standard_normal((6, dims.d_c + dims.d_r)), "bf16")
    prefix = load_rows(stored, "bf16", sc)
    e = decode_step_explicit(W, h, prefix, dims, "bf16")
    a = decode_step_absorbed(W, h, prefix, dims, "bf16")
    for key in ("u", "o_lat", "lse"):
        assert np.linalg.norm(e[key] - a[key]) / np.linalg.norm(a[key]) < 1e-10, key
