"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test checks one oracle function against a published table, a library routine,
a closed form, an invariant, or a brute-force computation written independently
(pure-Python loops / exact rationals) on tiny inputs.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from bit_moe_expert_amd import workloads as wl
from tests.conftest import read_golden


# ----------------------------------------------------------------------------
# Number formats
# ----------------------------------------------------------------------------
def test_e2m1_all_codes_match_ocp_table():
    rows = read_golden("e2m1_values.txt")
    codes = np.array([c for c, _ in rows])
    want = np.array([v for _, v in rows])
    got = oracle.e2m1_value(codes)
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))  # code 8 is -0


def test_e4m3_all_codes_match_torch_float8():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_value(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_e4m3_landmarks_match_ofp8_spec():
    for code, val in read_golden("e4m3_landmarks.txt"):
        got = float(oracle.e4m3_value(np.array([code]))[0])
        if math.isnan(val):
            assert math.isnan(got)
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), hex(code)


def test_bf16_value_matches_torch():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 1 << 16, 4096).astype(np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]  # finite values only
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.bf16_value(bits), ref)


def _rne_bf16_exact(v: float) -> float:
    """Round to 8 significant bits, ties to even, in exact rationals (normal range)."""
    if v == 0:
        return v
    f = Fraction(v)
    sign = -1 if f < 0 else 1
    f = abs(f)
    e = 0
    while f >= 2:
        f /= 2
        e += 1
    while f < 1:
        f *= 2
        e -= 1
    q = f * 128
    n = math.floor(q)
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * float(Fraction(n, 128) * Fraction(2) ** e)


def test_bf16_round_exact_rationals_and_ties():
    rng = np.random.default_rng(12)
    v = rng.standard_normal(2000) * np.exp2(rng.integers(-30, 30, 2000))
    # exact ties: a BF16 value plus half its ulp, and the same minus half
    base = oracle.bf16_value(rng.integers(0x3000, 0x4F00, 200).astype(np.uint16))
    half = np.exp2(np.floor(np.log2(base)) - 8)
    v = np.concatenate([v, base + half, base - half, -(base + half), [0.0, -0.0]])
    got = oracle.bf16_round(v)
    want = np.array([_rne_bf16_exact(float(a)) for a in v])
    assert np.array_equal(got, want)


def test_bf16_round_matches_torch_on_float32_values():
    rng = np.random.default_rng(13)
    v = (rng.standard_normal(100000) * 1e3).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.bf16_round(v.astype(np.float64)), ref)


def test_unpack_codes_low_nibble_first():
    rng = np.random.default_rng(2)
    codes = rng.integers(0, 16, (3, 64)).astype(np.uint8)
    packed = np.zeros((3, 32), dtype=np.uint8)
    for r in range(3):
        for j in range(32):
            packed[r, j] = int(codes[r, 2 * j]) + 16 * int(codes[r, 2 * j + 1])
    assert np.array_equal(oracle.unpack_codes(packed), codes)


def test_dequant_matches_elementwise_definition_and_is_exact_in_bf16():
    rng = np.random.default_rng(3)
    N, K = 5, 64
    packed = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    scales = wl.to_e4m3_codes(np.exp2(rng.uniform(-4, 2, (N, K // 16))))
    ts = 0.5
    W = oracle.dequant(packed, scales, ts)
    e2m1 = dict(read_golden("e2m1_values.txt"))
    sc = torch.from_numpy(scales).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for n in range(N):
        for k in range(K):
            byte = int(packed[n, k // 2])
            code = byte & 15 if k % 2 == 0 else byte >> 4
            assert W[n, k] == e2m1[code] * sc[n, k // 16] * ts
    # code * scale has <= 6 significant bits: BF16 holds it exactly
    bf = torch.from_numpy(W).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(bf, W)


def test_dequant_full_e4m3_range_products_exact_in_bf16():
    # every (code, scale) pair of the formats, tensor scale 1
    codes = np.arange(16)
    scales = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    prod = oracle.e2m1_value(codes)[:, None] * oracle.e4m3_value(scales)[None, :]
    bf = torch.from_numpy(prod).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(bf, prod)


# ----------------------------------------------------------------------------
# Router, top-k, plan
# ----------------------------------------------------------------------------
def test_router_logits_brute_force_exact():
    rng = np.random.default_rng(4)
    T, E, H = 3, 4, 16
    x = wl.to_bf16_bits(rng.standard_normal((T, H)))
    wr = wl.to_bf16_bits(rng.standard_normal((E, H)) * 0.02)
    got = oracle.router_logits(x, wr)
    xf = oracle.bf16_value(x)
    wf = oracle.bf16_value(wr)
    for t in range(T):
        for e in range(E):
            exact = sum(Fraction(float(xf[t, h])) * Fraction(float(wf[e, h])) for h in range(H))
            assert abs(Fraction(float(got[t, e])) - exact) <= abs(exact) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 80)


def _margin_logits(T, E, k, seed):
    w = wl.Workload("t", T=T, H=128, E=E, k=k, I=128, routing="normal", margin=1e-3)
    return wl._draw_logits(np.random.SeedSequence(seed), w, T)


@pytest.mark.parametrize("E,k", [(8, 2), (128, 8), (160, 8), (256, 8), (7, 7), (5, 1)])
def test_route_matches_torch_topk_and_softmax(E, k):
    L = _margin_logits(64, E, k, seed=E * 31 + k)
    idx, w = oracle.route(L, k)
    tl = torch.from_numpy(L.astype(np.float64))
    vals, ti = torch.topk(tl, k, dim=1, largest=True, sorted=True)
    assert np.array_equal(idx, ti.numpy().astype(np.int32))
    ref_w = torch.softmax(vals, dim=1).numpy()
    np.testing.assert_allclose(w, ref_w, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-13)


def test_route_k_equals_e_is_full_softmax_and_k1_is_one():
    L = _margin_logits(16, 6, 5, seed=9)
    idx, w = oracle.route(L, 6)
    full = torch.softmax(torch.from_numpy(L.astype(np.float64)), dim=1).numpy()
    np.testing.assert_allclose(w, np.take_along_axis(full, idx.astype(np.int64), 1), rtol=1e-13)
    idx1, w1 = oracle.route(L, 1)
    assert np.all(w1 == 1.0)
    assert np.array_equal(idx1[:, 0], np.argmax(L, axis=1))


def test_route_ties_go_to_lower_index():
    L = np.array([[1.0, 3.0, 3.0, 0.5, 3.0, 2.0]])
    idx, w = oracle.route(L, 4)
    assert idx.tolist() == [[1, 2, 4, 5]]
    np.testing.assert_allclose(w[0, :3], w[0, 0])


@pytest.mark.parametrize("T,k,E,mode", [(64, 8, 128, "uniform"), (16, 2, 8, "uniform"),
                                        (40, 4, 16, "one_hot_expert"), (1, 8, 128, "uniform"),
                                        (12, 6, 6, "all_experts"), (30, 2, 64, "sparse")])
def test_permute_matches_stable_argsort(T, k, E, mode):
    rng = np.random.default_rng(T * k + E)
    if mode == "one_hot_expert":
        idx = np.full((T, k), 3, dtype=np.int32)
        idx[:, 1:] = rng.integers(0, E, (T, k - 1))
    elif mode == "all_experts":
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    elif mode == "sparse":
        idx = rng.choice([5, 9, 63], (T, k)).astype(np.int32)
    else:
        idx = rng.integers(0, E, (T, k)).astype(np.int32)
    offsets, perm, inv = oracle.permute(idx, E)
    flat = idx.reshape(-1)
    assert np.array_equal(perm, np.argsort(flat, kind="stable").astype(np.int32))
    assert np.array_equal(np.diff(offsets), np.bincount(flat, minlength=E))
    assert offsets[0] == 0 and offsets[-1] == flat.size
    assert np.array_equal(perm[inv], np.arange(flat.size))   # perm o inv = id
    assert np.array_equal(inv[perm], np.arange(flat.size))   # inv o perm = id
    assert np.array_equal(flat[perm], np.sort(flat, kind="stable"))


def test_permute_empty():
    offsets, perm, inv = oracle.permute(np.zeros((0, 4), dtype=np.int32), 8)
    assert offsets.tolist() == [0] * 9 and perm.size == 0 and inv.size == 0


# ----------------------------------------------------------------------------
# Expert FFN
# ----------------------------------------------------------------------------
def _brute_swiglu(x, w13, w2, bf16_acts=True):
    """Pure-Python loops, math.exp, exact-rational rounding: independent of numpy's
    matmul and of the oracle's rounding. With bf16_acts the hidden and output
    activations are rounded to BF16 as W4A16 prescribes."""
    rnd = _rne_bf16_exact if bf16_acts else (lambda v: v)
    R, H = x.shape
    I = w13.shape[0] // 2
    out = np.zeros((R, w2.shape[0]))
    for r in range(R):
        a = []
        for i in range(I):
            g = math.fsum(float(x[r, h]) * float(w13[i, h]) for h in range(H))
            u = math.fsum(float(x[r, h]) * float(w13[I + i, h]) for h in range(H))
            a.append(rnd(g / (1.0 + math.exp(-g)) * u))
        for n in range(w2.shape[0]):
            out[r, n] = rnd(math.fsum(float(w2[n, i]) * a[i] for i in range(I)))
    return out


def test_swiglu_ffn_brute_force():
    rng = np.random.default_rng(5)
    R, H, I = 3, 32, 16
    x = oracle.bf16_value(wl.to_bf16_bits(rng.standard_normal((R, H))))
    w13 = oracle.dequant(rng.integers(0, 256, (2 * I, H // 2)).astype(np.uint8),
                         wl.to_e4m3_codes(np.exp2(rng.uniform(-4, 2, (2 * I, H // 16)))), 1.0)
    w2 = oracle.dequant(rng.integers(0, 256, (H, I // 2)).astype(np.uint8),
                        wl.to_e4m3_codes(np.exp2(rng.uniform(-4, 2, (H, I // 16)))), 1.0)
    got = oracle.swiglu_ffn(x, w13, w2)
    want = _brute_swiglu(x, w13, w2)
    # BF16 outputs: equal, except where fp64 summation order moves a value across a
    # rounding boundary (then one BF16 ulp apart)
    ulp = np.exp2(np.floor(np.log2(np.abs(want))) - 7)
    assert np.all(np.abs(got - want) <= ulp)
    assert np.mean(got == want) > 0.98
    # the hidden activation alone (unrounded): brute force with W2 = identity
    eye = np.eye(I)
    np.testing.assert_allclose(oracle.swiglu_hidden(x, w13), _brute_swiglu(x, w13, eye, bf16_acts=False),
                               rtol=1e-11, atol=1e-9)


def test_e1_k1_layer_is_a_dense_swiglu_mlp_via_torch():
    """E=1, k=1: every token goes to the one expert with weight 1; the layer is a
    dense SwiGLU MLP + residual + RMSNorm, computed here with torch library ops on
    weights decoded through torch's float8 type and the OCP E2M1 table."""
    w = wl.Workload("dense", T=6, H=128, E=1, k=1, I=128, routing="normal")
    inp = wl.make_inputs(w, seed=11)
    out = oracle.layer(inp)
    assert np.all(out["idx"] == 0) and np.all(out["w"] == 1.0)
    e2m1 = torch.tensor([v for _, v in read_golden("e2m1_values.txt")], dtype=torch.float64)

    def deq(m):
        p = torch.from_numpy(m.packed[0].astype(np.int64))
        codes = torch.stack([p & 15, p >> 4], dim=-1).reshape(p.shape[0], -1)
        sc = torch.from_numpy(m.scales[0]).view(torch.float8_e4m3fn).to(torch.float64)
        return e2m1[codes] * sc.repeat_interleave(16, dim=1) * float(m.tscale[0])

    x = torch.from_numpy(inp.x.view(np.int16)).view(torch.bfloat16).double()
    r = torch.from_numpy(inp.residual.view(np.int16)).view(torch.bfloat16).double()
    g = torch.from_numpy(inp.gamma.view(np.int16)).view(torch.bfloat16).double()
    W13, W2 = deq(inp.w13), deq(inp.w2)
    I = w.I
    hmid = torch.nn.functional.silu(x @ W13[:I].T) * (x @ W13[I:].T)
    # BF16 activations (rounding pinned on its own above)
    hmid = torch.from_numpy(oracle.bf16_round(hmid.numpy()))
    o = r + torch.from_numpy(oracle.bf16_round((hmid @ W2.T).numpy()))
    n = torch.nn.functional.rms_norm(o, (w.H,), weight=g, eps=w.eps)
    np.testing.assert_allclose(out["o"], o.numpy(), rtol=1e-12, atol=1e-10)
    np.testing.assert_allclose(out["n"], n.numpy(), rtol=1e-12, atol=1e-10)


def test_expert_outputs_equal_per_token_loop():
    w = wl.workload("tiny")
    inp = wl.make_inputs(w, seed=0)
    idx, _ = oracle.route(inp.logits, w.k)
    y = oracle.expert_outputs(inp.x, idx, inp.w13, inp.w2)
    x = oracle.bf16_value(inp.x)
    for t in (0, 5, 15):
        for j in range(w.k):
            e = int(idx[t, j])
            W13 = oracle.dequant(inp.w13.packed[e], inp.w13.scales[e], inp.w13.tscale[e])
            W2 = oracle.dequant(inp.w2.packed[e], inp.w2.scales[e], inp.w2.tscale[e])
            np.testing.assert_allclose(y[t, j], oracle.swiglu_ffn(x[t:t + 1], W13, W2)[0], rtol=1e-11)


# ----------------------------------------------------------------------------
# Combine + RMSNorm
# ----------------------------------------------------------------------------
def test_combine_norm_matches_torch_rms_norm():
    rng = np.random.default_rng(6)
    T, k, H = 5, 3, 64
    y = rng.standard_normal((T, k, H))
    w = rng.random((T, k))
    res = wl.to_bf16_bits(rng.standard_normal((T, H)))
    gam = wl.to_bf16_bits(rng.uniform(0.5, 1.5, H))
    sh = rng.standard_normal((T, H))
    o, n = oracle.combine_norm(y, w, res, gam, 1e-6, shared=sh)
    o_ref = oracle.bf16_value(res) + sum(w[:, j:j + 1] * y[:, j] for j in range(k)) + sh
    np.testing.assert_allclose(o, o_ref, rtol=1e-14, atol=1e-14)
    n_ref = torch.nn.functional.rms_norm(torch.from_numpy(o_ref), (H,),
                                         weight=torch.from_numpy(oracle.bf16_value(gam)), eps=1e-6)
    np.testing.assert_allclose(n, n_ref.numpy(), rtol=1e-13, atol=1e-14)


def test_combine_norm_closed_forms():
    rng = np.random.default_rng(7)
    T, k, H = 4, 2, 128
    res = wl.to_bf16_bits(rng.standard_normal((T, H)))
    ones = wl.to_bf16_bits(np.ones(H))
    r = oracle.bf16_value(res)
    # y = 0: o = r, n = r / rms(r)
    o, n = oracle.combine_norm(np.zeros((T, k, H)), np.full((T, k), 0.5), res, ones, 1e-12)
    np.testing.assert_array_equal(o, r)
    np.testing.assert_allclose(n, r / np.sqrt(np.mean(r * r, axis=1, keepdims=True)), rtol=1e-12)
    # gamma = 1: rms(n) = 1 (eps small against mean square)
    np.testing.assert_allclose(np.sqrt(np.mean(n * n, axis=1)), 1.0, rtol=1e-10)
    # scale invariance of the norm: n(c * o) = n(o) for c = 4 (exact power of two)
    y = rng.standard_normal((T, k, H))
    w = rng.random((T, k))
    _, n1 = oracle.combine_norm(y, w, res, ones, 1e-30)
    res4 = wl.to_bf16_bits(4 * r)
    _, n4 = oracle.combine_norm(4 * y, w, res4, ones, 1e-30)
    np.testing.assert_allclose(n4, n1, rtol=1e-12)


# ----------------------------------------------------------------------------
# RMSNorm glue: add_rmsnorm and group_rmsnorm
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("group", [8, 24, 96])
def test_group_rmsnorm_matches_torch_rms_norm_per_group(group):
    # the library routine applied to each group's slice (a reshape), gamma after it
    rng = np.random.default_rng(11)
    T, H = 5, 96
    x = wl.to_bf16_bits(rng.standard_normal((T, H)) * rng.uniform(0.1, 10, (T, 1)))
    gam = wl.to_bf16_bits(rng.uniform(0.5, 1.5, H))
    n = oracle.group_rmsnorm(x, group, gam, 1e-6)
    xv = torch.from_numpy(oracle.bf16_value(x)).reshape(T, H // group, group)
    ref = torch.nn.functional.rms_norm(xv, (group,), eps=1e-6).reshape(T, H)
    ref = ref * torch.from_numpy(oracle.bf16_value(gam))
    np.testing.assert_allclose(n, ref.numpy(), rtol=1e-13, atol=1e-14)


def test_add_rmsnorm_matches_torch_rms_norm():
    rng = np.random.default_rng(12)
    T, H = 6, 128
    x = wl.to_bf16_bits(rng.standard_normal((T, H)))
    res = wl.to_bf16_bits(rng.standard_normal((T, H)))
    gam = wl.to_bf16_bits(rng.uniform(0.5, 1.5, H))
    o, n = oracle.add_rmsnorm(x, res, gam, 1e-6)
    # the sum of two BF16 values is exact in fp64
    o_ref = torch.from_numpy(oracle.bf16_value(x)) + torch.from_numpy(oracle.bf16_value(res))
    np.testing.assert_array_equal(o, o_ref.numpy())
    n_ref = torch.nn.functional.rms_norm(o_ref, (H,), weight=torch.from_numpy(oracle.bf16_value(gam)), eps=1e-6)
    np.testing.assert_allclose(n, n_ref.numpy(), rtol=1e-13, atol=1e-14)


def test_group_rmsnorm_closed_forms():
    ones = wl.to_bf16_bits(np.ones(32))
    # a constant group c: every value becomes sign(c) (eps small against c^2)
    x = np.concatenate([np.full(8, -3.0), np.full(8, 0.5), np.full(16, 2.0)])[None, :]
    n = oracle.group_rmsnorm(wl.to_bf16_bits(x), 8, ones, 1e-30)
    np.testing.assert_allclose(n[0], np.sign(x[0]), rtol=1e-14)
    # one group of size H is the plain norm; groups differing only by a power-of-two
    # scale normalise to the same values
    rng = np.random.default_rng(13)
    v = rng.standard_normal(8)
    x2 = np.concatenate([v, 4 * v, 0.25 * v, v])[None, :]
    n2 = oracle.group_rmsnorm(wl.to_bf16_bits(x2), 8, ones, 1e-30)
    for g in range(1, 4):
        np.testing.assert_allclose(n2[0, 8 * g:8 * g + 8], n2[0, :8], rtol=1e-12)
    # gamma = 1: each group's rms is 1
    x3 = wl.to_bf16_bits(rng.standard_normal((3, 32)))
    n3 = oracle.group_rmsnorm(x3, 16, ones, 1e-30).reshape(3, 2, 16)
    np.testing.assert_allclose(np.sqrt(np.mean(n3 * n3, axis=2)), 1.0, rtol=1e-12)
    # a brute-force pure-Python loop on a tiny row with eps mattering
    xs = [1.0, -2.0, 0.5, 4.0, 0.0, 0.0, 0.0, 0.0]
    gs = [1.0, 0.5, 2.0, 1.5, 1.0, 1.0, 1.0, 1.0]
    eps = 0.25
    want = []
    for g0 in (0, 4):
        ms = sum(v * v for v in xs[g0:g0 + 4]) / 4
        want += [xs[h] / math.sqrt(ms + eps) * gs[h] for h in range(g0, g0 + 4)]
    got = oracle.group_rmsnorm(wl.to_bf16_bits(np.array([xs])), 4, wl.to_bf16_bits(np.array(gs)), eps)
    np.testing.assert_allclose(got[0], want, rtol=1e-15, atol=0)
    with pytest.raises(ValueError):
        oracle.group_rmsnorm(x3, 12, ones, 1e-6)


# ----------------------------------------------------------------------------
# Whole layer: per-token independence
# ----------------------------------------------------------------------------
def test_layer_rows_are_independent_of_batch():
    w = wl.workload("tiny")
    inp = wl.make_inputs(w, seed=0)
    full = oracle.layer(inp)
    sub = oracle.layer(inp, tokens=np.array([3, 7, 11]))
    np.testing.assert_array_equal(sub["idx"], full["idx"][[3, 7, 11]])
    # equal up to the rounding order of the library matmul
    np.testing.assert_allclose(sub["o"], full["o"][[3, 7, 11]], rtol=1e-11)
    np.testing.assert_allclose(sub["n"], full["n"][[3, 7, 11]], rtol=1e-11)


def test_layer_composition_matches_steps():
    w = wl.workload("tiny")
    inp = wl.make_inputs(w, seed=0)
    out = oracle.layer(inp)
    offsets, perm, inv = oracle.permute(out["idx"], w.E)
    assert np.array_equal(out["perm_src"], perm) and np.array_equal(out["inv"], inv)
    assert np.array_equal(out["offsets"], offsets)
    np.testing.assert_allclose(out["w"].sum(axis=1), 1.0, atol=1e-14)


# ----------------------------------------------------------------------------
# Whole layer with the shared expert (TensorFold issue #627, jschmied's Oct 14
# comment: a shared expert runs beside the routed chain, ungated)
# ----------------------------------------------------------------------------
def _torch_dequant(m, e):
    """One expert of a grouped 4-bit tensor, decoded with torch's float8 type for the
    E4M3 scales and the OCP E2M1 table from the golden file (not the oracle's)."""
    e2m1 = torch.tensor([v for _, v in read_golden("e2m1_values.txt")], dtype=torch.float64)
    p = torch.from_numpy(m.packed[e].astype(np.int64))
    codes = torch.stack([p & 15, p >> 4], dim=-1).reshape(p.shape[0], -1)
    sc = torch.from_numpy(m.scales[e]).view(torch.float8_e4m3fn).to(torch.float64)
    return e2m1[codes] * sc.repeat_interleave(16, dim=1) * float(m.tscale[e])


def test_layer_with_shared_expert_matches_torch_composition():
    """The layer with one shared expert, composed independently from torch library
    ops: torch.topk + torch.softmax routing, a per-token loop over the selected
    experts' SwiGLU FFNs (torch silu, BF16 activations), the shared expert's dense
    SwiGLU FFN on every token with weight 1, the residual, then torch rms_norm."""
    w = wl.Workload("shared_pin", T=7, H=128, E=6, k=2, I=128, routing="normal", n_shared=1)
    inp = wl.make_inputs(w, seed=21)
    out = oracle.layer(inp)
    bf = lambda t: torch.from_numpy(oracle.bf16_round(t.numpy()))  # rounding pinned above
    val = lambda bits: torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double()
    x, r, g = val(inp.x), val(inp.residual), val(inp.gamma)
    L = torch.from_numpy(inp.logits.astype(np.float64))
    sel = torch.topk(L, w.k, dim=1)  # margins >= 1e-3: no ties
    p = torch.softmax(L, dim=1).gather(1, sel.indices)
    p = p / p.sum(dim=1, keepdim=True)
    I = w.I

    def ffn(xr, W13, W2):
        hmid = bf(torch.nn.functional.silu(xr @ W13[:I].T) * (xr @ W13[I:].T))
        return bf(hmid @ W2.T)

    experts = {e: (_torch_dequant(inp.w13, e), _torch_dequant(inp.w2, e)) for e in range(w.E)}
    routed = torch.zeros((w.T, w.H), dtype=torch.float64)
    for t in range(w.T):
        for j in range(w.k):
            e = int(sel.indices[t, j])
            routed[t] += p[t, j] * ffn(x[t:t + 1], *experts[e])[0]
    shared = ffn(x, _torch_dequant(inp.shared13, 0), _torch_dequant(inp.shared2, 0))
    o = r + routed + shared
    n = torch.nn.functional.rms_norm(o, (w.H,), weight=g, eps=w.eps)
    assert np.array_equal(out["idx"], sel.indices.numpy())
    np.testing.assert_allclose(out["w"], p.numpy(), rtol=1e-13)
    np.testing.assert_allclose(out["o"], o.numpy(), rtol=1e-12, atol=1e-10)
    np.testing.assert_allclose(out["n"], n.numpy(), rtol=1e-12, atol=1e-10)
    # the shared term is not negligible here: leaving it out moves o by >> the bar
    assert np.max(np.abs(shared.numpy())) > 100 * 1e-10
    # a token subset gives the same rows (the shared expert sees the subset's own rows)
    sub = oracle.layer(inp, tokens=np.array([5, 1]))
    np.testing.assert_allclose(sub["o"], o.numpy()[[5, 1]], rtol=1e-12, atol=1e-10)
    np.testing.assert_allclose(sub["n"], n.numpy()[[5, 1]], rtol=1e-12, atol=1e-10)


# ----------------------------------------------------------------------------
# FP8 (W4A8) variant: E4M3 rounding, block-scaled activations, the FFN
# ----------------------------------------------------------------------------
def _e4m3_grid():
    """Every finite non-negative E4M3FN value, from its bit fields (closed form)."""
    vals = []
    for e in range(16):
        for m in range(8):
            if e == 15 and m == 7:
                continue  # NaN
            vals.append(Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7))
    return sorted(set(vals))


def _nearest_even(v, grid):
    """Nearest grid value to the rational v (ties -> even mantissa code), saturating."""
    a = abs(v)
    if a >= grid[-1]:
        return grid[-1] * (1 if v >= 0 else -1)
    import bisect
    i = bisect.bisect_left(grid, a)
    if grid[i] == a:
        r = a
    else:
        lo, hi = grid[i - 1], grid[i]
        if a - lo < hi - a:
            r = lo
        elif hi - a < a - lo:
            r = hi
        else:  # tie: the one whose mantissa code is even (its index in the grid is even)
            r = lo if (i - 1) % 2 == 0 else hi
    return r if v >= 0 else -r


def test_e4m3_round_matches_brute_force_grid():
    grid = _e4m3_grid()
    assert len(grid) == 127 and grid[-1] == 448 and grid[1] == Fraction(1, 512)
    rng = np.random.default_rng(31)
    vals = np.concatenate([rng.standard_normal(300) * np.exp2(rng.uniform(-12, 10, 300)),
                           [0.0, 448.0, -448.0, 464.0, 480.0, 1e9, 2.0 ** -10, 3 * 2.0 ** -11, 1.0625, 1.1875]])
    got = oracle.e4m3_round(vals)
    for v, g in zip(vals, got):
        assert Fraction(g) == _nearest_even(Fraction(v), grid), v


def test_e4m3_round_matches_torch_float8_in_range():
    rng = np.random.default_rng(32)
    v = (rng.standard_normal(5000) * np.exp2(rng.uniform(-11, 8, 5000))).astype(np.float32).astype(np.float64)
    v = v[np.abs(v) < 440]
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.e4m3_round(v), ref)


def test_mxfp8_quantize_block_scale_and_rounding():
    rng = np.random.default_rng(33)
    grid = _e4m3_grid()
    x = rng.standard_normal((6, 96)) * np.exp2(rng.uniform(-20, 20, (6, 1)))
    x[0, :32] = 0.0                                    # an all-zero block
    x[1, :64] = 0.0
    x[1, 5] = 1.75 * 2.0 ** 3                           # amax with mantissa exactly 1.75
    x[1, 6] = -0.3
    x[1, 40] = 1.875 * 2.0 ** -2                        # just above 1.75
    x[1, 41] = 2.0 ** -12
    q, e = oracle.mxfp8_quantize(x)
    assert q.shape == x.shape and e.shape == (6, 3)
    assert e[0, 0] == 0 and np.all(q[0, :32] == 0)
    assert e[1, 0] == 3 - 8                             # 1.75 * 2^8 = 448 fits
    assert e[1, 1] == -2 - 7                            # 1.875 * 2^8 > 448: one more
    amax = np.max(np.abs(x.reshape(6, 3, 32)), axis=-1)
    nz = amax > 0
    assert np.all(amax[nz] * np.exp2(-e[nz]) <= 448)    # fits without saturating ...
    assert np.all(amax[nz] * np.exp2(-(e[nz] - 1)) > 448)  # ... and e is the smallest that does
    for r in range(6):
        for c in range(96):
            s = Fraction(2) ** int(e[r, c // 32])
            assert Fraction(q[r, c]) == _nearest_even(Fraction(x[r, c]) / s, grid)


def test_w4a8_reduces_to_w4a16_on_fp8_exact_inputs():
    """With integer activations in [-4, 4] (exact in E4M3 after any power-of-two block
    scale) and power-of-two weight scales 2^-4..2^0 (code * scale then has at most 2
    significant bits, exact in E4M3), the FP8 up projection equals the W4A16 one, and
    the FP8 FFN equals the W4A16 down projection of MXFP8(BF16(h))."""
    rng = np.random.default_rng(34)
    R, H, I = 5, 64, 64
    x = rng.integers(-4, 5, (R, H)).astype(np.float64)
    codes13 = rng.integers(0, 256, (2 * I, H // 2)).astype(np.uint8)
    sc13 = wl.to_e4m3_codes(np.exp2(rng.integers(-4, 1, (2 * I, H // 16)).astype(np.float64)))
    codes2 = rng.integers(0, 256, (H, I // 2)).astype(np.uint8)
    sc2 = wl.to_e4m3_codes(np.exp2(rng.integers(-4, 1, (H, I // 16)).astype(np.float64)))
    W13, W2 = oracle.dequant(codes13, sc13, 1.0), oracle.dequant(codes2, sc2, 1.0)
    W13_8, W2_8 = oracle.dequant_e4m3(codes13, sc13), oracle.dequant_e4m3(codes2, sc2)
    np.testing.assert_array_equal(W13_8, W13)
    np.testing.assert_array_equal(W2_8, W2)
    np.testing.assert_allclose(oracle.swiglu_hidden_w4a8(x, W13_8, 0.5), oracle.swiglu_hidden(x, W13 * 0.5),
                               rtol=1e-13)
    h = oracle.bf16_round(oracle.swiglu_hidden(x, W13))
    q, e = oracle.mxfp8_quantize(h)
    hq = q * np.repeat(np.exp2(e), 32, axis=1)
    np.testing.assert_allclose(oracle.swiglu_ffn_w4a8(x, W13_8, 1.0, W2_8, 2.0),
                               oracle.bf16_round(2.0 * hq @ W2.T), rtol=1e-13)


def test_w4a8_ffn_brute_force():
    """The FP8 FFN on a tiny shape against pure-Python loops: block scales by search
    over the grid, exact rational products, math.fsum."""
    rng = np.random.default_rng(35)
    R, H, I = 2, 32, 32
    grid = _e4m3_grid()
    x = oracle.bf16_value(wl.to_bf16_bits(rng.standard_normal((R, H))))
    codes13 = rng.integers(0, 256, (2 * I, H // 2)).astype(np.uint8)
    sc13 = wl.to_e4m3_codes(np.exp2(rng.uniform(-4, 2, (2 * I, H // 16))))
    codes2 = rng.integers(0, 256, (H, I // 2)).astype(np.uint8)
    sc2 = wl.to_e4m3_codes(np.exp2(rng.uniform(-4, 2, (H, I // 16))))
    W13 = oracle.dequant(codes13, sc13, 1.0)
    W2 = oracle.dequant(codes2, sc2, 1.0)
    w8 = lambda W: [[float(_nearest_even(Fraction(v), grid)) for v in row] for row in W]
    W13_8, W2_8 = w8(W13), w8(W2)

    def mx(row):  # one block of 32
        amax = max(abs(Fraction(v)) for v in row)
        if amax == 0:
            return [0.0] * len(row)
        e = -130
        while amax / Fraction(2) ** e > 448:
            e += 1
        return [float(_nearest_even(Fraction(v) / Fraction(2) ** e, grid) * Fraction(2) ** e) for v in row]

    got = oracle.swiglu_ffn_w4a8(x, np.array(W13_8), 1.0, np.array(W2_8), 1.0)
    for r in range(R):
        xq = mx(list(x[r]))
        hrow = []
        for i in range(I):
            g = math.fsum(xq[c] * W13_8[i][c] for c in range(H))
            u = math.fsum(xq[c] * W13_8[I + i][c] for c in range(H))
            hrow.append(float(oracle.bf16_round(np.array(g / (1.0 + math.exp(-g)) * u))))
        hq = mx(hrow)
        for n in range(H):
            want = float(oracle.bf16_round(np.array(math.fsum(hq[i] * W2_8[n][i] for i in range(I)))))
            ulp = 2.0 ** (math.floor(math.log2(abs(want))) - 7) if want else 0.0
            assert abs(got[r, n] - want) <= ulp, (r, n, got[r, n], want)


def test_dequant_e4m3_rounds_each_weight():
    rng = np.random.default_rng(36)
    grid = _e4m3_grid()
    codes = rng.integers(0, 256, (8, 16)).astype(np.uint8)
    sc = wl.to_e4m3_codes(np.exp2(rng.uniform(-9, 8.7, (8, 2))))
    got = oracle.dequant_e4m3(codes, sc)
    exact = oracle.dequant(codes, sc, 1.0)
    assert np.any(got != exact)                          # 6-bit products do get rounded
    for r in range(8):
        for c in range(32):
            assert Fraction(got[r, c]) == _nearest_even(Fraction(exact[r, c]), grid)


def test_layer_w4a8_matches_torch_composition():
    """The FP8 layer, composed independently: torch.topk + torch.softmax routing, a
    per-token loop over the selected experts' FP8 FFNs (swiglu_ffn_w4a8, pinned by brute
    force above), the shared expert's FP8 FFN with weight 1, the residual, torch
    rms_norm."""
    w = wl.Workload("w4a8_pin", T=5, H=128, E=6, k=2, I=128, routing="normal", n_shared=1)
    inp = wl.make_inputs(w, seed=23)
    out = oracle.layer_w4a8(inp)
    val = lambda bits: torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double()
    x, r, g = val(inp.x), val(inp.residual), val(inp.gamma)
    L = torch.from_numpy(inp.logits.astype(np.float64))
    sel = torch.topk(L, w.k, dim=1)
    p = torch.softmax(L, dim=1).gather(1, sel.indices)
    p = p / p.sum(dim=1, keepdim=True)
    ffn = lambda xr, m13, m2, e: oracle.swiglu_ffn_w4a8(
        xr, oracle.dequant_e4m3(m13.packed[e], m13.scales[e]), m13.tscale[e],
        oracle.dequant_e4m3(m2.packed[e], m2.scales[e]), m2.tscale[e])
    o = r.clone()
    for t in range(w.T):
        for j in range(w.k):
            o[t] += p[t, j] * torch.from_numpy(ffn(x[t:t + 1].numpy(), inp.w13, inp.w2, int(sel.indices[t, j]))[0])
    o += torch.from_numpy(ffn(x.numpy(), inp.shared13, inp.shared2, 0))
    n = torch.nn.functional.rms_norm(o, (w.H,), weight=g, eps=w.eps)
    assert np.array_equal(out["idx"], sel.indices.numpy())
    np.testing.assert_allclose(out["o"], o.numpy(), rtol=1e-12, atol=1e-10)
    np.testing.assert_allclose(out["n"], n.numpy(), rtol=1e-12, atol=1e-10)
    # the FP8 layer is not the W4A16 one (the quantisation shows at the sampled size)
    assert not np.allclose(out["o"], oracle.layer(inp)["o"], rtol=1e-6)
