"""HIP path vs the fp64 oracle, through the C ABI (needs an MI355X).

Bars: routing indices, offsets, perm_src and inv bit-exact; routing weights within
1e-5 (and summing to 1 within 1e-5); layer outputs o and n within 2e-2 * rms(ref)
as max-abs error. Step-level checks use the tighter bars derived in their docstrings.
"""
import dataclasses
import sys
import zlib

import numpy as np
import pytest
import torch

import oracle
from bit_moe_expert_amd import binding as B
from bit_moe_expert_amd import workloads as wl
from tests.gpu_util import (LAYER_TOL, GpuLayer, assert_bf16_close, assert_layer_close, bf16_f64, bf16_ulp,
                            condition_router_margin, rel_rms_err, require_gpu, to_dev, to_host_bits,
                            upload_weights)

pytestmark = pytest.mark.gpu



@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# ----------------------------------------------------------------------------
# Route
# ----------------------------------------------------------------------------
ROUTE_GIVEN = [
    ("tiny", None), ("batched_t64", None), ("batched_t256", None), ("prefill", None),
    ("long_prefill", None),
    # edge cases: k = 1, k = E, E = 256 with k = 16, ragged T, T = 1
    ("edge_k1", wl.Workload("edge_k1", T=37, H=128, E=64, k=1, I=128, routing="normal")),
    ("edge_k_eq_e", wl.Workload("edge_k_eq_e", T=19, H=128, E=16, k=16, I=128, routing="normal")),
    ("edge_e256_k16", wl.Workload("edge_e256_k16", T=33, H=128, E=256, k=16, I=128, routing="zipf")),
    ("edge_t1", wl.Workload("edge_t1", T=1, H=128, E=160, k=8, I=128, routing="zipf")),
]


def _logits_only(w: wl.Workload, seed=0):
    return wl._draw_logits(np.random.SeedSequence([seed, 99]), w, w.T)


@pytest.mark.parametrize("name,w", ROUTE_GIVEN, ids=[n for n, _ in ROUTE_GIVEN])
def test_route_given_logits(name, w):
    w = wl.workload(name) if w is None else w
    note(f"route given logits: {name} T={w.T} E={w.E} k={w.k}")
    L = _logits_only(w)
    shape = B.make_shape(w.T, w.H, w.E, w.k, w.I)
    logits = to_dev(L)
    idx = torch.full((w.T, w.k), -1, dtype=torch.int32, device="cuda")
    wt = torch.zeros((w.T, w.k), dtype=torch.float32, device="cuda")
    B.moe4_route(shape, None, None, logits, idx, wt)
    torch.cuda.synchronize()
    ref_idx, ref_w = oracle.route(L.astype(np.float64), w.k)
    assert np.array_equal(idx.cpu().numpy(), ref_idx)
    got_w = wt.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(got_w - ref_w)) <= 1e-5
    assert np.max(np.abs(got_w.sum(axis=1) - 1.0)) <= 1e-5


@pytest.mark.parametrize("E,k", [(8, 1), (8, 8), (128, 8), (256, 16), (160, 3)])
def test_route_ties_and_special_values(E, k):
    """Exact ties (lower index wins), -0 equal to +0, -inf logits: indices bit-exact."""
    note(f"route ties/special values: E={E} k={k}")
    rng = np.random.default_rng(1234 + E * 17 + k)
    T = 64
    vals = np.array([-2.0, -1.0, -0.0, 0.0, 0.5, 1.0, -np.inf], dtype=np.float32)
    L = vals[rng.integers(0, vals.size, size=(T, E))]
    L[0, :] = 0.25                                          # all equal
    L[1, :] = np.where(np.arange(E) % 2 == 0, -0.0, 0.0)    # signed zeros only
    L[2, :] = -np.inf
    L[2, E - 1] = 3.0                                       # one finite logit at the end
    L[3, :] = np.float32(1e30) * np.where(np.arange(E) % 3 == 0, 1.0, -1.0)
    shape = B.make_shape(T, 128, E, k, 128)
    idx = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
    wt = torch.zeros((T, k), dtype=torch.float32, device="cuda")
    B.moe4_route(shape, None, None, to_dev(L), idx, wt)
    torch.cuda.synchronize()
    ref_idx, ref_w = oracle.route(L.astype(np.float64), k)
    assert np.array_equal(idx.cpu().numpy(), ref_idx)
    got_w = wt.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(got_w - ref_w)) <= 1e-5


@pytest.mark.parametrize("T", [1, 8, 37, 64])
def test_route_computed_logits(T):
    w = wl.workload("decode_t8")
    note(f"route computed logits: T={T} H={w.H} E={w.E}")
    inp = wl.make_inputs(w, seed=0, T=T)
    condition_router_margin(inp)
    shape = B.make_shape(T, w.H, w.E, w.k, w.I)
    x, wr = to_dev(inp.x), to_dev(inp.w_router)
    logits = torch.zeros((T, w.E), dtype=torch.float32, device="cuda")
    idx = torch.full((T, w.k), -1, dtype=torch.int32, device="cuda")
    wt = torch.zeros((T, w.k), dtype=torch.float32, device="cuda")
    B.moe4_route(shape, x, wr, logits, idx, wt)
    torch.cuda.synchronize()
    ref_L = oracle.router_logits(inp.x, inp.w_router)
    got_L = logits.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(got_L - ref_L)) < 5e-4  # well inside the 1e-3 margin
    ref_idx, ref_w = oracle.route(ref_L, w.k)
    assert np.array_equal(idx.cpu().numpy(), ref_idx)
    assert np.max(np.abs(wt.cpu().numpy() - ref_w)) <= 1e-5


# ----------------------------------------------------------------------------
# Permute
# ----------------------------------------------------------------------------
def _idx_case(case, rng):
    if case == "t1":
        return rng.permutation(128)[:8][None, :].astype(np.int32), 128
    if case == "tiny":
        return rng.integers(0, 8, (16, 2)).astype(np.int32), 8
    if case == "decode_t8":
        return np.stack([rng.permutation(128)[:8] for _ in range(8)]).astype(np.int32), 128
    if case == "batched_t256":
        return np.stack([rng.permutation(256)[:8] for _ in range(256)]).astype(np.int32), 256
    if case == "single_max":   # exactly the largest one-workgroup plan
        return rng.integers(0, 8, (2048, 8)).astype(np.int32), 8
    if case == "multi_min":    # just past it: three-kernel path, ragged last slice
        return rng.integers(0, 64, (2049, 8)).astype(np.int32), 64
    if case == "prefill_zipf":
        w = wl.workload("prefill")
        L = _logits_only(w)
        return oracle.route(L.astype(np.float64), 8)[0], 128
    if case == "long_zipf":
        w = wl.workload("long_prefill")
        L = _logits_only(w)
        return oracle.route(L.astype(np.float64), 8)[0], 160
    if case == "one_expert":   # every pair to expert 0 (k = 1)
        return np.zeros((5000, 1), dtype=np.int32), 32
    if case == "k_eq_e":
        return np.stack([rng.permutation(16) for _ in range(100)]).astype(np.int32), 16
    if case == "sparse_e256":  # most experts empty
        return rng.choice([3, 200, 255], (3001, 7)).astype(np.int32), 256
    if case == "t0":
        return np.zeros((0, 8), dtype=np.int32), 128
    raise ValueError(case)


PERMUTE_CASES = ["t1", "tiny", "decode_t8", "batched_t256", "single_max", "multi_min", "prefill_zipf",
                 "long_zipf", "one_expert", "k_eq_e", "sparse_e256", "t0"]


@pytest.mark.parametrize("case", PERMUTE_CASES)
def test_permute_bit_exact(case):
    rng = np.random.default_rng(zlib.crc32(case.encode()))
    idx, E = _idx_case(case, rng)
    T, k = idx.shape
    note(f"permute: {case} T={T} k={k} E={E}")
    shape = B.make_shape(T, 128, E, k, 128)
    d_idx = to_dev(idx) if T else torch.zeros((0, k), dtype=torch.int32, device="cuda")
    off = torch.full((E + 1,), -7, dtype=torch.int32, device="cuda")
    perm = torch.full((max(1, T * k),), -7, dtype=torch.int32, device="cuda")
    inv = torch.full((max(1, T * k),), -7, dtype=torch.int32, device="cuda")
    nws = B.moe4_permute_workspace_bytes(shape)
    ws = torch.empty(max(1, nws), dtype=torch.uint8, device="cuda") if nws else None
    B.moe4_permute(shape, d_idx if T else torch.zeros(1, dtype=torch.int32, device="cuda"), off, perm, inv, ws)
    torch.cuda.synchronize()
    r_off, r_perm, r_inv = oracle.permute(idx, E)
    if T == 0:  # a no-op: nothing written
        assert np.all(off.cpu().numpy() == -7)
        return
    assert np.array_equal(off.cpu().numpy(), r_off)
    if T:
        assert np.array_equal(perm.cpu().numpy(), r_perm)
        assert np.array_equal(inv.cpu().numpy(), r_inv)


# ----------------------------------------------------------------------------
# Weight re-layout
# ----------------------------------------------------------------------------
def tiled_reference(packed, scales):
    """The tiled layout of include/moe4.h, written with numpy reshapes: tile
    (g, b, s) in order, lane l = rn + 16*kq owns 16 code bytes and 2 scale bytes."""
    G, N, K2 = packed.shape
    K = 2 * K2
    c = packed.reshape(G, N // 16, 16, K // 128, 4, 16).transpose(0, 1, 3, 4, 2, 5)
    s = scales.reshape(G, N // 16, 16, K // 128, 4, 2).transpose(0, 1, 3, 4, 2, 5)
    return np.ascontiguousarray(c).reshape(-1), np.ascontiguousarray(s).reshape(-1)


def untile(tc, ts, G, N, K):
    c = tc.reshape(G, N // 16, K // 128, 4, 16, 16).transpose(0, 1, 4, 2, 3, 5)
    s = ts.reshape(G, N // 16, K // 128, 4, 16, 2).transpose(0, 1, 4, 2, 3, 5)
    return (np.ascontiguousarray(c).reshape(G, N, K // 2), np.ascontiguousarray(s).reshape(G, N, K // 16))


@pytest.mark.parametrize("G,N,K", [(1, 32, 128), (3, 96, 384), (8, 1024, 512), (2, 4096, 1536)])
def test_prepack_layout_bit_exact_and_lossless(G, N, K):
    note(f"prepack G={G} N={N} K={K}")
    rng = np.random.default_rng(G * N + K)
    packed = rng.integers(0, 256, (G, N, K // 2)).astype(np.uint8)
    scales = rng.integers(0, 256, (G, N, K // 16)).astype(np.uint8)
    tc = torch.empty(packed.size, dtype=torch.uint8, device="cuda")
    ts = torch.empty(scales.size, dtype=torch.uint8, device="cuda")
    B.moe4_prepack_w4(G, N, K, to_dev(packed), to_dev(scales), tc, ts)
    torch.cuda.synchronize()
    got_c, got_s = tc.cpu().numpy(), ts.cpu().numpy()
    want_c, want_s = tiled_reference(packed, scales)
    assert np.array_equal(got_c, want_c) and np.array_equal(got_s, want_s)
    back_c, back_s = untile(got_c, got_s, G, N, K)
    assert np.array_equal(back_c, packed) and np.array_equal(back_s, scales)


# ----------------------------------------------------------------------------
# Expert FFN
# ----------------------------------------------------------------------------
FFN_CASES = [
    ("tiny", None, None),
    ("decode_t1", None, None),
    ("decode_t8", None, None),
    ("batched_t64", None, None),
    # rows of one expert staged per pass (all rows do not fit LDS), several passes,
    # K split over the workgroup's waves
    ("expert_staged", wl.Workload("expert_staged", T=40, H=512, E=4, k=2, I=1024, routing="zipf"), None),
    # all rows staged once, many experts with rows
    ("all_staged", wl.Workload("all_staged", T=8, H=1024, E=256, k=8, I=1536, routing="normal"), None),
    # few rows per expert on average (3), staged 8 rows a pass (16 do not fit LDS); the
    # skewed routing gives some experts several passes
    ("expert8_passes", wl.Workload("expert8_passes", T=48, H=2048, E=128, k=8, I=256, routing="zipf"), None),
    # activations in registers (neither all rows nor one expert's rows fit LDS), several passes
    ("regs_passes", wl.Workload("regs_passes", T=40, H=2048, E=4, k=2, I=256, routing="zipf"), None),
    # all rows staged, one wave per pair in one round: one workgroup per CU of 8, 11
    # (2688 pairs, a ragged last round of units) and 16 waves for the up launch
    ("all_rows_8_waves", wl.Workload("all_rows_8_waves", T=8, H=2048, E=128, k=8, I=512, routing="router"), None),
    ("all_rows_11_waves", wl.Workload("all_rows_11_waves", T=7, H=2048, E=128, k=8, I=768, routing="router"), None),
    ("all_rows_16_waves", wl.Workload("all_rows_16_waves", T=8, H=2048, E=128, k=8, I=1024, routing="router"), None),
    # many rows per expert (the MFMA-tile kernel), ragged tails
    ("rows_ragged", wl.Workload("rows_ragged", T=301, H=512, E=8, k=2, I=256, routing="zipf"), None),
    ("prefill_small", wl.Workload("prefill_small", T=1024, H=1024, E=16, k=4, I=384, routing="zipf"), None),
]


def _plan_on_host(inp):
    L = inp.logits.astype(np.float64) if inp.logits is not None else oracle.router_logits(inp.x, inp.w_router)
    idx, w = oracle.route(L, inp.w.k)
    off, perm, inv = oracle.permute(idx, inp.w.E)
    return idx, w, off, perm, inv


def _run_routed_ffn(inp, w, off, perm, layout="tiled"):
    """moe4_expert_ffn on the plan (off, perm) with the weights in `layout`; h, y bits."""
    shape = B.make_shape(inp.T, w.H, w.E, w.k, w.I)
    w13, w2, *_ = upload_weights(inp, layout)
    R = inp.T * w.k
    h = torch.zeros((R, w.I), dtype=torch.int16, device="cuda")
    y = torch.zeros((R, w.H), dtype=torch.int16, device="cuda")
    B.moe4_expert_ffn(shape, to_dev(inp.x), to_dev(off), to_dev(perm), w13, w2, h, y)
    torch.cuda.synchronize()
    return to_host_bits(h), to_host_bits(y)


def _check_routed_ffn(inp, w, off, perm, canonical_too=True):
    """Runs moe4_expert_ffn on the plan (off, perm) and checks h against the oracle's
    SwiGLU and y against the oracle's down projection of the GPU's own h. With the
    weights in the canonical layout the same kernels must give the same bits."""
    h_bits, y_bits = _run_routed_ffn(inp, w, off, perm)
    if canonical_too:
        ch, cy = _run_routed_ffn(inp, w, off, perm, "canonical")
        assert np.array_equal(ch, h_bits), "h differs between the canonical and the tiled layout"
        assert np.array_equal(cy, y_bits), "y differs between the canonical and the tiled layout"
    got_h, got_y = oracle.bf16_value(h_bits), oracle.bf16_value(y_bits)
    x = oracle.bf16_value(inp.x)
    tok = perm // w.k
    exp_of_row = np.repeat(np.arange(w.E), np.diff(off))
    ref_h = np.zeros_like(got_h)
    ref_y = np.zeros_like(got_y)
    for e in np.unique(exp_of_row):
        rows = np.flatnonzero(exp_of_row == e)
        W13 = oracle.dequant(inp.w13.packed[e], inp.w13.scales[e], inp.w13.tscale[e])
        W2 = oracle.dequant(inp.w2.packed[e], inp.w2.scales[e], inp.w2.tscale[e])
        ref_h[rows] = oracle.bf16_round(oracle.swiglu_hidden(x[tok[rows]], W13))
        # down projection checked on the GPU's own h (isolates the second GEMM)
        ref_y[rows] = oracle.bf16_round(got_h[rows] @ W2.T)
    assert_bf16_close(got_h, ref_h, "h")
    assert_bf16_close(got_y, ref_y, "y", slack_rms=2.0 ** -16)


@pytest.mark.parametrize("name,w,_", FFN_CASES, ids=[c[0] for c in FFN_CASES])
def test_expert_ffn_routed(name, w, _):
    w = wl.workload(name) if w is None else w
    note(f"expert ffn routed: {name} T={w.T} H={w.H} E={w.E} k={w.k} I={w.I}")
    inp = wl.make_inputs(w, seed=1)
    idx, _, off, perm, inv = _plan_on_host(inp)
    _check_routed_ffn(inp, w, off, perm)


def test_expert_ffn_tile_edges():
    """Expert groups on the prefill GEMM's tile boundaries: a tile computes its rows
    rounded up to 32 (2 to 8 blocks of 32 rows a wave), so 64/65, 96/97, 128/129,
    160/161, 192/193, 224/225 and 256/257 rows sit on the block edges (128 and below
    are the schedule's half tiles, 129 to 192 its three-quarter ones); 384 (a full tile
    and a half one), 416 (a full and a three-quarter one) and 1 row."""
    counts = [64, 65, 96, 97, 128, 129, 160, 161, 192, 193, 224, 225, 256, 257, 384, 416, 1]
    w = wl.Workload("tile_edges", T=sum(counts), H=512, E=len(counts), k=1, I=256, routing="normal")
    note(f"expert ffn tile edges: groups {counts}")
    inp = wl.make_inputs(w, seed=3)
    idx = np.random.default_rng(5).permutation(np.repeat(np.arange(w.E), counts)).astype(np.int32)[:, None]
    off, perm, inv = oracle.permute(idx, w.E)
    assert np.array_equal(np.diff(off), counts)
    _check_routed_ffn(inp, w, off, perm)


def test_expert_ffn_prefill_schedule_edges():
    """The prefill GEMM's tile schedule over 256 experts, most of them empty: rows only
    at the ends of the 64-expert rounds of its per-expert count (experts 0, 63, 64, 127,
    128, 191, 255), groups that give half tiles (1, 100 rows and a 57-row tail),
    three-quarter tiles (129, 170), padded full tiles (200) and tails of each kind after
    full tiles (300, 385, 450), and few tiles per XCD for the down GEMM (one N tile)."""
    counts = np.zeros(256, dtype=np.int64)
    for e, c in {0: 100, 1: 170, 2: 200, 3: 450, 63: 129, 64: 300, 127: 256, 128: 1, 191: 385}.items():
        counts[e] = c
    T = 64 * 256  # k = 1: as many rows as the prefill kernel needs over 256 experts
    counts[255] = T - counts.sum()
    w = wl.Workload("sched_edges", T=T, H=256, E=256, k=1, I=256, routing="normal")
    note(f"expert ffn prefill schedule edges: groups {dict((int(e), int(c)) for e, c in enumerate(counts) if c)}")
    inp = wl.make_inputs(w, seed=4)
    idx = np.random.default_rng(6).permutation(np.repeat(np.arange(w.E), counts)).astype(np.int32)[:, None]
    off, perm, inv = oracle.permute(idx, w.E)
    assert np.array_equal(np.diff(off), counts)
    _check_routed_ffn(inp, w, off, perm)


WIDE_CASES = ["decode_t8", "expert_staged", "expert8_passes", "batched_t64"]


@pytest.mark.parametrize("name", WIDE_CASES)
def test_expert_ffn_wide_range_rows(name):
    """Activation rows of very different magnitudes (row scales 2^-50 .. 2^26) whose
    values each span 2^31 below the row's largest: the staged forms of the streaming
    kernel scale each row (or row slice) by its own power of two into FP16, which keeps
    the BF16 result's bits while a row's values lie within 2^32 of its maximum. Each
    row of h is checked against the oracle on its own scale (1 BF16 ulp plus 2^-12 of
    the row's rms), and each row of y against fp64 sums over the GPU's own h."""
    w = dict((c[0], c[1]) for c in FFN_CASES)[name] or wl.workload(name)
    note(f"expert ffn wide-range rows: {name} T={w.T} H={w.H} E={w.E} k={w.k} I={w.I}")
    inp = wl.make_inputs(w, seed=8)
    rng = np.random.default_rng(81)
    row_scale = np.exp2(rng.uniform(-50, 26, (inp.T, 1)))
    within = np.exp2(rng.uniform(-31, 0, (inp.T, w.H)))
    inp.x[:] = wl.to_bf16_bits(rng.standard_normal((inp.T, w.H)) * within * row_scale)
    idx, _, off, perm, inv = _plan_on_host(inp)
    h_bits, y_bits = _run_routed_ffn(inp, w, off, perm)
    got_h, got_y = oracle.bf16_value(h_bits), oracle.bf16_value(y_bits)
    x = oracle.bf16_value(inp.x)
    tok = perm // w.k
    exp_of_row = np.repeat(np.arange(w.E), np.diff(off))
    for e in np.unique(exp_of_row):
        rows = np.flatnonzero(exp_of_row == e)
        W13 = oracle.dequant(inp.w13.packed[e], inp.w13.scales[e], inp.w13.tscale[e])
        W2 = oracle.dequant(inp.w2.packed[e], inp.w2.scales[e], inp.w2.tscale[e])
        ref_h = oracle.bf16_round(oracle.swiglu_hidden(x[tok[rows]], W13))
        ref_y = oracle.bf16_round(got_h[rows] @ W2.T)
        for i, r in enumerate(rows):
            assert_bf16_close(got_h[r], ref_h[i], f"h row {r} (expert {e})", min_equal=0.8)
            assert_bf16_close(got_y[r], ref_y[i], f"y row {r} (expert {e})", slack_rms=2.0 ** -16,
                              min_equal=0.8)


SIGNED_SCALE_CASES = ["decode_t8", "regs_passes", "expert_staged", "rows_ragged", "prefill_small"]


@pytest.mark.parametrize("name", SIGNED_SCALE_CASES)
def test_expert_ffn_signed_block_scales(name):
    """Block scales of both signs over a wider range (E4M3 codes with the sign bit set
    half the time, magnitudes 2^-6 .. 2^6): a negative code times a negative scale is
    positive in every dequantisation form (the streaming kernel's BF16 and FP16 forms,
    the GEMM's BF16 one; tiled and canonical layouts). Checked as the routed cases
    are."""
    w = dict((c[0], c[1]) for c in FFN_CASES)[name] or wl.workload(name)
    note(f"expert ffn signed block scales: {name} T={w.T} H={w.H} E={w.E} k={w.k} I={w.I}")
    inp = wl.make_inputs(w, seed=12)
    rng = np.random.default_rng(121)
    for m in (inp.w13, inp.w2):
        m.scales[:] = wl.to_e4m3_codes(np.exp2(rng.uniform(-6, 6, m.scales.shape)))
        m.scales[:] |= (rng.random(m.scales.shape) < 0.5).astype(np.uint8) << 7  # sign bit
    assert np.any(oracle.e4m3_value(inp.w13.scales) < 0) and np.any(oracle.e4m3_value(inp.w13.scales) > 0)
    idx, _, off, perm, inv = _plan_on_host(inp)
    _check_routed_ffn(inp, w, off, perm)


@pytest.mark.parametrize("T", [1, 8, 17, 39, 50, 77, 100, 150, 200, 220, 300])
def test_expert_ffn_dense_shared(T):
    """Dense (shared expert) mode: on the streaming kernel below 40 rows (1, 8, 17 and
    39 rows: one or several 16-row passes, a ragged last one), and on the prefill GEMM
    from 40: tiles of 2, 3, 4, 5 and 7 blocks of 32 rows (50, 77, 100, 150, 200, 220)
    and a full tile plus a 2-block one (300)."""
    w = wl.Workload("shared_small", T=T, H=1024, E=1, k=1, I=512, routing="normal")
    note(f"expert ffn dense (shared expert mode) T={T}")
    inp = wl.make_inputs(w, seed=2)
    shape = B.make_shape(inp.T, w.H, 1, 1, w.I)
    w13, w2, *_ = upload_weights(inp)
    h = torch.zeros((inp.T, w.I), dtype=torch.int16, device="cuda")
    y = torch.zeros((inp.T, w.H), dtype=torch.int16, device="cuda")
    B.moe4_expert_ffn(shape, to_dev(inp.x), None, None, w13, w2, h, y)
    torch.cuda.synchronize()
    x = oracle.bf16_value(inp.x)
    W13 = oracle.dequant(inp.w13.packed[0], inp.w13.scales[0], inp.w13.tscale[0])
    W2 = oracle.dequant(inp.w2.packed[0], inp.w2.scales[0], inp.w2.tscale[0])
    got_h = bf16_f64(h)
    assert_bf16_close(got_h, oracle.bf16_round(oracle.swiglu_hidden(x, W13)), "h")
    assert_bf16_close(bf16_f64(y), oracle.bf16_round(got_h @ W2.T), "y", slack_rms=2.0 ** -16)
    # end to end against the oracle's FFN: within 2e-2 of rms, plus one BF16 ulp of y
    # (the two BF16 y may round to neighbouring values)
    ref_y = oracle.swiglu_ffn(x, W13, W2)
    rms = float(np.sqrt(np.mean(ref_y ** 2)))
    assert np.all(np.abs(bf16_f64(y) - ref_y) <= 2e-2 * rms + bf16_ulp(ref_y))


@pytest.mark.parametrize("T,H,E,k,I", [(8, 2048, 128, 8, 768), (300, 512, 4, 2, 256)])
def test_expert_ffn_integer_exact(T, H, E, k, I):
    """Integer activations in [-4, 4] and power-of-two scales 2^-4..2^0 make every
    partial sum of g and u a multiple of 2^-5 below 2^18, so FP32 accumulation is
    exact in any order: h must be within 1 BF16 ulp of silu(g)*u from the exact g, u
    (the one rounding plus the exp approximation). y is then checked against fp64
    sums over the GPU's own h: within 1 BF16 ulp plus FP32 accumulation slack."""
    note(f"expert ffn integer-exact T={T} H={H} E={E}")
    rng = np.random.default_rng(T + H)
    w = wl.Workload("intexact", T=T, H=H, E=E, k=k, I=I, routing="normal")
    inp = wl.make_inputs(w, seed=3)
    inp.x[:] = wl.to_bf16_bits(rng.integers(-4, 5, (T, H)).astype(np.float64))
    for m in (inp.w13, inp.w2):
        m.scales[:] = wl.to_e4m3_codes(np.exp2(rng.integers(-4, 1, m.scales.shape).astype(np.float64)))
    idx, _, off, perm, inv = _plan_on_host(inp)
    shape = B.make_shape(T, H, E, k, I)
    w13, w2, *_ = upload_weights(inp)
    h = torch.zeros((T * k, I), dtype=torch.int16, device="cuda")
    y = torch.zeros((T * k, H), dtype=torch.int16, device="cuda")
    B.moe4_expert_ffn(shape, to_dev(inp.x), to_dev(off), to_dev(perm), w13, w2, h, y)
    torch.cuda.synchronize()
    got_h, got_y = bf16_f64(h), bf16_f64(y)
    x = oracle.bf16_value(inp.x)
    tok = perm // k
    exp_of_row = np.repeat(np.arange(E), np.diff(off))
    for e in np.unique(exp_of_row):
        rows = np.flatnonzero(exp_of_row == e)
        W13 = oracle.dequant(inp.w13.packed[e], inp.w13.scales[e], inp.w13.tscale[e])
        W2 = oracle.dequant(inp.w2.packed[e], inp.w2.scales[e], inp.w2.tscale[e])
        ref_h = oracle.swiglu_hidden(x[tok[rows]], W13)
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref_h), 1e-30))) - 7)
        assert np.all(np.abs(got_h[rows] - ref_h) <= ulp * 1.01 + 1e-30), f"expert {e}"
        ref_y = got_h[rows] @ W2.T
        ulp_y = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref_y), 1e-30))) - 7)
        slack = 2.0 ** -20 * np.sqrt(np.mean(ref_y ** 2))
        assert np.all(np.abs(got_y[rows] - ref_y) <= ulp_y + slack), f"expert {e}"


# ----------------------------------------------------------------------------
# Combine + RMSNorm
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("T,H,k,shared", [(1, 2048, 8, False), (8, 2048, 8, False), (37, 4096, 8, True),
                                          (16, 256, 2, False), (5, 16384, 16, True)])
def test_combine_norm(T, H, k, shared):
    note(f"combine_norm T={T} H={H} k={k} shared={shared}")
    rng = np.random.default_rng(T * H + k)
    E = max(k, 16)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    off, perm, inv = oracle.permute(idx, E)
    y = wl.to_bf16_bits(rng.standard_normal((T * k, H)) * 3)
    wts = rng.random((T, k)).astype(np.float32)
    wts /= wts.sum(axis=1, keepdims=True)
    res = wl.to_bf16_bits(rng.standard_normal((T, H)))
    gam = wl.to_bf16_bits(rng.uniform(0.5, 1.5, H))
    sh = wl.to_bf16_bits(rng.standard_normal((T, H))) if shared else None
    shape = B.make_shape(T, H, E, k, 128)
    d_res = to_dev(res)
    out_o = torch.zeros((T, H), dtype=torch.int16, device="cuda")
    out_n = torch.zeros((T, H), dtype=torch.int16, device="cuda")
    B.moe4_combine_norm(shape, to_dev(y), to_dev(inv), to_dev(wts), to_dev(sh) if shared else None,
                        d_res, to_dev(gam), out_o, out_n)
    torch.cuda.synchronize()
    yt = oracle.bf16_value(y)[inv.reshape(T, k)]   # [T, k, H] in token order
    ref_o, ref_n = oracle.combine_norm(yt, wts.astype(np.float64), res, gam, 1e-6,
                                       shared=oracle.bf16_value(sh) if shared else None)
    got_o, got_n = bf16_f64(out_o), bf16_f64(out_n)
    # one BF16 rounding of an FP32 sum: 2^-8 relative, plus FP32 slack
    assert np.all(np.abs(got_o - ref_o) <= 2 ** -8 * np.abs(ref_o) + 1e-5 * np.sqrt(np.mean(ref_o ** 2)))
    assert np.all(np.abs(got_n - ref_n) <= 2 ** -7 * np.abs(ref_n) + 1e-5 * np.sqrt(np.mean(ref_n ** 2)))
    # in-place: residual_out aliases residual
    B.moe4_combine_norm(shape, to_dev(y), to_dev(inv), to_dev(wts), to_dev(sh) if shared else None,
                        d_res, to_dev(gam), d_res, out_n)
    torch.cuda.synchronize()
    assert np.array_equal(to_host_bits(d_res), to_host_bits(out_o))


def test_combine_norm_closed_form_zero_experts():
    """y = 0: o = residual exactly and n = r / rms(r) * gamma."""
    T, H, k, E = 4, 2048, 8, 128
    rng = np.random.default_rng(5)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    _, _, inv = oracle.permute(idx, E)
    res = wl.to_bf16_bits(rng.standard_normal((T, H)))
    gam = wl.to_bf16_bits(rng.uniform(0.5, 1.5, H))
    shape = B.make_shape(T, H, E, k, 128)
    out_o = torch.zeros((T, H), dtype=torch.int16, device="cuda")
    out_n = torch.zeros((T, H), dtype=torch.int16, device="cuda")
    wts = np.full((T, k), 1.0 / k, dtype=np.float32)
    B.moe4_combine_norm(shape, torch.zeros((T * k, H), dtype=torch.int16, device="cuda"), to_dev(inv),
                        to_dev(wts), None, to_dev(res), to_dev(gam), out_o, out_n)
    torch.cuda.synchronize()
    assert np.array_equal(to_host_bits(out_o), res)
    r = oracle.bf16_value(res)
    ref_n = r / np.sqrt(np.mean(r * r, axis=1, keepdims=True) + 1e-6) * oracle.bf16_value(gam)
    assert np.all(np.abs(bf16_f64(out_n) - ref_n) <= 2 ** -7 * np.abs(ref_n) + 1e-6)


# ----------------------------------------------------------------------------
# Whole layer
# ----------------------------------------------------------------------------
LAYER_CASES = [("tiny", None), ("decode_t1", None), ("decode_t8", None), ("batched_t64", None),
               ("batched_t256", None), ("prefill", 1024)]


@pytest.mark.parametrize("name,sample", LAYER_CASES, ids=[c[0] for c in LAYER_CASES])
def test_layer_parity(name, sample):
    w = wl.workload(name)
    note(f"layer parity: {name} T={w.T} H={w.H} E={w.E} k={w.k} I={w.I} shared={w.n_shared}")
    inp = wl.make_inputs(w, seed=0, chunk=0)
    if w.routing == "router":
        condition_router_margin(inp)
    g = GpuLayer(inp)
    g.run()
    got = g.host()
    # routing: every token
    L = inp.logits.astype(np.float64) if inp.logits is not None else oracle.router_logits(inp.x, inp.w_router)
    ref_idx, ref_w = oracle.route(L, w.k)
    assert np.array_equal(got["idx"], ref_idx)
    assert np.max(np.abs(got["w"] - ref_w)) <= 1e-5
    assert np.max(np.abs(got["w"].sum(axis=1) - 1)) <= 1e-5
    # outputs: every token, or a seeded sample of them for the prefill shapes
    tokens = None
    if sample is not None:
        tokens = np.sort(np.random.default_rng(123).choice(w.T, sample, replace=False))
    ref = oracle.layer(inp, tokens=tokens, logits=L if tokens is None else L[tokens])
    sel = ref["tokens"]
    assert_layer_close(got["o"][sel], got["n"][sel], ref, inp.gamma, w.eps, name)


def test_long_prefill_layer_parity_all_chunks():
    """Long prefill, all four chunks of 8192 tokens (one shared set of weights): routing
    of every token bit-exact; o and n of a seeded sample of 1024 tokens per chunk
    within the bar of one oracle pass over the 4096 sampled tokens (tokens are
    independent, so the oracle can take them together)."""
    w = wl.workload("long_prefill")
    note("layer parity: long prefill, 4 chunks x 8192 tokens, 1024 sampled per chunk")
    base = wl.make_inputs(w, seed=0, chunk=0)
    weights = upload_weights(base)
    rng = np.random.default_rng(321)
    parts, got_o, got_n, sizes = [], [], [], []
    for c in range(w.chunks):
        inp = base if c == 0 else wl.make_inputs(w, seed=0, chunk=c, weights_from=base)
        g = GpuLayer(inp, weights=weights)
        g.run()
        got = g.host()
        del g
        L = inp.logits.astype(np.float64)
        ref_idx, ref_w = oracle.route(L, w.k)
        assert np.array_equal(got["idx"], ref_idx), f"chunk {c}: routing"
        assert np.max(np.abs(got["w"] - ref_w)) <= 1e-5, f"chunk {c}: routing weights"
        tok = np.sort(rng.choice(w.T, 1024, replace=False))
        parts.append((inp.x[tok], inp.residual[tok], inp.logits[tok]))
        got_o.append(got["o"][tok])
        got_n.append(got["n"][tok])
        note(f"  chunk {c}: GPU done, routing exact")
    combined = dataclasses.replace(base, x=np.concatenate([p[0] for p in parts]),
                                   residual=np.concatenate([p[1] for p in parts]),
                                   logits=np.concatenate([p[2] for p in parts]))
    ref = oracle.layer(combined)
    for c in range(w.chunks):
        sl = slice(1024 * c, 1024 * (c + 1))
        assert_layer_close(got_o[c], got_n[c], ref, base.gamma, w.eps, f"chunk {c}", sel=sl)


def _deq_pair(m13, m2, e):
    return (oracle.dequant(m13.packed[e], m13.scales[e], m13.tscale[e]),
            oracle.dequant(m2.packed[e], m2.scales[e], m2.tscale[e]))


def _sample_plan_rows(off, rng):
    """Rows of the plan to check, per expert: the first and last row, the first row and
    a middle row of the last M tile (a half or three-quarter tile when the expert's
    count is not a multiple of 256), and two random rows; plus every row of the
    hottest expert and of one expert whose last tile is three-quarter (129-192 rows)
    and one whose last tile is half (1-128 rows)."""
    cnt = np.diff(off)
    rows = []
    for e in np.flatnonzero(cnt):
        a, b = int(off[e]), int(off[e + 1])
        lt = a + (cnt[e] - 1) // 256 * 256
        rows += [a, b - 1, lt, (lt + b - 1) // 2, *rng.integers(a, b, 2)]
    full = [int(np.argmax(cnt))]
    rem = cnt % 256
    for lo, hi in ((129, 192), (1, 128)):
        cand = np.flatnonzero((rem >= lo) & (rem <= hi) & (cnt > 256))
        cand = cand if cand.size else np.flatnonzero((rem >= lo) & (rem <= hi))
        if cand.size:
            full.append(int(cand[0]))
    for e in full:
        rows += list(range(int(off[e]), int(off[e + 1])))
    return np.unique(np.array(rows, dtype=np.int64)), full


@pytest.mark.parametrize("name", ["prefill", "long_prefill"])
def test_expert_ffn_full_size_sampled_rows(name):
    """The expert FFN at the full prefill and long-prefill shapes (8192 tokens, Zipf
    routing, the real tile schedule with its three-quarter and half last tiles and its
    per-XCD runs): h of sampled plan rows (see _sample_plan_rows) against the oracle's
    SwiGLU, and y of the same rows against fp64 sums over the GPU's own h, at the
    step-level bars; for long prefill also the shared expert (dense, 8192 rows)."""
    from concurrent.futures import ThreadPoolExecutor

    w = wl.workload(name)
    inp = wl.make_inputs(w, seed=0, chunk=0)
    idx, _, off, perm, inv = _plan_on_host(inp)
    rng = np.random.default_rng(55)
    rows, full = _sample_plan_rows(off, rng)
    note(f"expert ffn full size: {name}: {rows.size} plan rows checked, every row of experts {full} "
         f"(counts {[int(off[e + 1] - off[e]) for e in full]})")
    h_bits, y_bits = _run_routed_ffn(inp, w, off, perm)
    got_h, got_y = oracle.bf16_value(h_bits), oracle.bf16_value(y_bits)
    del h_bits, y_bits
    x = oracle.bf16_value(inp.x)
    tok = perm // w.k
    exp_of_row = np.repeat(np.arange(w.E), np.diff(off))

    def check_expert(e):
        rr = rows[exp_of_row[rows] == e]
        if rr.size == 0:
            return
        W13, W2 = _deq_pair(inp.w13, inp.w2, e)
        assert_bf16_close(got_h[rr], oracle.bf16_round(oracle.swiglu_hidden(x[tok[rr]], W13)), f"h expert {e}")
        assert_bf16_close(got_y[rr], oracle.bf16_round(got_h[rr] @ W2.T), f"y expert {e}", slack_rms=2.0 ** -16)

    with ThreadPoolExecutor(8) as ex:
        list(ex.map(check_expert, range(w.E)))
    if w.n_shared:
        shape = B.make_shape(inp.T, w.H, 1, 1, w.I)
        s13 = B.DeviceW4.from_host(inp.shared13)
        s2 = B.DeviceW4.from_host(inp.shared2)
        h = torch.zeros((inp.T, w.I), dtype=torch.int16, device="cuda")
        y = torch.zeros((inp.T, w.H), dtype=torch.int16, device="cuda")
        B.moe4_expert_ffn(shape, to_dev(inp.x), None, None, s13, s2, h, y)
        torch.cuda.synchronize()
        sr = np.unique(np.concatenate([[0, 255, 256, inp.T - 1], rng.integers(0, inp.T, 500)]))
        sh, sy = bf16_f64(h)[sr], bf16_f64(y)[sr]
        W13, W2 = _deq_pair(inp.shared13, inp.shared2, 0)
        assert_bf16_close(sh, oracle.bf16_round(oracle.swiglu_hidden(x[sr], W13)), "shared h")
        assert_bf16_close(sy, oracle.bf16_round(sh @ W2.T), "shared y", slack_rms=2.0 ** -16)


def test_layer_deterministic_and_batch_independent():
    w = wl.workload("decode_t8")
    note("layer determinism / batch independence: decode T=8 vs T=1")
    inp = wl.make_inputs(w, seed=0)
    condition_router_margin(inp)
    g = GpuLayer(inp)
    g.run()
    a = g.host()
    g.run()
    b = g.host()
    assert np.array_equal(a["o_bits"], b["o_bits"]) and np.array_equal(a["n_bits"], b["n_bits"])
    # token 3 alone gives the same bytes as inside the batch of 8
    one = dataclasses.replace(inp, x=inp.x[3:4].copy(), residual=inp.residual[3:4].copy())
    g1 = GpuLayer(one, weights=(g.w13, g.w2, None, None, g.w_router))
    g1.run()
    c = g1.host()
    assert np.array_equal(c["idx"][0], a["idx"][3])
    assert np.array_equal(c["o_bits"][0], a["o_bits"][3])
    assert np.array_equal(c["n_bits"][0], a["n_bits"][3])
    # and inside a batch of 9 (72 routed rows: the down projection stages its rows in LDS
    # as FP16, where 8 tokens read them from the cache as BF16; the bits must not change)
    nine = dataclasses.replace(inp, x=np.concatenate([inp.x, inp.x[5:6]]),
                               residual=np.concatenate([inp.residual, inp.residual[5:6]]))
    g9 = GpuLayer(nine, weights=(g.w13, g.w2, None, None, g.w_router))
    g9.run()
    d = g9.host()
    assert np.array_equal(d["idx"][:8], a["idx"])
    assert np.array_equal(d["o_bits"][:8], a["o_bits"]) and np.array_equal(d["n_bits"][:8], a["n_bits"])
    # the ninth token repeats token 5; its activation row is staged by the up kernel's
    # second copy round (9 rows of 2048 columns are 2304 16-byte chunks, 2048 a round)
    assert np.array_equal(d["idx"][8], a["idx"][5])
    assert np.array_equal(d["o_bits"][8], a["o_bits"][5]) and np.array_equal(d["n_bits"][8], a["n_bits"][5])


# moe4_layer takes the fused top-k + plan launch for small batches and may pick other
# kernel forms than the separate entry points; both must give the same bytes, on every
# one of several calls. The cases span one to 136 routed pairs, given or computed
# router logits, and one or two token groups of the router.
FUSED_ROUTE_CASES = [
    ("tiny", None), ("decode_t1", None), ("decode_t8", None),
    ("pairs_128", wl.Workload("pairs_128", T=16, H=256, E=64, k=8, I=256, routing="normal")),
    ("pairs_136", wl.Workload("pairs_136", T=17, H=256, E=64, k=8, I=256, routing="normal")),
    ("router_t16", wl.Workload("router_t16", T=16, H=256, E=64, k=8, I=256, routing="router")),
    ("router_t17", wl.Workload("router_t17", T=17, H=256, E=64, k=8, I=256, routing="router")),
]


@pytest.mark.parametrize("name,w", FUSED_ROUTE_CASES, ids=[c[0] for c in FUSED_ROUTE_CASES])
def test_layer_matches_entry_points(name, w):
    w = wl.workload(name) if w is None else w
    note(f"layer vs entry points: {name} T={w.T} H={w.H} E={w.E} k={w.k} I={w.I}")
    inp = wl.make_inputs(w, seed=2)
    g = GpuLayer(inp)
    g.run()
    a = g.host()
    for _ in range(2):
        g.run()
        b = g.host()
        assert np.array_equal(b["idx"], a["idx"]) and np.array_equal(b["o_bits"], a["o_bits"])
        assert np.array_equal(b["n_bits"], a["n_bits"])
    T, k, E, H, I = inp.T, w.k, w.E, w.H, w.I
    shape = g.shape
    logits = g.logits.clone() if inp.logits is not None else torch.empty((T, E), dtype=torch.float32,
                                                                           device="cuda")
    idx = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
    tw = torch.zeros((T, k), dtype=torch.float32, device="cuda")
    B.moe4_route(shape, g.x if g.w_router is not None else None, g.w_router, logits, idx, tw)
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(T * k, dtype=torch.int32, device="cuda")
    inv = torch.empty(T * k, dtype=torch.int32, device="cuda")
    n = B.moe4_permute_workspace_bytes(shape)
    B.moe4_permute(shape, idx, off, perm, inv, torch.empty(n, dtype=torch.uint8, device="cuda") if n else None)
    h = torch.zeros((T * k, I), dtype=torch.int16, device="cuda")
    y = torch.zeros((T * k, H), dtype=torch.int16, device="cuda")
    B.moe4_expert_ffn(shape, g.x, off, perm, g.w13, g.w2, h, y)
    o = torch.zeros((T, H), dtype=torch.int16, device="cuda")
    nrm = torch.zeros((T, H), dtype=torch.int16, device="cuda")
    B.moe4_combine_norm(shape, y, inv, tw, None, g.residual, g.gamma, o, nrm)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), a["idx"])
    assert np.array_equal(tw.cpu().numpy().view(np.int32), g.topk_w.cpu().numpy().view(np.int32))
    assert np.array_equal(to_host_bits(o), a["o_bits"])
    assert np.array_equal(to_host_bits(nrm), a["n_bits"])
    # The layer's own plan (white box: the layer keeps offsets, perm_src and inv at the
    # start of its workspace, each padded to 256 bytes) is the oracle's stable plan,
    # whichever of the fused top-k + plan forms built it.
    pad = lambda v: (v + 255) // 256 * 256
    ws = g.ws.cpu().numpy()
    p0 = pad((E + 1) * 4)
    i0 = p0 + pad(T * k * 4)
    ref_off, ref_perm, ref_inv = oracle.permute(a["idx"], E)
    assert np.array_equal(ws[:(E + 1) * 4].view(np.int32), ref_off)
    assert np.array_equal(ws[p0:p0 + T * k * 4].view(np.int32), ref_perm)
    assert np.array_equal(ws[i0:i0 + T * k * 4].view(np.int32), ref_inv)
    assert np.array_equal(off.cpu().numpy(), ref_off) and np.array_equal(perm.cpu().numpy(), ref_perm)


def _check_against_oracle(inp, got):
    """Routing bit-exact and outputs within the layer bar of the oracle (all tokens)."""
    ref = oracle.layer(inp)
    assert np.array_equal(got["idx"], ref["idx"])
    assert np.max(np.abs(got["w"] - ref["w"])) <= 1e-5
    assert_layer_close(got["o"], got["n"], ref, inp.gamma, inp.w.eps, "vs oracle")


GRAPH_CASES = [
    ("decode_t8", None),
    ("prefill_small", wl.Workload("prefill_small", T=1024, H=1024, E=16, k=4, I=384, routing="zipf")),
]


@pytest.mark.parametrize("name,w", GRAPH_CASES, ids=[c[0] for c in GRAPH_CASES])
def test_layer_graph_replay(name, w):
    """moe4_layer captured into a HIP graph (torch.cuda.CUDAGraph) and replayed several
    times, with eager calls and synchronisations in between: every replay must give
    the eager call's bytes, which match the oracle."""
    w = wl.workload(name) if w is None else w
    note(f"layer graph replay: {name} T={w.T} H={w.H} E={w.E} k={w.k} I={w.I}")
    inp = wl.make_inputs(w, seed=4)
    if w.routing == "router":
        condition_router_margin(inp)
    g = GpuLayer(inp)
    g.run()
    ref = g.host()
    _check_against_oracle(inp, ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        g.run()  # warm-up on the capture stream's side
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g.run()
    for _ in range(3):
        g.res_out.zero_()
        g.norm_out.zero_()
        g.topk_idx.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = g.host()
        assert np.array_equal(got["idx"], ref["idx"])
        assert np.array_equal(got["o_bits"], ref["o_bits"]) and np.array_equal(got["n_bits"], ref["n_bits"])
        g.run()  # eager work between the replays
        torch.cuda.synchronize()
        again = g.host()
        assert np.array_equal(again["o_bits"], ref["o_bits"])


SIDE_CASES = [
    ("shared_decode", wl.Workload("shared_decode", T=8, H=1024, E=32, k=4, I=256, routing="normal",
                                  n_shared=1)),
    ("shared_prefill", wl.Workload("shared_prefill", T=1024, H=1024, E=8, k=2, I=256, routing="zipf",
                                   n_shared=1)),
]


@pytest.mark.parametrize("name,w", SIDE_CASES, ids=[c[0] for c in SIDE_CASES])
def test_layer_side_stream(name, w):
    """moe4_layer_side (routed chain on a side stream, shared expert on the main stream)
    gives moe4_layer's bytes, which match the oracle, eagerly and captured into a HIP
    graph as a fork and join."""
    note(f"layer side stream: {name} T={w.T} H={w.H} E={w.E} k={w.k} I={w.I} shared={w.n_shared}")
    inp = wl.make_inputs(w, seed=5)
    g = GpuLayer(inp)
    g.run()
    ref = g.host()
    _check_against_oracle(inp, ref)
    side = torch.cuda.Stream()
    for _ in range(2):
        g.res_out.zero_()
        g.norm_out.zero_()
        torch.cuda.synchronize()
        g.run(side_stream=side)
        got = g.host()
        assert np.array_equal(got["idx"], ref["idx"])
        assert np.array_equal(got["o_bits"], ref["o_bits"]) and np.array_equal(got["n_bits"], ref["n_bits"])
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g.run(side_stream=side)
    for _ in range(2):
        g.res_out.zero_()
        g.norm_out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = g.host()
        assert np.array_equal(got["o_bits"], ref["o_bits"]) and np.array_equal(got["n_bits"], ref["n_bits"])


CANONICAL_CASES = [
    ("tiny", None), ("decode_t8", None), ("batched_t64", None),
    ("shared_prefill", wl.Workload("shared_prefill", T=1024, H=1024, E=8, k=2, I=256, routing="zipf",
                                   n_shared=1)),
    ("shared_decode", wl.Workload("shared_decode", T=8, H=1024, E=32, k=4, I=256, routing="normal",
                                  n_shared=1)),
]


@pytest.mark.parametrize("name,w", CANONICAL_CASES, ids=[c[0] for c in CANONICAL_CASES])
def test_layer_canonical_weights(name, w):
    """moe4_layer on weights in the canonical (checkpoint) layout, read as they are:
    the same bits as on the tiled layout, and within the bar of the oracle."""
    w = wl.workload(name) if w is None else w
    note(f"layer canonical weights: {name} T={w.T} H={w.H} E={w.E} k={w.k} I={w.I} shared={w.n_shared}")
    inp = wl.make_inputs(w, seed=6)
    if w.routing == "router":
        condition_router_margin(inp)
    g = GpuLayer(inp, weights=upload_weights(inp, "canonical"))
    g.run()
    got = g.host()
    gt = GpuLayer(inp)
    gt.run()
    ref_bits = gt.host()
    assert np.array_equal(got["idx"], ref_bits["idx"])
    assert np.array_equal(got["o_bits"], ref_bits["o_bits"]) and np.array_equal(got["n_bits"], ref_bits["n_bits"])
    ref = oracle.layer(inp)
    assert np.array_equal(got["idx"], ref["idx"])
    assert_layer_close(got["o"], got["n"], ref, inp.gamma, w.eps, name)


def test_layer_t0_is_a_noop():
    w = wl.workload("tiny")
    inp = wl.make_inputs(w, seed=0, T=0)
    g = GpuLayer(inp)
    g.run()
    torch.cuda.synchronize()


def test_long_prefill_chunks_match_one_call():
    """Tokens are independent, so four calls of 2 048 tokens equal one call of 8 192
    on the routing and, up to FP32 summation order, on the outputs."""
    w = wl.workload("long_prefill")
    note("long prefill: 4 chunks vs 1 call")
    inp = wl.make_inputs(w, seed=0, chunk=1)
    g = GpuLayer(inp)
    g.run()
    full = g.host()
    weights = (g.w13, g.w2, g.shared13, g.shared2, None)
    for c in range(4):
        sl = slice(c * 2048, (c + 1) * 2048)
        part = dataclasses.replace(inp, x=inp.x[sl].copy(), residual=inp.residual[sl].copy(),
                                   logits=inp.logits[sl].copy())
        gp = GpuLayer(part, weights=weights)
        gp.run()
        got = gp.host()
        assert np.array_equal(got["idx"], full["idx"][sl])
        assert rel_rms_err(got["o"], full["o"][sl]) < 1e-2
        assert rel_rms_err(got["n"], full["n"][sl]) < 1e-2
