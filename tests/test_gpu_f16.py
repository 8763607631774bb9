"""The up projection's GEMM on FP16 activations (moe4_act_f16 + moe4_expert_up_f16, and
moe4_layer, which takes that form wherever its up projections run on the GEMM).

The pre-pass is checked against its definition written out here (a per-row power of two
from the row's largest magnitude, then round to nearest FP16); the GEMM against the BF16
GEMM (moe4_expert_up) bit for bit wherever the FP16 rows hold x exactly, and against the
oracle's SwiGLU in every case."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from bit_moe_expert_amd import binding as B
from bit_moe_expert_amd import workloads as wl
from tests.gpu_util import assert_bf16_close, bf16_f64, require_gpu, to_dev, to_host_bits, upload_weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def note(msg):
    print(f"[f16] {msg}", flush=True)


def act_f16_reference(x_bits: np.ndarray):
    """xexp[t]: the smallest integer e with max_k |x[t][k]| * 2^-e < 2^15 (0 for a zero
    row; NaN ignored); x16 = x * 2^-e rounded to FP16 (numpy's float64 -> float16 is
    round to nearest even, subnormals included; x * 2^-e is exact in float64)."""
    x = oracle.bf16_value(x_bits)
    a = np.where(np.isnan(x), 0.0, np.abs(x))
    amax = a.max(axis=1)
    _, ex = np.frexp(amax)                       # amax = m * 2^ex, 0.5 <= m < 1
    e = np.where(amax > 0, ex.astype(np.int64) - 1 - 14, 0)
    x16 = np.ldexp(x, -e[:, None]).astype(np.float16)
    return x16.view(np.uint16), e.astype(np.int32)


def run_act_f16(x_bits: np.ndarray):
    rows, K = x_bits.shape
    x16 = torch.zeros((rows, K), dtype=torch.float16, device="cuda")
    xexp = torch.zeros(rows, dtype=torch.int32, device="cuda")
    B.moe4_act_f16(to_dev(x_bits), x16, xexp)
    torch.cuda.synchronize()
    return x16, xexp


def test_act_f16_matches_definition():
    """Rows of N(0,1) values, rows at scales 2^-120 .. 2^120, rows whose values span 2^40
    below their maximum (down into FP16 subnormals and zero), BF16 subnormals, a zero row,
    a row with one nonzero value, signed zeros, and K = 8 and 16384 (the limits)."""
    rng = np.random.default_rng(31)
    for K in (8, 2048, 6144, 16384):
        rows = []
        rows.append(rng.standard_normal((4, K)))
        rows.append(rng.standard_normal((4, K)) * np.exp2(rng.uniform(-120, 120, (4, 1))))
        rows.append(rng.standard_normal((4, K)) * np.exp2(rng.uniform(-40, 0, (4, K))))
        rows.append(rng.standard_normal((1, K)) * 2.0 ** -130)            # BF16 subnormals
        rows.append(np.zeros((1, K)))
        one = np.zeros((1, K))
        one[0, K // 3] = -3.0
        rows.append(one)
        rows.append(-np.zeros((1, K)))
        x_bits = wl.to_bf16_bits(np.concatenate(rows))
        note(f"act_f16 K={K} rows={x_bits.shape[0]}")
        x16, xexp = run_act_f16(x_bits)
        ref16, refe = act_f16_reference(x_bits)
        assert np.array_equal(xexp.cpu().numpy(), refe), f"K={K}: exponents"
        got = x16.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, ref16), f"K={K}: FP16 rows ({np.count_nonzero(got != ref16)} values differ)"


def _up_both(inp, w, off, perm, layout="tiled", dense=False):
    """h of the BF16 GEMM (moe4_expert_up) and of the FP16-activation GEMM, as bits."""
    G = 1 if dense else w.E
    shape = B.make_shape(inp.T, w.H, G, 1 if dense else w.k, w.I)
    w13, *_ = upload_weights(inp, layout)
    R = inp.T if dense else inp.T * w.k
    x = to_dev(inp.x)
    offs = None if dense else to_dev(off)
    ps = None if dense else to_dev(perm)
    h = torch.zeros((R, w.I), dtype=torch.int16, device="cuda")
    B.moe4_expert_up(shape, x, offs, ps, w13, h)
    x16 = torch.zeros((inp.T, w.H), dtype=torch.float16, device="cuda")
    xexp = torch.zeros(inp.T, dtype=torch.int32, device="cuda")
    B.moe4_act_f16(x, x16, xexp)
    h16 = torch.full((R, w.I), -1, dtype=torch.int16, device="cuda")
    B.moe4_expert_up_f16(shape, x16, xexp, offs, ps, w13, h16)
    torch.cuda.synchronize()
    return to_host_bits(h), to_host_bits(h16)


def _ref_h(inp, w, off, perm):
    x = oracle.bf16_value(inp.x)
    tok = perm // w.k
    exp_of_row = np.repeat(np.arange(w.E), np.diff(off))
    ref = np.zeros((len(perm), w.I))
    for e in np.unique(exp_of_row):
        rows = np.flatnonzero(exp_of_row == e)
        W13 = oracle.dequant(inp.w13.packed[e], inp.w13.scales[e], inp.w13.tscale[e])
        ref[rows] = oracle.bf16_round(oracle.swiglu_hidden(x[tok[rows]], W13))
    return ref


def _plan(inp):
    idx, _ = oracle.route(inp.logits.astype(np.float64), inp.w.k)
    return oracle.permute(idx, inp.w.E)


ROUTED = [
    ("rows_ragged", wl.Workload("rows_ragged", T=301, H=512, E=8, k=2, I=256, routing="zipf")),
    ("prefill_small", wl.Workload("prefill_small", T=1024, H=1024, E=16, k=4, I=384, routing="zipf")),
    # few rows per expert: the FP16 entry point still runs the GEMM (half tiles)
    ("few_rows", wl.Workload("few_rows", T=64, H=1024, E=32, k=4, I=256, routing="normal")),
]


@pytest.mark.parametrize("name,w", ROUTED, ids=[c[0] for c in ROUTED])
@pytest.mark.parametrize("layout", ["tiled", "canonical"])
def test_expert_up_f16_same_bits(name, w, layout):
    note(f"expert up f16: {name} T={w.T} H={w.H} E={w.E} k={w.k} I={w.I} {layout}")
    inp = wl.make_inputs(w, seed=21)
    off, perm, _ = _plan(inp)
    h, h16 = _up_both(inp, w, off, perm, layout)
    if w.T * w.k >= 40 * w.E:
        # moe4_expert_up runs the BF16 GEMM here (below 40 rows per expert on average it
        # streams the weights instead, summing in another order)
        assert np.array_equal(h16, h), f"{np.count_nonzero(h16 != h)} of {h.size} h values differ from the BF16 GEMM"
    assert_bf16_close(oracle.bf16_value(h16), _ref_h(inp, w, off, perm), "h")


def test_expert_up_f16_tile_edges():
    """Expert groups on the GEMM's tile boundaries (as the BF16 GEMM's tile-edge test)."""
    counts = [64, 65, 96, 97, 128, 129, 160, 161, 192, 193, 224, 225, 256, 257, 384, 416, 1]
    w = wl.Workload("tile_edges", T=sum(counts), H=512, E=len(counts), k=1, I=256, routing="normal")
    note(f"expert up f16 tile edges: {counts}")
    inp = wl.make_inputs(w, seed=23)
    idx = np.random.default_rng(25).permutation(np.repeat(np.arange(w.E), counts)).astype(np.int32)[:, None]
    off, perm, _ = oracle.permute(idx, w.E)
    h, h16 = _up_both(inp, w, off, perm)
    assert np.array_equal(h16, h)
    assert_bf16_close(oracle.bf16_value(h16), _ref_h(inp, w, off, perm), "h")


@pytest.mark.parametrize("T", [40, 77, 100, 150, 220, 300])
def test_expert_up_f16_dense(T):
    """Dense (shared expert) mode: tiles of 2, 3, 4, 5 and 7 blocks of 32 rows, a full
    tile plus a 2-block one."""
    w = wl.Workload("shared_small", T=T, H=1024, E=1, k=1, I=512, routing="normal")
    note(f"expert up f16 dense T={T}")
    inp = wl.make_inputs(w, seed=22)
    h, h16 = _up_both(inp, w, None, None, dense=True)
    assert np.array_equal(h16, h)
    x = oracle.bf16_value(inp.x)
    W13 = oracle.dequant(inp.w13.packed[0], inp.w13.scales[0], inp.w13.tscale[0])
    assert_bf16_close(oracle.bf16_value(h16), oracle.bf16_round(oracle.swiglu_hidden(x, W13)), "h")


def test_expert_up_f16_wide_range_rows():
    """Rows at scales 2^-50 .. 2^26 (larger ones overflow h = silu(g) * u) whose values
    span up to 2^31 below the row's largest
    (x16 holds x exactly: the BF16 GEMM's bits), then rows spanning 2^45 (the smallest
    values round in FP16: each row of h still within the oracle's bar on its own scale)."""
    w = wl.Workload("wide_f16", T=512, H=1024, E=8, k=2, I=256, routing="zipf")
    inp = wl.make_inputs(w, seed=27)
    off, perm, _ = _plan(inp)
    rng = np.random.default_rng(271)
    for span, exact in ((31, True), (45, False)):
        note(f"expert up f16 wide-range rows: values within 2^{span} of each row's maximum")
        scale = np.exp2(rng.uniform(-50, 26, (inp.T, 1)))
        within = np.exp2(rng.uniform(-span, 0, (inp.T, w.H)))
        inp.x[:] = wl.to_bf16_bits(rng.standard_normal((inp.T, w.H)) * within * scale)
        h, h16 = _up_both(inp, w, off, perm)
        if exact:
            assert np.array_equal(h16, h)
        got = oracle.bf16_value(h16)
        ref = _ref_h(inp, w, off, perm)
        for r in range(len(perm)):
            assert_bf16_close(got[r], ref[r], f"h row {r}", min_equal=0.8)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["prefill", "long_prefill"])
def test_expert_up_f16_full_size_same_bits(name):
    """At the full prefill shapes (T = 8192: 128 experts, I = 1536; 160 experts, H = 6144,
    I = 2048, plus the shared expert's dense call), every h value of the FP16 GEMM equals
    the BF16 GEMM's."""
    w = wl.workload(name)
    note(f"expert up f16 full size: {name}")
    inp = wl.make_inputs(w, seed=0)
    off, perm, _ = _plan(inp)
    h, h16 = _up_both(inp, w, off, perm)
    assert np.array_equal(h16, h), f"{np.count_nonzero(h16 != h)} of {h.size} h values differ"
    if w.n_shared:
        sw = dataclasses.replace(w, E=1, k=1)
        h, h16 = _up_both(dataclasses.replace(inp, w13=inp.shared13), sw, None, None, dense=True)
        assert np.array_equal(h16, h), "shared expert"
