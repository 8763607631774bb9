"""The FP8 (W4A8) prefill variant on the GPU vs the oracle's reading of it, through the
C ABI (needs an MI355X).

Bars:
  * the activation quantiser: E4M3 codes and E8M0 scale bytes bit-exact (the scale
    choice and the rounding are exact decisions on exact values; a signed zero counts
    as zero);
  * h of the up projection: within one BF16 ulp plus 2^-12 of rms(ref) of the
    oracle's W4A8 SwiGLU, most elements bit-equal (FP8 x FP8 products are exact, so
    the only difference is the GPU's summation against fp64);
  * y of the down projection: the oracle quantises the GPU's own BF16 h the same way
    and sums in fp64; within one BF16 ulp plus 2^-12 of rms(ref). The W4A16 path's
    down step holds 2^-16, but the block-scaled FP8 MFMA does not sum its 64 exact
    products in exact FP32 (measured on gfx950: unit-scale sums of magnitude 275 off by
    up to 2^-9, about 2^-17 of the sum), so its error over I terms reaches a few
    2^-16 of rms; the h step's slack covers it with room. For the same reason more
    sums land across a BF16 rounding boundary than in the W4A16 path (about 10 % at
    K = 2048 against a few %), so at least 75 % of elements must be bit-equal (a
    wrong rounding mode would leave about half);
  * the layer: routing bit-exact; o and n against oracle.layer_w4a8 at the W4A16
    layer bar widened by the E4M3 code flips of h the step bars allow
    (gpu_util.assert_layer_close_w4a8 gives the derivation).
"""
import dataclasses
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
from bit_moe_expert_amd import binding as B
from bit_moe_expert_amd import workloads as wl
from tests.gpu_util import (assert_bf16_close, assert_layer_close_w4a8, bf16_f64, bf16_ulp, condition_router_margin,
                            require_gpu, to_dev, to_host_bits, upload_weights)
from tests.test_gpu_parity import _plan_on_host, _sample_plan_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# ----------------------------------------------------------------------------
# Activation quantiser
# ----------------------------------------------------------------------------
_E4M3_VALUES = oracle.e4m3_value(np.arange(256, dtype=np.uint8))


def _bf16_bits(v):
    """fp64 -> BF16 bits by truncation (the inputs only need to be BF16 values)."""
    return (np.asarray(v, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _quant_cases(rng):
    """Rows of 256 BF16 values (8 blocks each) covering the quantiser's decisions."""
    rows = []
    rows.append(rng.standard_normal((64, 256)))                                    # ordinary
    scale = np.exp2(rng.uniform(-120, 120, (64, 1)))                               # wide range
    rows.append(rng.standard_normal((64, 256)) * np.exp2(rng.uniform(-20, 0, (64, 256))) * scale)
    z = rng.standard_normal((8, 256))
    z[:, 32:64] = 0.0                                                              # zero blocks
    z[:, 64:96] = 0.0
    z[:, 70] = -3.0                                                                # one value
    rows.append(z)
    b = rng.uniform(-1, 1, (16, 256))                                              # scale boundary:
    for j in range(8):                                                             # amax = m * 2^E,
        m = [1.75, 1.7421875, 1.7578125, 1.0, 1.9921875, 1.5, 1.25, 1.875][j]       # m at and around 1.75
        b[:, 32 * j + 5] = m * np.exp2(rng.integers(-30, 30, 16)) * rng.choice([-1, 1], 16)
    rows.append(b)
    tiny = rng.standard_normal((8, 256)) * 2.0 ** -133                             # BF16 subnormals
    tiny[:, :32] = 2.0 ** -133
    rows.append(tiny)
    big = rng.uniform(-1, 1, (8, 256)) * 3.0e38                                    # near the BF16 max
    rows.append(big)
    # E4M3 rounding ties: values halfway between two E4M3 values of a block scaled by 1
    # (amax 448 gives e = 0)
    t = np.zeros((8, 256))
    t[:, ::32] = 448.0
    mids = (_E4M3_VALUES[1:0x7e] + _E4M3_VALUES[2:0x7f]) / 2
    fill = np.resize(mids, (8, 256))
    mask = np.ones(256, dtype=bool)
    mask[::32] = False
    t[:, mask] = fill[:, mask] * rng.choice([-1, 1], (8, int(mask.sum())))
    rows.append(t)
    return _bf16_bits(np.concatenate(rows))


def test_quant_mxfp8_bit_exact():
    rng = np.random.default_rng(2024)
    xb = _quant_cases(rng)
    R, K = xb.shape
    note(f"mxfp8 quant: {R} rows x {K}")
    x = to_dev(xb)
    q = torch.zeros((R, K), dtype=torch.uint8, device="cuda")
    e = torch.zeros((R, K // 32), dtype=torch.uint8, device="cuda")
    B.moe4_quant_mxfp8(x, q, e)
    torch.cuda.synchronize()
    got_q, got_e = q.cpu().numpy(), e.cpu().numpy()
    ref_q, ref_e = oracle.mxfp8_quantize(oracle.bf16_value(xb))
    assert np.array_equal(got_e.astype(np.int64) - 127, ref_e), "scale bytes"
    assert not np.any((got_q & 0x7f) == 0x7f), "NaN codes"
    assert np.array_equal(_E4M3_VALUES[got_q], ref_q), "E4M3 codes"


# ----------------------------------------------------------------------------
# Expert FFN
# ----------------------------------------------------------------------------
W4A8_FFN_CASES = [
    ("tiny", None),
    ("decode_t8", None),
    ("rows_ragged", wl.Workload("rows_ragged", T=301, H=512, E=8, k=2, I=256, routing="zipf")),
    ("prefill_small", wl.Workload("prefill_small", T=1024, H=1024, E=16, k=4, I=384, routing="zipf")),
    ("batched_t64", None),
]


def _w4a8_pair(inp_w13, inp_w2, e):
    return (oracle.dequant_e4m3(inp_w13.packed[e], inp_w13.scales[e]),
            oracle.dequant_e4m3(inp_w2.packed[e], inp_w2.scales[e]))


def _run_w4a8_ffn(inp, w, off, perm, layout="tiled", weights=None):
    dense = off is None
    shape = B.make_shape(inp.T, w.H, 1 if dense else w.E, 1 if dense else w.k, w.I)
    w13, w2 = weights if weights is not None else upload_weights(inp, layout)[:2]
    R = inp.T if dense else inp.T * w.k
    h = torch.zeros((R, w.I), dtype=torch.int16, device="cuda")
    y = torch.zeros((R, w.H), dtype=torch.int16, device="cuda")
    ws = torch.empty(B.moe4_w4a8_workspace_bytes(shape), dtype=torch.uint8, device="cuda")
    B.moe4_expert_ffn_w4a8(shape, to_dev(inp.x), None if dense else to_dev(off),
                           None if dense else to_dev(perm), w13, w2, h, y, ws)
    torch.cuda.synchronize()
    return to_host_bits(h), to_host_bits(y)


def _check_rows(got_h, got_y, x_rows, W13, ts13, W2, ts2, what, min_equal=0.75):
    ref_h = oracle.bf16_round(oracle.swiglu_hidden_w4a8(x_rows, W13, ts13))
    assert_bf16_close(got_h, ref_h, f"h {what}", min_equal=min_equal)
    # the down projection on the GPU's own h (isolates the second GEMM; the oracle
    # quantises the same BF16 values)
    ref_y = oracle.bf16_round(float(ts2) * (oracle._mx_value(got_h) @ W2.T))
    assert_bf16_close(got_y, ref_y, f"y {what}", slack_rms=2.0 ** -12, min_equal=min_equal)


def _check_routed(inp, w, off, perm, rows=None, canonical_too=True):
    h_bits, y_bits = _run_w4a8_ffn(inp, w, off, perm)
    if canonical_too:
        ch, cy = _run_w4a8_ffn(inp, w, off, perm, "canonical")
        assert np.array_equal(ch, h_bits), "h differs between the canonical and the tiled layout"
        assert np.array_equal(cy, y_bits), "y differs between the canonical and the tiled layout"
    got_h, got_y = oracle.bf16_value(h_bits), oracle.bf16_value(y_bits)
    x = oracle.bf16_value(inp.x)
    tok = perm // w.k
    exp_of_row = np.repeat(np.arange(w.E), np.diff(off))
    rows = np.arange(inp.T * w.k) if rows is None else rows

    def check_expert(e):
        rr = rows[exp_of_row[rows] == e]
        if rr.size == 0:
            return
        W13, W2 = _w4a8_pair(inp.w13, inp.w2, e)
        _check_rows(got_h[rr], got_y[rr], x[tok[rr]], W13, inp.w13.tscale[e], W2, inp.w2.tscale[e], f"expert {e}")

    with ThreadPoolExecutor(8) as ex:
        list(ex.map(check_expert, range(w.E)))


@pytest.mark.parametrize("name,w", W4A8_FFN_CASES, ids=[c[0] for c in W4A8_FFN_CASES])
def test_expert_ffn_w4a8_routed(name, w):
    w = wl.workload(name) if w is None else w
    note(f"w4a8 expert ffn routed: {name} T={w.T} H={w.H} E={w.E} k={w.k} I={w.I}")
    inp = wl.make_inputs(w, seed=1)
    idx, _, off, perm, inv = _plan_on_host(inp)
    _check_routed(inp, w, off, perm)


def test_expert_ffn_w4a8_tile_edges():
    """Expert groups on the GEMM's tile boundaries (as for the W4A16 GEMM: tiles of 2 to
    8 blocks of 32 rows and their edges at 64/65, 96/97, 128/129, 160/161, 192/193,
    224/225, 256/257, full tiles with half and three-quarter last ones, 1 row)."""
    counts = [64, 65, 96, 97, 128, 129, 160, 161, 192, 193, 224, 225, 256, 257, 384, 416, 1]
    w = wl.Workload("tile_edges", T=sum(counts), H=512, E=len(counts), k=1, I=256, routing="normal")
    note(f"w4a8 expert ffn tile edges: groups {counts}")
    inp = wl.make_inputs(w, seed=3)
    idx = np.random.default_rng(5).permutation(np.repeat(np.arange(w.E), counts)).astype(np.int32)[:, None]
    off, perm, inv = oracle.permute(idx, w.E)
    _check_routed(inp, w, off, perm)


def test_expert_ffn_w4a8_weight_extremes_and_wide_rows():
    """Weights whose code * scale leaves E4M3's range at both ends: block scales up to
    448 (6 * 448 = 2688 saturates to 448; 4 * 128 = 512 too) and down to E4M3's
    smallest subnormal 2^-9 (0.5 * 2^-9 rounds to 0, ties to even), half of them
    negative (a negative code times a negative scale is positive), non-unit tensor
    scales, and activation rows of very different magnitudes (2^-40 .. 2^20, each
    value within 2^-20 of its row's largest; h grows as the square of x, so larger
    rows would leave FP32) with zero blocks. Checked against the summation bound
    (_check_rows_condition): an element error scales with the sum of its products'
    magnitudes, which such rows make far larger than their rms."""
    w = wl.Workload("w4a8_extremes", T=300, H=512, E=4, k=2, I=256, routing="zipf")
    note("w4a8 expert ffn: saturating and subnormal weights, wide activation rows")
    inp = wl.make_inputs(w, seed=9)
    rng = np.random.default_rng(99)
    for m in (inp.w13, inp.w2):
        u = rng.uniform(-12, 9, m.scales.shape)
        m.scales[:] = wl.to_e4m3_codes(np.minimum(np.exp2(u), 448.0))
        m.scales[m.scales == 0x7f] = 0x7e
        m.scales[:] |= (rng.random(m.scales.shape) < 0.5).astype(np.uint8) << 7  # sign bit
        m.tscale[:] = rng.uniform(0.25, 2.0, m.tscale.shape).astype(np.float32)
    row_scale = np.exp2(rng.uniform(-40, 20, (inp.T, 1)))
    xv = rng.standard_normal((inp.T, w.H)) * np.exp2(rng.uniform(-20, 0, (inp.T, w.H))) * row_scale
    xv[:, 64:128] = 0.0
    inp.x[:] = wl.to_bf16_bits(xv)
    W13 = oracle.dequant(inp.w13.packed[0], inp.w13.scales[0], 1.0)
    assert np.any(np.abs(W13) > 448) and np.any((W13 != 0) & (np.abs(W13) < 2.0 ** -9))
    assert np.any(oracle.e4m3_value(inp.w13.scales[0]) < 0)
    idx, _, off, perm, inv = _plan_on_host(inp)
    h_bits, y_bits = _run_w4a8_ffn(inp, w, off, perm)
    got_h, got_y = oracle.bf16_value(h_bits), oracle.bf16_value(y_bits)
    x = oracle.bf16_value(inp.x)
    tok = perm // w.k
    exp_of_row = np.repeat(np.arange(w.E), np.diff(off))
    for e in np.unique(exp_of_row):
        W13, W2 = _w4a8_pair(inp.w13, inp.w2, e)
        rr = np.flatnonzero(exp_of_row == e)
        _check_rows_condition(got_h[rr], got_y[rr], x[tok[rr]], W13, inp.w13.tscale[e], W2, inp.w2.tscale[e],
                              f"expert {e}")


def _check_rows_condition(got_h, got_y, x_rows, W13, ts13, W2, ts2, what, eps=2.0 ** -12):
    """Step check with the summation bound in place of an rms slack: each element of
    g, u (and y) may be off by eps times the sum of the magnitudes of its products
    (a summation's error scales with that sum, and with weights spanning 2^21 within a
    row it can far exceed the row's rms), carried through SwiGLU (|silu'| <= 1.1),
    plus one BF16 ulp. eps = 2^-12 is 8x the FP8 MFMA's measured error per
    instruction relative to its largest product."""
    I = W13.shape[0] // 2
    xq = oracle._mx_value(x_rows)
    g, u = float(ts13) * (xq @ W13[:I].T), float(ts13) * (xq @ W13[I:].T)
    ag, au = abs(float(ts13)) * (np.abs(xq) @ np.abs(W13[:I]).T), abs(float(ts13)) * (np.abs(xq) @ np.abs(W13[I:]).T)
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-g))
    ref_h = oracle.bf16_round(g * sig * u)
    tol_h = bf16_ulp(ref_h) + eps * (1.1 * np.abs(u) * ag + np.abs(g * sig) * au)
    assert np.all(np.abs(got_h - ref_h) <= tol_h), f"h {what}: worst {float(np.max(np.abs(got_h - ref_h) / tol_h)):.2f}x"
    hq = oracle._mx_value(got_h)
    ref_y = oracle.bf16_round(float(ts2) * (hq @ W2.T))
    tol_y = bf16_ulp(ref_y) + eps * abs(float(ts2)) * (np.abs(hq) @ np.abs(W2).T)
    assert np.all(np.abs(got_y - ref_y) <= tol_y), f"y {what}: worst {float(np.max(np.abs(got_y - ref_y) / tol_y)):.2f}x"


@pytest.mark.parametrize("T", [1, 50, 77, 100, 150, 220, 300])
def test_expert_ffn_w4a8_dense_shared(T):
    """Dense (shared expert) mode: tiles of 2, 3, 4, 5 and 7 blocks of 32 rows, a full
    tile plus a 2-block one; T = 1 as the degenerate case."""
    w = wl.Workload("shared_small", T=T, H=1024, E=1, k=1, I=512, routing="normal")
    note(f"w4a8 expert ffn dense T={T}")
    inp = wl.make_inputs(w, seed=2)
    h_bits, y_bits = _run_w4a8_ffn(inp, w, None, None)
    W13, W2 = _w4a8_pair(inp.w13, inp.w2, 0)
    _check_rows(oracle.bf16_value(h_bits), oracle.bf16_value(y_bits), oracle.bf16_value(inp.x), W13,
                inp.w13.tscale[0], W2, inp.w2.tscale[0], "dense")


@pytest.mark.parametrize("name", ["prefill", "long_prefill"])
def test_expert_ffn_w4a8_full_size_sampled_rows(name):
    """The W4A8 FFN at the full prefill and long-prefill shapes (8192 tokens, Zipf
    routing): sampled plan rows (first and last rows of every expert, rows of its last
    tile, random rows, every row of the hottest expert and of experts with a half and a
    three-quarter last tile) at the step bars."""
    w = wl.workload(name)
    inp = wl.make_inputs(w, seed=0, chunk=0)
    idx, _, off, perm, inv = _plan_on_host(inp)
    rows, full = _sample_plan_rows(off, np.random.default_rng(56))
    note(f"w4a8 expert ffn full size: {name}: {rows.size} plan rows checked, every row of experts {full}")
    _check_routed(inp, w, off, perm, rows=rows, canonical_too=False)


# ----------------------------------------------------------------------------
# Layer
# ----------------------------------------------------------------------------
class GpuLayerW4A8:
    def __init__(self, inp, weights=None):
        w = inp.w
        self.shape = B.make_shape(inp.T, w.H, w.E, w.k, w.I, w.n_shared, w.eps)
        self.x, self.residual, self.gamma = to_dev(inp.x), to_dev(inp.residual), to_dev(inp.gamma)
        self.w13, self.w2, self.s13, self.s2, self.wr = weights if weights is not None else upload_weights(inp)
        self.logits = (to_dev(inp.logits) if inp.logits is not None
                       else torch.empty((inp.T, w.E), dtype=torch.float32, device="cuda"))
        self.idx = torch.full((inp.T, w.k), -1, dtype=torch.int32, device="cuda")
        self.tw = torch.zeros((inp.T, w.k), dtype=torch.float32, device="cuda")
        self.o = torch.zeros((inp.T, w.H), dtype=torch.int16, device="cuda")
        self.n = torch.zeros((inp.T, w.H), dtype=torch.int16, device="cuda")
        self.ws = torch.empty(B.moe4_w4a8_workspace_bytes(self.shape), dtype=torch.uint8, device="cuda")

    def run(self):
        B.moe4_layer_w4a8(self.shape, self.x, self.wr, self.logits, self.w13, self.w2, self.s13, self.s2,
                          self.residual, self.gamma, self.idx, self.tw, self.o, self.n, self.ws)
        torch.cuda.synchronize()
        return (self.idx.cpu().numpy(), self.tw.cpu().numpy().astype(np.float64), bf16_f64(self.o),
                bf16_f64(self.n))


# (batched_t64's 256 experts are covered by the FFN step test and by the routing test
# below, which runs the whole layer at that shape)
@pytest.mark.parametrize("name,sample", [("tiny", None), ("decode_t8", None), ("prefill", 1024)])
def test_layer_w4a8(name, sample):
    w = wl.workload(name)
    note(f"w4a8 layer: {name} T={w.T} H={w.H} E={w.E} k={w.k} I={w.I} shared={w.n_shared}")
    inp = wl.make_inputs(w, seed=0)
    if w.routing == "router":
        condition_router_margin(inp)
    idx, tw, o, n = GpuLayerW4A8(inp).run()
    L = inp.logits.astype(np.float64) if inp.logits is not None else oracle.router_logits(inp.x, inp.w_router)
    ref_idx, ref_w = oracle.route(L, w.k)
    assert np.array_equal(idx, ref_idx)
    assert np.max(np.abs(tw - ref_w)) <= 1e-5
    tokens = None if sample is None else np.sort(np.random.default_rng(123).choice(w.T, sample, replace=False))
    ref = oracle.layer_w4a8(inp, tokens=tokens, logits=L if tokens is None else L[tokens])
    sel = ref["tokens"]
    assert_layer_close_w4a8(o[sel], n[sel], ref, inp, f"w4a8 {name}")


def test_layer_w4a8_long_prefill_chunk():
    """Long prefill (shared expert, 160 experts, H = 6144): one chunk of 8192 tokens,
    routing of every token bit-exact, o and n of 512 sampled tokens at the layer bar."""
    w = wl.workload("long_prefill")
    note("w4a8 layer: long prefill chunk 1, 512 sampled tokens")
    base = wl.make_inputs(w, seed=0, chunk=0)
    inp = wl.make_inputs(w, seed=0, chunk=1, weights_from=base)
    idx, tw, o, n = GpuLayerW4A8(inp).run()
    L = inp.logits.astype(np.float64)
    assert np.array_equal(idx, oracle.route(L, w.k)[0])
    tok = np.sort(np.random.default_rng(77).choice(w.T, 512, replace=False))
    ref = oracle.layer_w4a8(inp, tokens=tok, logits=L[tok])
    assert_layer_close_w4a8(o[tok], n[tok], ref, inp, "w4a8 long prefill")


def test_layer_w4a8_shares_routing_with_w4a16():
    """The FP8 form changes only the expert FFNs: the routing outputs equal those of
    moe4_layer bit for bit, and the two layers' outputs differ by about the FP8
    quantisation: the oracle puts the rms of that difference near 6 % of rms(o) on
    workloads of this kind (E4M3 keeps 4 significant bits)."""
    from tests.gpu_util import GpuLayer
    w = wl.workload("batched_t64")
    inp = wl.make_inputs(w, seed=5)
    weights = upload_weights(inp)
    g = GpuLayer(inp, weights=weights)
    g.run()
    ref = g.host()
    idx, tw, o, n = GpuLayerW4A8(inp, weights=weights).run()
    assert np.array_equal(idx, ref["idx"])
    assert np.array_equal(tw, ref["w"])
    rel = float(np.sqrt(np.mean((o - ref["o"]) ** 2) / np.mean(ref["o"] ** 2)))
    note(f"  w4a8 vs w4a16 layer: rms difference {rel:.3f} of rms(o)")
    assert 0.01 <= rel <= 0.15


def test_w4a8_halves_compose_and_h_quantisation():
    """moe4_quant_mxfp8 -> moe4_expert_up_w4a8 -> moe4_expert_down_w4a8 gives the bits of
    moe4_expert_ffn_w4a8, and the FP8 h the up half writes is bit for bit the oracle's
    quantisation of its own BF16 h (the epilogue quantiser against the oracle)."""
    w = wl.Workload("rows_ragged", T=301, H=512, E=8, k=2, I=256, routing="zipf")
    inp = wl.make_inputs(w, seed=12)
    idx, _, off, perm, inv = _plan_on_host(inp)
    h_ref, y_ref = _run_w4a8_ffn(inp, w, off, perm)
    shape = B.make_shape(inp.T, w.H, w.E, w.k, w.I)
    w13, w2 = upload_weights(inp)[:2]
    R = inp.T * w.k
    x = to_dev(inp.x)
    x8 = torch.zeros((inp.T, w.H), dtype=torch.uint8, device="cuda")
    xs = torch.zeros((inp.T, w.H // 32), dtype=torch.uint8, device="cuda")
    h = torch.zeros((R, w.I), dtype=torch.int16, device="cuda")
    h8 = torch.zeros((R, w.I), dtype=torch.uint8, device="cuda")
    hs = torch.zeros((R, w.I // 32), dtype=torch.uint8, device="cuda")
    y = torch.zeros((R, w.H), dtype=torch.int16, device="cuda")
    offs, perms = to_dev(off), to_dev(perm)
    B.moe4_quant_mxfp8(x, x8, xs)
    B.moe4_expert_up_w4a8(shape, x8, xs, offs, perms, w13, h, h8, hs)
    B.moe4_expert_down_w4a8(shape, h8, hs, offs, w2, y)
    torch.cuda.synchronize()
    assert np.array_equal(to_host_bits(h), h_ref)
    assert np.array_equal(to_host_bits(y), y_ref)
    q, e = oracle.mxfp8_quantize(oracle.bf16_value(h_ref))
    assert np.array_equal(hs.cpu().numpy().astype(np.int64) - 127, e)
    assert np.array_equal(_E4M3_VALUES[h8.cpu().numpy()], q)
    # without the BF16 h the FP8 h is the same
    h8b = torch.zeros_like(h8)
    hsb = torch.zeros_like(hs)
    B.moe4_expert_up_w4a8(shape, x8, xs, offs, perms, w13, None, h8b, hsb)
    torch.cuda.synchronize()
    assert torch.equal(h8b, h8) and torch.equal(hsb, hs)


def test_layer_w4a8_canonical_weights_same_bits():
    """Weights in the canonical (checkpoint) layout run the same kernels and give the
    same bits as the tiled layout, and the layer meets the W4A8 bar."""
    w = wl.Workload("w4a8_canon", T=96, H=512, E=8, k=2, I=256, routing="zipf", n_shared=1)
    inp = wl.make_inputs(w, seed=21)
    tiled = GpuLayerW4A8(inp, weights=upload_weights(inp, "tiled")).run()
    canon = GpuLayerW4A8(inp, weights=upload_weights(inp, "canonical")).run()
    for a, b in zip(tiled, canon):
        assert np.array_equal(a, b)
    ref = oracle.layer_w4a8(inp)
    assert np.array_equal(tiled[0], ref["idx"])
    assert_layer_close_w4a8(tiled[2], tiled[3], ref, inp, "w4a8 canonical")


def test_w4a8_t0_is_a_noop():
    """T = 0 enqueues nothing and leaves the outputs untouched."""
    w = wl.workload("tiny")
    shape = B.make_shape(0, w.H, w.E, w.k, w.I)
    inp = wl.make_inputs(w, seed=0, T=1)
    w13, w2 = upload_weights(inp)[:2]
    y = torch.full((4, w.H), 7, dtype=torch.int16, device="cuda")
    x = to_dev(inp.x)
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    B.moe4_expert_ffn_w4a8(shape, x, None, None, w13, w2, None, y, ws)
    q = torch.full((1, w.H), 3, dtype=torch.uint8, device="cuda")
    e = torch.full((1, w.H // 32), 3, dtype=torch.uint8, device="cuda")
    B.moe4_quant_mxfp8(x[:0], q, e)
    torch.cuda.synchronize()
    assert bool((y == 7).all()) and bool((q == 3).all()) and bool((e == 3).all())


def test_expert_ffn_w4a8_all_rows_one_expert():
    """Every routed row on one expert of many (k = 1): a run of full tiles, a ragged
    last tile, and 63 empty experts in the schedule."""
    w = wl.Workload("w4a8_one", T=700, H=512, E=64, k=1, I=256, routing="normal")
    inp = wl.make_inputs(w, seed=22)
    idx = np.full((w.T, 1), 37, dtype=np.int32)
    off, perm, inv = oracle.permute(idx, w.E)
    note("w4a8 expert ffn: 700 rows on expert 37 of 64")
    _check_routed(inp, w, off, perm)


@pytest.mark.parametrize("name", ["decode_t1", "decode_t8"])
def test_layer_w4a8_decode_shapes_with_shared(name):
    """The FP8 form at decode shapes (one or eight tokens) with a shared expert: the
    prefill GEMM on a few rows per expert, dense mode with T < one tile."""
    w = dataclasses.replace(wl.workload(name), n_shared=1)
    inp = wl.make_inputs(w, seed=23)
    condition_router_margin(inp)
    idx, tw, o, n = GpuLayerW4A8(inp).run()
    ref = oracle.layer_w4a8(inp)
    assert np.array_equal(idx, ref["idx"])
    assert_layer_close_w4a8(o, n, ref, inp, f"w4a8 {name} + shared")
