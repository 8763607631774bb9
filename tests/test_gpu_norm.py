"""add_rmsnorm and group_rmsnorm: HIP path vs the fp64 oracle, through the C ABI.

Bars (derived from the arithmetic): the residual sum o is one FP32 sum of two BF16
values rounded once to BF16, so |o_gpu - o_ref| <= 2^-8 |o_ref| (+ FP32 slack); n is
computed in FP32 from the FP32 sums and rounded once to BF16, so |n_gpu - n_ref| <=
2^-7 |n_ref| (+ FP32 slack of the sum of squares).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from bit_moe_expert_amd import binding as B
from bit_moe_expert_amd import workloads as wl
from tests.gpu_util import bf16_f64, require_gpu, to_dev, to_host_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _rows(rng, T, H):
    # rows of different scales (1e-3 .. 1e3) so the norm's scale matters
    scale = 10.0 ** rng.uniform(-3, 3, (T, 1))
    return wl.to_bf16_bits(rng.standard_normal((T, H)) * scale)


def _check_o(got, ref):
    assert np.all(np.abs(got - ref) <= 2 ** -8 * np.abs(ref) + 1e-6 * np.abs(ref).max(axis=1, keepdims=True))


def _check_n(got, ref):
    assert np.all(np.abs(got - ref) <= 2 ** -7 * np.abs(ref) + 1e-5 * np.abs(ref).max(axis=1, keepdims=True))


# decode rows (H = 2048), batched and prefill rows (4096, 6144), the largest H, and
# ragged widths (chunks not a multiple of the 256 threads, fewer chunks than threads)
ADD_CASES = [(1, 2048), (8, 2048), (3, 8), (5, 24), (17, 4104), (64, 6144), (16, 16384), (8192, 4096),
             (0, 2048)]


@pytest.mark.parametrize("T,H", ADD_CASES, ids=[f"T{t}_H{h}" for t, h in ADD_CASES])
def test_add_rmsnorm(T, H):
    note(f"add_rmsnorm T={T} H={H}")
    rng = np.random.default_rng(1000 + T * 7 + H)
    x = _rows(rng, T, H)
    res = _rows(rng, T, H)
    gam = wl.to_bf16_bits(rng.uniform(0.5, 1.5, H))
    d_x, d_res, d_g = to_dev(x), to_dev(res), to_dev(gam)
    out_o = torch.zeros((T, H), dtype=torch.int16, device="cuda")
    out_n = torch.zeros((T, H), dtype=torch.int16, device="cuda")
    B.moe4_add_rmsnorm(d_x, d_res, d_g, out_o, out_n, eps=1e-6)
    torch.cuda.synchronize()
    if T == 0:
        return
    ref_o, ref_n = oracle.add_rmsnorm(x, res, gam, 1e-6)
    _check_o(bf16_f64(out_o), ref_o)
    _check_n(bf16_f64(out_n), ref_n)
    # in place: residual_out aliases residual, normed_out aliases x; same bits
    B.moe4_add_rmsnorm(d_x, d_res, d_g, d_res, d_x, eps=1e-6)
    torch.cuda.synchronize()
    assert np.array_equal(to_host_bits(d_res), to_host_bits(out_o))
    assert np.array_equal(to_host_bits(d_x), to_host_bits(out_n))


GROUP_CASES = [(8, 4096, 512), (1, 2048, 256), (3, 24, 8), (5, 2048, 2048), (7, 16384, 8), (9, 6144, 768),
               (4, 1000, 200), (33, 16384, 16384), (2048, 4096, 1024), (0, 64, 16)]


@pytest.mark.parametrize("T,H,G", GROUP_CASES, ids=[f"T{t}_H{h}_G{g}" for t, h, g in GROUP_CASES])
def test_group_rmsnorm(T, H, G):
    note(f"group_rmsnorm T={T} H={H} group={G}")
    rng = np.random.default_rng(2000 + T * 7 + H + G)
    x = _rows(rng, T, H)
    # groups of one row at different scales too
    if T:
        x = wl.to_bf16_bits(oracle.bf16_value(x) * np.repeat(10.0 ** rng.uniform(-2, 2, H // G), G)[None, :])
    gam = wl.to_bf16_bits(rng.uniform(0.5, 1.5, H))
    d_x = to_dev(x)
    out_n = torch.zeros((T, H), dtype=torch.int16, device="cuda")
    B.moe4_group_rmsnorm(d_x, G, to_dev(gam), out_n, eps=1e-6)
    torch.cuda.synchronize()
    if T == 0:
        return
    _check_n(bf16_f64(out_n), oracle.group_rmsnorm(x, G, gam, 1e-6))
    # in place
    B.moe4_group_rmsnorm(d_x, G, to_dev(gam), d_x, eps=1e-6)
    torch.cuda.synchronize()
    assert np.array_equal(to_host_bits(d_x), to_host_bits(out_n))


def test_group_rmsnorm_closed_form_and_batch_invariance():
    """A constant group c normalises to sign(c) * gamma; each row's bits do not depend
    on the batch it is computed in; group == H equals add_rmsnorm of x + 0."""
    T, H, G = 6, 2048, 256
    rng = np.random.default_rng(9)
    vals = rng.choice([-3.0, -0.5, 0.25, 2.0, 7.0], size=(T, H // G))
    x = wl.to_bf16_bits(np.repeat(vals, G, axis=1))
    gam = wl.to_bf16_bits(rng.uniform(0.5, 1.5, H))
    out = torch.zeros((T, H), dtype=torch.int16, device="cuda")
    B.moe4_group_rmsnorm(to_dev(x), G, to_dev(gam), out, eps=1e-12)
    torch.cuda.synchronize()
    want = np.sign(np.repeat(vals, G, axis=1)) * oracle.bf16_value(gam)[None, :]
    assert np.all(np.abs(bf16_f64(out) - want) <= 2 ** -8 * np.abs(want))

    xr = _rows(rng, T, H)
    full = torch.zeros((T, H), dtype=torch.int16, device="cuda")
    B.moe4_group_rmsnorm(to_dev(xr), G, to_dev(gam), full, eps=1e-6)
    for t in (0, T - 1):
        one = torch.zeros((1, H), dtype=torch.int16, device="cuda")
        B.moe4_group_rmsnorm(to_dev(xr[t:t + 1]), G, to_dev(gam), one, eps=1e-6)
        torch.cuda.synchronize()
        assert np.array_equal(to_host_bits(one)[0], to_host_bits(full)[t])

    zeros = np.zeros((T, H), dtype=np.uint16)
    o = torch.zeros((T, H), dtype=torch.int16, device="cuda")
    n_add = torch.zeros((T, H), dtype=torch.int16, device="cuda")
    n_grp = torch.zeros((T, H), dtype=torch.int16, device="cuda")
    B.moe4_add_rmsnorm(to_dev(xr), to_dev(zeros), to_dev(gam), o, n_add, eps=1e-6)
    B.moe4_group_rmsnorm(to_dev(xr), H, to_dev(gam), n_grp, eps=1e-6)
    torch.cuda.synchronize()
    assert np.array_equal(to_host_bits(o), xr)
    assert np.array_equal(to_host_bits(n_add), to_host_bits(n_grp))


def test_glue_graph_replay():
    """Both launches captured into a HIP graph: every replay, with eager work and
    synchronisations between replays, gives the eager launch's bits."""
    T, H, G = 8, 2048, 256
    rng = np.random.default_rng(21)
    x, res = to_dev(_rows(rng, T, H)), to_dev(_rows(rng, T, H))
    gam = to_dev(wl.to_bf16_bits(rng.uniform(0.5, 1.5, H)))
    outs = [torch.zeros((T, H), dtype=torch.int16, device="cuda") for _ in range(3)]
    B.moe4_add_rmsnorm(x, res, gam, outs[0], outs[1])
    B.moe4_group_rmsnorm(x, G, gam, outs[2])
    torch.cuda.synchronize()
    want = [to_host_bits(o) for o in outs]
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        B.moe4_add_rmsnorm(x, res, gam, outs[0], outs[1])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        B.moe4_add_rmsnorm(x, res, gam, outs[0], outs[1])
        B.moe4_group_rmsnorm(x, G, gam, outs[2])
    for rep in range(3):
        for o in outs:
            o.zero_()
        B.moe4_group_rmsnorm(res, 512, gam, torch.empty_like(res))   # unrelated eager work
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for o, w in zip(outs, want):
            assert np.array_equal(to_host_bits(o), w), f"replay {rep}"
