"""moe4_layer_noalloc (the layer on the library's static per-GPU scratch) gives the
same bytes as moe4_layer with a caller workspace, through the C ABI, on calls in a
row whose shapes shrink (the scratch keeps the previous call's contents)."""
import numpy as np
import pytest
import torch

from bit_moe_expert_amd import binding as B
from bit_moe_expert_amd import workloads as wl
from tests.gpu_util import GpuLayer, condition_router_margin, require_gpu, to_host_bits, upload_weights

pytestmark = pytest.mark.gpu


def _noalloc_outputs(g):
    T, w = g.inp.T, g.inp.w
    idx = torch.full((T, w.k), -1, dtype=torch.int32, device="cuda")
    tw = torch.zeros((T, w.k), dtype=torch.float32, device="cuda")
    o = torch.zeros((T, w.H), dtype=torch.int16, device="cuda")
    n = torch.zeros((T, w.H), dtype=torch.int16, device="cuda")
    logits = g.logits.clone() if g.inp.logits is not None else torch.zeros_like(g.logits)
    B.moe4_layer_noalloc(g.shape, g.x, g.w_router, logits, g.w13, g.w2, g.shared13, g.shared2, g.residual,
                         g.gamma, idx, tw, o, n)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), tw.cpu().numpy(), to_host_bits(o), to_host_bits(n)


def _same_as_workspace_call(inp, weights):
    g = GpuLayer(inp, weights=weights)
    g.run()
    ref = g.host()
    idx, tw, o, n = _noalloc_outputs(g)
    assert np.array_equal(idx, ref["idx"])
    assert np.array_equal(tw.view(np.int32), g.topk_w.cpu().numpy().view(np.int32))
    assert np.array_equal(o, ref["o_bits"]) and np.array_equal(n, ref["n_bits"])


# (workload, token counts of the calls in a row: each later call smaller)
CASES = [
    ("shared_batch", wl.Workload("shared_batch", T=64, H=1024, E=32, k=4, I=256, routing="zipf", n_shared=1),
     [64, 5]),
    ("decode", wl.workload("decode_t8"), [8, 1]),
    ("batched_t256", wl.workload("batched_t256"), [256, 40]),
    # enough rows per expert for the GEMM: the up projections run on FP16 activation
    # rows, which the scratch holds too (the second call still on the GEMM, the third
    # back on the streaming kernels)
    ("gemm_f16", wl.Workload("gemm_f16", T=1024, H=1024, E=8, k=2, I=256, routing="zipf", n_shared=1),
     [1024, 600, 24]),
]


@pytest.mark.parametrize("name,w,Ts", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_workspace_layer(name, w, Ts):
    require_gpu()
    print(f"noalloc layer: {name} calls T={Ts}", flush=True)
    base = wl.make_inputs(w, seed=12, T=Ts[0])
    if w.routing == "router":
        condition_router_margin(base)
    weights = upload_weights(base)
    for T in Ts:
        inp = wl.make_inputs(w, seed=12, T=T, weights_from=base)
        if w.routing == "router":
            condition_router_margin(inp)
        _same_as_workspace_call(inp, weights)
