"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in the oracle (monkeypatching a function of the
``oracle`` module, so the other oracle functions see it too) and checks that at
least one of the pins in ``test_oracle_pins`` then fails.
"""
import dataclasses

import numpy as np
import pytest

import oracle
from tests import test_oracle_pins as pins

_orig = {name: getattr(oracle, name) for name in oracle.__all__}


def _e2m1_bias0(code):  # exponent bias 0 instead of 1
    return _orig["e2m1_value"](code) * 2.0


def _e4m3_bias8(code):  # the FNUZ exponent bias
    return _orig["e4m3_value"](code) / 2.0


def _unpack_high_first(packed):
    c = _orig["unpack_codes"](packed)
    out = c.copy()
    out[..., 0::2], out[..., 1::2] = c[..., 1::2], c[..., 0::2]
    return out


def _dequant_block32(packed, scales, tscale):  # scales applied per 32 instead of per 16
    codes = oracle.unpack_codes(packed)
    block = np.repeat(oracle.e4m3_value(scales), 32, axis=-1)[..., : codes.shape[-1]]
    return oracle.e2m1_value(codes) * block * float(tscale)


def _dequant_no_tscale(packed, scales, tscale):
    return _orig["dequant"](packed, scales, 1.0)


def _router_drop_last_term(x_bits, wr_bits):
    return oracle.bf16_value(x_bits)[:, :-1] @ oracle.bf16_value(wr_bits)[:, :-1].T


def _route_no_renorm(logits, k):
    idx, _ = _orig["route"](logits, k)
    L = np.asarray(logits, dtype=np.float64)
    p = np.exp(L - L.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    return idx, np.take_along_axis(p, idx.astype(np.int64), 1)


def _route_ties_high(logits, k):
    L = np.asarray(logits, dtype=np.float64)
    idx, w = _orig["route"](L[:, ::-1], k)
    return (L.shape[1] - 1 - idx).astype(np.int32), w


def _permute_unstable(idx, E):
    offsets, perm, inv = _orig["permute"](idx, E)
    perm = perm.copy()
    for e in range(E):
        perm[offsets[e]:offsets[e + 1]] = perm[offsets[e]:offsets[e + 1]][::-1]
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size, dtype=np.int32)
    return offsets, perm, inv


def _swiglu_swapped(x, w13, w2):
    I = w13.shape[0] // 2
    return _orig["swiglu_ffn"](x, np.concatenate([w13[I:], w13[:I]]), w2)


def _hidden_swapped(x, w13):
    I = w13.shape[0] // 2
    return _orig["swiglu_hidden"](x, np.concatenate([w13[I:], w13[:I]]))


def _hidden_no_silu(x, w13):
    I = w13.shape[0] // 2
    return (x @ w13[:I].T) * (x @ w13[I:].T)


def _swiglu_w2_transposed_use(x, w13, w2):
    I = w13.shape[0] // 2
    g = x @ w13[:I].T
    u = x @ w13[I:].T
    a = g / (1.0 + np.exp(-g)) * u
    return a @ w2[:, ::-1].T  # columns of W2 in the wrong order


def _combine_no_residual(y, w, residual_bits, gamma_bits, eps, shared=None):
    return _orig["combine_norm"](y, w, np.zeros_like(residual_bits), gamma_bits, eps, shared)


def _combine_no_gamma(y, w, residual_bits, gamma_bits, eps, shared=None):
    ones = np.full_like(gamma_bits, 0x3F80)
    return _orig["combine_norm"](y, w, residual_bits, ones, eps, shared)


def _combine_shared_dropped(y, w, residual_bits, gamma_bits, eps, shared=None):
    return _orig["combine_norm"](y, w, residual_bits, gamma_bits, eps, None)


def _group_norm_whole_row(x_bits, group, gamma_bits, eps):  # the group ignored
    x = np.asarray(x_bits)
    return _orig["group_rmsnorm"](x_bits, x.shape[1], gamma_bits, eps)


def _group_norm_no_eps(x_bits, group, gamma_bits, eps):
    return _orig["group_rmsnorm"](x_bits, group, gamma_bits, 0.0)


def _group_norm_gamma_per_group(x_bits, group, gamma_bits, eps):  # gamma[h % group]
    g = np.asarray(gamma_bits)
    return _orig["group_rmsnorm"](x_bits, group, np.tile(g[:group], g.shape[0] // group), eps)


def _add_norm_of_x(x_bits, residual_bits, gamma_bits, eps):  # normalises x, not x + residual
    o, _ = _orig["add_rmsnorm"](x_bits, residual_bits, gamma_bits, eps)
    return o, oracle.group_rmsnorm(x_bits, o.shape[1], gamma_bits, eps)


def _add_norm_no_residual(x_bits, residual_bits, gamma_bits, eps):
    return _orig["add_rmsnorm"](x_bits, np.zeros_like(residual_bits), gamma_bits, eps)


def _bf16_truncate(v):
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)
    return np.ldexp(np.trunc(np.ldexp(v, 8 - e)), e - 8)


def _ffn_unrounded(x, w13, w2):
    return oracle.swiglu_hidden(x, w13) @ w2.T


def _no_shared(inp):
    return dataclasses.replace(inp, shared13=None, shared2=None)


def _layer_with_shared(inp, tokens, cache, logits, shared_of):
    """The original layer without its shared expert, then the combine redone with
    shared_of(out, x) as the shared term."""
    out = _orig["layer"](_no_shared(inp), tokens, cache, logits)
    if inp.shared13 is None:
        return out
    tok = out["tokens"]
    W13 = oracle.dequant(inp.shared13.packed[0], inp.shared13.scales[0], inp.shared13.tscale[0])
    W2 = oracle.dequant(inp.shared2.packed[0], inp.shared2.scales[0], inp.shared2.tscale[0])
    s = shared_of(out, oracle.bf16_value(np.asarray(inp.x)[tok]), W13, W2)
    out["o"], out["n"] = oracle.combine_norm(out["y"], out["w"], np.asarray(inp.residual)[tok], inp.gamma,
                                             inp.w.eps, s)
    return out


def _layer_shared_dropped(inp, tokens=None, cache=None, logits=None):
    return _orig["layer"](_no_shared(inp), tokens, cache, logits)


def _layer_shared_gated(inp, tokens=None, cache=None, logits=None):  # scaled by w_0
    return _layer_with_shared(inp, tokens, cache, logits,
                              lambda out, x, W13, W2: out["w"][:, :1] * oracle.swiglu_ffn(x, W13, W2))


def _layer_shared_wrong_rows(inp, tokens=None, cache=None, logits=None):  # rows reversed
    return _layer_with_shared(inp, tokens, cache, logits,
                              lambda out, x, W13, W2: oracle.swiglu_ffn(x[::-1], W13, W2))


def _layer_shared_up_as_gate(inp, tokens=None, cache=None, logits=None):  # halves swapped
    def f(out, x, W13, W2):
        I = W13.shape[0] // 2
        return _orig["swiglu_ffn"](x, np.concatenate([W13[I:], W13[:I]]), W2)
    return _layer_with_shared(inp, tokens, cache, logits, f)


def _e4m3_truncate(v):  # rounds toward zero
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, e = np.frexp(a)
    e = np.maximum(e - 1, -6)
    return np.copysign(np.minimum(np.ldexp(np.trunc(np.ldexp(a, 3 - e)), e - 3), 448.0), v)


def _e4m3_no_saturation(v):  # overflow rounds on past 448
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, e = np.frexp(a)
    e = np.maximum(e - 1, -6)
    return np.copysign(np.ldexp(np.rint(np.ldexp(a, 3 - e)), e - 3), v)


def _e4m3_fnuz_subnormals(v):  # subnormal range starting one binade lower
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, e = np.frexp(a)
    e = np.maximum(e - 1, -7)
    return np.copysign(np.minimum(np.ldexp(np.rint(np.ldexp(a, 3 - e)), e - 3), 448.0), v)


def _mx_scale_saturating(x, block=32):  # e = E - 8 always: large blocks saturate
    x = np.asarray(x, dtype=np.float64)
    xb = x.reshape(x.shape[:-1] + (x.shape[-1] // block, block))
    amax = np.max(np.abs(xb), axis=-1)
    _, E = np.frexp(amax)
    e = np.where(amax == 0, 0, E - 1 - 8).astype(np.int64)
    return oracle.e4m3_round(np.ldexp(xb, -e[..., None])).reshape(x.shape), e


def _mx_block16(x, block=32):
    q, e = _orig["mxfp8_quantize"](x, 16)
    return q, e[..., ::2]


def _dequant_e4m3_unrounded(packed, scales):
    return oracle.dequant(packed, scales, 1.0)


def _hidden_w4a8_unquantized(x, w13_8, tscale):
    I = w13_8.shape[0] // 2
    g = float(tscale) * (np.asarray(x) @ w13_8[:I].T)
    u = float(tscale) * (np.asarray(x) @ w13_8[I:].T)
    return g / (1.0 + np.exp(-g)) * u


def _hidden_w4a8_no_tscale(x, w13_8, tscale):
    return _orig["swiglu_hidden_w4a8"](x, w13_8, 1.0)


def _ffn_w4a8_h_unquantized(x, w13_8, ts13, w2_8, ts2):
    h = oracle.bf16_round(oracle.swiglu_hidden_w4a8(x, w13_8, ts13))
    return oracle.bf16_round(float(ts2) * (h @ w2_8.T))


def _ffn_w4a8_no_ts2(x, w13_8, ts13, w2_8, ts2):
    return _orig["swiglu_ffn_w4a8"](x, w13_8, ts13, w2_8, 1.0)


def _layer_w4a8_as_w4a16(inp, tokens=None, logits=None):  # the FP8 steps left out
    return _orig["layer"](inp, tokens=tokens, logits=logits)


def _layer_w4a8_shared_dropped(inp, tokens=None, logits=None):
    return _orig["layer_w4a8"](_no_shared(inp), tokens, logits)


MUTANTS = {
    "bf16_round": [_bf16_truncate],
    "e2m1_value": [_e2m1_bias0],
    "e4m3_value": [_e4m3_bias8],
    "unpack_codes": [_unpack_high_first],
    "dequant": [_dequant_block32, _dequant_no_tscale],
    "router_logits": [_router_drop_last_term],
    "route": [_route_no_renorm, _route_ties_high],
    "permute": [_permute_unstable],
    "swiglu_hidden": [_hidden_swapped, _hidden_no_silu],
    "swiglu_ffn": [_swiglu_swapped, _swiglu_w2_transposed_use, _ffn_unrounded],
    "combine_norm": [_combine_no_residual, _combine_no_gamma, _combine_shared_dropped],
    "group_rmsnorm": [_group_norm_whole_row, _group_norm_no_eps, _group_norm_gamma_per_group],
    "add_rmsnorm": [_add_norm_of_x, _add_norm_no_residual],
    "layer": [_layer_shared_dropped, _layer_shared_gated, _layer_shared_wrong_rows, _layer_shared_up_as_gate],
    "e4m3_round": [_e4m3_truncate, _e4m3_no_saturation, _e4m3_fnuz_subnormals],
    "mxfp8_quantize": [_mx_scale_saturating, _mx_block16],
    "dequant_e4m3": [_dequant_e4m3_unrounded],
    "swiglu_hidden_w4a8": [_hidden_w4a8_unquantized, _hidden_w4a8_no_tscale],
    "swiglu_ffn_w4a8": [_ffn_w4a8_h_unquantized, _ffn_w4a8_no_ts2],
    "layer_w4a8": [_layer_w4a8_as_w4a16, _layer_w4a8_shared_dropped],
}

CASES = [(name, fn) for name, fns in MUTANTS.items() for fn in fns]


def _all_pins():
    out = []
    for name in dir(pins):
        if not name.startswith("test_"):
            continue
        fn = getattr(pins, name)
        marks = getattr(fn, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        if params:
            argnames, values = params[0].args[0], params[0].args[1]
            argnames = [a.strip() for a in argnames.split(",")]
            for v in values:
                v = v if isinstance(v, tuple) else (v,)
                out.append((name, fn, dict(zip(argnames, v))))
        else:
            out.append((name, fn, {}))
    return out


@pytest.mark.parametrize("target,mutant", CASES, ids=[f"{n}:{f.__name__}" for n, f in CASES])
def test_pins_catch_planted_mistake(target, mutant, monkeypatch):
    monkeypatch.setattr(oracle, target, mutant)
    caught = []
    # a planted mistake may divide by zero or overflow on a pin's edge case; numpy's
    # warning about it is expected here, the pins' verdict is what counts
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        for name, fn, kwargs in _all_pins():
            try:
                fn(**kwargs)
            except (AssertionError, ValueError, IndexError):
                caught.append(name)
    assert caught, f"no pin fails with {target} replaced by {mutant.__name__}"


def test_pins_pass_without_mutation():
    failed = []
    for name, fn, kwargs in _all_pins():
        try:
            fn(**kwargs)
        except AssertionError:
            failed.append(name)
    assert not failed
