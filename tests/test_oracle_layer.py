"""Pins of the oracle's expert FFN and whole-layer forward."""
import numpy as np
import pytest

import oracle
from oracle import expert_ffn, forward
from synth import MoeConfig, generate_layer, to_numpy_inputs
from synth.configs import CONFIGS
from tests.bruteforce import layer_bruteforce


def test_swiglu_closed_form():
    """h = silu(gate) * up with sigmoid(ln 3) = 3/4: gate and up cannot be swapped."""
    ln3 = np.log(3.0)
    X = np.array([[1.0, 0.0, 0.0]], np.float32)
    wg = np.array([[ln3, 0, 0], [0, 0, 0], [-ln3, 0, 0]], np.float32)
    wu = np.array([[2.0, 0, 0], [5.0, 0, 0], [4.0, 0, 0]], np.float32)
    wd = np.eye(3, dtype=np.float32)
    y = expert_ffn(X, wg, wu, wd)
    exp = np.array([[2 * 0.75 * ln3, 0.0, 4 * (-0.25) * ln3]])
    assert np.allclose(y, exp, rtol=2e-7, atol=1e-7)
    # a down projection that is not the identity is applied as h @ Wd^T
    wd2 = np.array([[1, 2, 0], [0, 0, 3], [1, 0, 0]], np.float32)
    assert np.allclose(expert_ffn(X, wg, wu, wd2), exp @ wd2.T, rtol=1e-6)


def test_silu_extremes_are_finite():
    X = np.array([[1.0]], np.float32)
    for g, want in ((-200.0, 0.0), (200.0, 200.0), (0.0, 0.0)):
        y = expert_ffn(X, np.array([[g]], np.float32), np.ones((1, 1), np.float32),
                       np.ones((1, 1), np.float32))
        assert np.isfinite(y).all() and abs(float(y[0, 0]) - want) <= 1e-4 * max(1.0, abs(want))


def _rel_inf(out, ref):
    num = np.abs(out - ref).max(axis=1)
    den = np.abs(ref).max(axis=1)
    return float((num / np.maximum(den, 1e-30)).max())


def _check_against_bruteforce(cfg, rtol):
    li = generate_layer(cfg, "cpu")
    inp = to_numpy_inputs(li)
    res = forward(inp)
    ref, ref_idx, ref_logits, gap = layer_bruteforce(inp)
    ok = gap > 1e-5                                   # exclude float64-vs-fp32 near-ties
    assert np.array_equal(res.topk_idx[ok], ref_idx[ok])
    assert _rel_inf(res.out[ok], ref[ok]) <= rtol
    assert np.allclose(res.logits, ref_logits, rtol=0, atol=1e-4)


def test_tiny_config_vs_bruteforce():
    _check_against_bruteforce(CONFIGS[0], 1e-4)


@pytest.mark.parametrize("case", range(12))
def test_random_micro_shapes_vs_bruteforce(case):
    rng = np.random.default_rng(1000 + case)
    E = int(rng.integers(1, 13))
    fp8 = bool(case % 3 == 2)
    cfg = MoeConfig(f"micro{case}", 100 + case, T=int(rng.integers(1, 41)),
                    H=int(rng.choice([128, 256])), E=E, k=int(rng.integers(1, min(E, 4) + 1)),
                    I=int(rng.choice([128, 256])), n_shared=int(case % 2),
                    wdtype="fp8" if fp8 else "bf16",
                    zipf_s=1.1 if case % 4 == 1 else None)
    # fp8: the oracle quantises h from fp32 sums, the brute force from float64 sums,
    # so an element may land on the neighbouring code (one e4m3 step, 2^-3 relative).
    _check_against_bruteforce(cfg, 2e-2 if fp8 else 1e-4)


def test_identical_experts_make_routing_irrelevant():
    cfg = MoeConfig("same", 7, T=24, H=128, E=6, k=3, I=128, zipf_s=1.1)
    inp = to_numpy_inputs(generate_layer(cfg))
    for key in ("w_gate", "w_up", "w_down"):
        inp[key] = np.ascontiguousarray(np.broadcast_to(inp[key][0], inp[key].shape))
    res = forward(inp)
    x = oracle.bf16_bits_to_f32(inp["x_bf16"])
    dense = expert_ffn(x, *oracle.expert_weights_f32(inp, 0))
    assert _rel_inf(res.out, dense) <= 1e-5


def test_single_expert_is_dense_mlp():
    cfg = MoeConfig("dense", 8, T=10, H=256, E=1, k=1, I=128)
    inp = to_numpy_inputs(generate_layer(cfg))
    res = forward(inp)
    assert np.all(res.topk_idx == 0) and np.all(res.topk_w == 1.0)
    assert res.offsets.tolist() == [0, 10] and res.src_row.tolist() == list(range(10))
    x = oracle.bf16_bits_to_f32(inp["x_bf16"])
    assert np.array_equal(res.out, expert_ffn(x, *oracle.expert_weights_f32(inp, 0)))


def test_logits_override_routes_from_given_logits():
    inp = to_numpy_inputs(generate_layer(CONFIGS[0]))
    T, E = inp["x_bf16"].shape[0], inp["w_router"].shape[0]
    forced = np.zeros((T, E), np.float32)
    forced[:, 5] = 1.0
    forced[:, 2] = 0.5
    res = forward(inp, logits_override=forced)
    assert np.all(res.topk_idx == np.array([5, 2])) and res.counts.tolist() == [0, 0, T, 0, 0, T, 0, 0]


@pytest.mark.parametrize("ci", [0, 3])
def test_forward_tokens_matches_full_forward(ci):
    """The per-token evaluation equals the permuted evaluation on every token."""
    from synth.configs import MoeConfig as C
    base = CONFIGS[ci]
    cfg = C(base.name + "_small", base.seed, T=48, H=256, E=min(base.E, 64), k=min(base.k, 6),
            I=256, n_shared=base.n_shared, wdtype=base.wdtype, zipf_s=base.zipf_s)
    inp = to_numpy_inputs(generate_layer(cfg))
    full = forward(inp)
    toks = np.array([0, 5, 17, 47, 3])
    part = oracle.forward_tokens(inp, toks)
    assert np.array_equal(part.topk_idx, full.topk_idx[toks])
    assert _rel_inf(part.out, full.out[toks]) <= 1e-5


def test_forward_tokens_fp8_shared_vs_bruteforce():
    cfg = MoeConfig("fp8s", 11, T=20, H=256, E=9, k=3, I=256, n_shared=1, wdtype="fp8")
    inp = to_numpy_inputs(generate_layer(cfg))
    ref, ref_idx, _, gap = layer_bruteforce(inp)
    toks = np.arange(20)
    part = oracle.forward_tokens(inp, toks)
    ok = gap > 1e-5
    assert np.array_equal(part.topk_idx[ok], ref_idx[ok])
    assert _rel_inf(part.out[ok], ref[ok]) <= 2e-2


@pytest.mark.parametrize("case", range(6))
def test_mxfp8_micro_shapes_vs_bruteforce(case):
    """MXFP8 layers (weights, x and h in MX blocks of 32) against the float64
    brute force, whose MX codec is torch.frexp + torch's e4m3fn cast."""
    rng = np.random.default_rng(2000 + case)
    E = int(rng.integers(1, 10))
    cfg = MoeConfig(f"mx{case}", 200 + case, T=int(rng.integers(1, 33)),
                    H=int(rng.choice([128, 256])), E=E, k=int(rng.integers(1, min(E, 4) + 1)),
                    I=int(rng.choice([128, 256])), n_shared=int(case % 2), wdtype="mxfp8",
                    zipf_s=1.1 if case % 3 == 1 else None)
    # as for fp8: h quantised from fp32 vs float64 sums may differ by one code
    _check_against_bruteforce(cfg, 2e-2)


def test_mxfp8_forward_tokens_matches_full_forward():
    cfg = MoeConfig("mxs", 12, T=24, H=256, E=6, k=2, I=128, n_shared=1, wdtype="mxfp8")
    inp = to_numpy_inputs(generate_layer(cfg))
    full = forward(inp)
    toks = np.array([0, 5, 23, 11])
    part = oracle.forward_tokens(inp, toks)
    assert np.array_equal(part.topk_idx, full.topk_idx[toks])
    assert _rel_inf(part.out, full.out[toks]) <= 1e-5
