"""GPU parity of every C-ABI entry point against the CPU oracle (MI355X).

Bars: routing (top-k indices, counts, offsets, dest, src_row, permuted rows and
fp8 / mxfp8 codes and scales) bit-exact given the same fp32 logits; weights
within 1e-6 of a float64 evaluation; combine bit-exact given the same y_perm;
layer output within a per-token infinity-norm relative error of 2e-2 (bf16) /
5e-2 (fp8, mxfp8).
"""
import numpy as np
import pytest
import torch

import expert_ffn_layer_gemm_amd as moe
import oracle
from synth import CONFIGS, EXTRA_CONFIGS, MoeConfig, generate_layer, to_numpy_inputs
from tests.gpu_helpers import (DEV, bf16_bits_np, bf16_np, layer, rel_inf, run_ffn, run_forward,
                               run_permute, run_route, to_bf16_rne)

pytestmark = pytest.mark.gpu
TOL = {"bf16": 2e-2, "fp8": 5e-2, "mxfp8": 5e-2}


def _route_inputs(li):
    return dict(x_bf16=bf16_bits_np(li.x), w_router=li.w_router.cpu().numpy(),
                router_bias=None if li.router_bias is None else li.router_bias.cpu().numpy())


# ------------------------------------------------------------------ top-k ----
def _crafted_logits(rng, T, E):
    one = np.float32(1.0)
    up = np.nextafter(one, np.float32(2))
    kinds = [
        lambda: rng.standard_normal(E).astype(np.float32),
        lambda: np.array([-1.0, -0.0, 0.0, 0.5, 1.0], np.float32)[rng.integers(0, 5, E)],
        lambda: np.where(rng.random(E) < 0.5, one, up).astype(np.float32),
        lambda: np.zeros(E, np.float32) * np.where(rng.random(E) < 0.5, -1, 1).astype(np.float32),
        lambda: (rng.standard_normal(E) * 1e4).astype(np.float32),
    ]
    return np.stack([kinds[t % len(kinds)]() for t in range(T)])


@pytest.mark.parametrize("E,k", [(8, 2), (37, 5), (128, 8), (512, 10), (1024, 16), (16, 16), (1, 1)])
def test_topk_from_logits_bitexact(E, k):
    rng = np.random.default_rng(E * 31 + k)
    T = 203
    lg = _crafted_logits(rng, T, E)
    idx_ref, w_ref = oracle.topk_softmax(lg, k)
    sh = moe.make_shape(T, 128, E, k, 128)
    logits = torch.from_numpy(lg).to(DEV)
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    moe.moe_route_from_logits(sh, logits, idx, w)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    sel = np.take_along_axis(lg.astype(np.float64), idx_ref.astype(np.int64), 1)
    p = np.exp(sel - sel[:, :1])
    p /= p.sum(1, keepdims=True)
    assert np.abs(w.cpu().numpy() - p).max() <= 1e-6
    assert np.abs(w.cpu().numpy() - w_ref).max() <= 1e-6


# ----------------------------------------------------------------- router ----
@pytest.mark.parametrize("ci", range(len(CONFIGS)))
def test_route_configs(ci):
    cfg = CONFIGS[ci]
    li = layer(cfg)
    logits, idx, w = run_route(cfg, li)
    inp = _route_inputs(li)
    x = oracle.bf16_bits_to_f32(inp["x_bf16"])
    ref = oracle.router_logits(x, inp["w_router"], inp["router_bias"])
    lg = logits.cpu().numpy()
    # fp32 dot-product error bound (Higham): |err| <= H u sum|x_h w_h|, u = 2^-24
    mag = np.abs(x) @ np.abs(inp["w_router"]).T
    if inp["router_bias"] is not None:
        mag = mag + np.abs(inp["router_bias"])[None, :]
    bound = (cfg.H + 2) * 2.0 ** -24 * mag
    assert np.all(np.abs(lg - ref) <= bound)
    delta = float(np.abs(lg - ref).max())
    print(f"{cfg.name}: max |logit_gpu - logit_oracle| = {delta:.3e}")
    # routing bit-exact on the GPU's own logits
    idx_ref, w_ref = oracle.topk_softmax(lg, cfg.k)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    assert np.abs(w.cpu().numpy() - w_ref).max() <= 1e-6


# Shapes that exercise the router GEMM's edges: token and expert tiles cut
# short (T, E not multiples of 128), H split into slices of unequal length,
# one slice (partial sums written in place, bias added there), T = E = 1, and
# E > 512 for the top-k.
@pytest.mark.parametrize("T,H,E,k,zipf", [(300, 384, 200, 6, 1.1), (1000, 1280, 256, 8, None),
                                          (130, 1152, 130, 4, 1.1), (32768, 128, 128, 2, 1.1),
                                          (1, 256, 1, 1, None), (5, 128, 1000, 16, 1.1)])
def test_route_ragged_shapes(T, H, E, k, zipf):
    cfg = MoeConfig(f"route_{T}_{H}_{E}", 11, T=T, H=H, E=E, k=k, I=128, zipf_s=zipf)
    li = generate_layer(cfg, DEV)
    logits, idx, w = run_route(cfg, li)
    inp = _route_inputs(li)
    x = oracle.bf16_bits_to_f32(inp["x_bf16"])
    ref = oracle.router_logits(x, inp["w_router"], inp["router_bias"])
    mag = np.abs(x) @ np.abs(inp["w_router"]).T
    if inp["router_bias"] is not None:
        mag = mag + np.abs(inp["router_bias"])[None, :]
    lg = logits.cpu().numpy()
    assert np.all(np.abs(lg - ref) <= (cfg.H + 2) * 2.0 ** -24 * mag)
    idx_ref, w_ref = oracle.topk_softmax(lg, cfg.k)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    assert np.abs(w.cpu().numpy() - w_ref).max() <= 1e-6


def test_route_max_hidden():
    # H at the supported maximum: the router splits it into hundreds of slices.
    cfg = MoeConfig("route_hmax", 12, T=3, H=131072, E=16, k=2, I=128)
    li = generate_layer(cfg, DEV)
    logits, idx, w = run_route(cfg, li)
    inp = _route_inputs(li)
    x = oracle.bf16_bits_to_f32(inp["x_bf16"])
    ref = oracle.router_logits(x, inp["w_router"], None)
    mag = np.abs(x) @ np.abs(inp["w_router"]).T
    lg = logits.cpu().numpy()
    assert np.all(np.abs(lg - ref) <= (cfg.H + 2) * 2.0 ** -24 * mag)
    idx_ref, w_ref = oracle.topk_softmax(lg, cfg.k)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)


def test_route_zero_router_weight_ties():
    cfg = MoeConfig("zero_router", 5, T=70, H=512, E=24, k=6, I=128)
    li = generate_layer(cfg, DEV)
    li.w_router.zero_()
    logits, idx, w = run_route(cfg, li)
    assert np.all(idx.cpu().numpy() == np.arange(6)[None, :])
    assert np.all(w.cpu().numpy() == np.float32(1.0) / np.float32(6.0))


# ---------------------------------------------------------------- permute ----
def _check_permute(cfg, li, idx):
    counts, offsets, dest, src, x_perm, x_scale = run_permute(cfg, idx, li.x)
    c_ref, o_ref, d_ref, s_ref = oracle.counting_sort(idx.cpu().numpy(), cfg.E, cfg.n_shared,
                                                      cfg.e_first, cfg.e_local)
    R = int(o_ref[-1])                   # rows of the share (R = T*(k + n_shared) for the layer)
    assert np.array_equal(counts.cpu().numpy(), c_ref)
    assert np.array_equal(offsets.cpu().numpy(), o_ref)
    assert np.array_equal(dest.cpu().numpy(), d_ref)
    assert np.array_equal(src.cpu().numpy()[:R], s_ref)
    xb = bf16_bits_np(li.x)
    if cfg.wdtype == "fp8":
        codes, scales = oracle.quantize_groups_128(oracle.bf16_bits_to_f32(xb))
        assert np.array_equal(x_perm.cpu().numpy()[:R], codes[s_ref])
        assert np.array_equal(x_scale.cpu().numpy()[:, :R].T, scales[s_ref])   # [H/128, R] layout
    elif cfg.wdtype == "mxfp8":
        codes, e8 = oracle.mx_quantize_rows(oracle.bf16_bits_to_f32(xb))
        assert np.array_equal(x_perm.cpu().numpy()[:R], codes[s_ref])
        assert np.array_equal(x_scale.cpu().numpy()[:R], e8[s_ref])
    else:
        assert np.array_equal(bf16_bits_np(x_perm)[:R], xb[s_ref])


@pytest.mark.parametrize("ci", range(len(CONFIGS)))
def test_permute_configs(ci):
    cfg = CONFIGS[ci]
    li = layer(cfg)
    _, idx, _ = run_route(cfg, li)
    _check_permute(cfg, li, idx)


@pytest.mark.parametrize("T,E,k,ns,wdtype", [(1, 1, 1, 0, "bf16"), (257, 7, 3, 1, "fp8"),
                                             (600, 1024, 16, 0, "bf16"), (513, 5, 5, 1, "bf16"),
                                             (300, 9, 2, 1, "mxfp8")])
def test_permute_ragged_shapes(T, E, k, ns, wdtype):
    cfg = MoeConfig("perm", 9, T=T, H=256, E=E, k=k, I=128, n_shared=ns, wdtype=wdtype)
    rng = np.random.default_rng(T + E)
    p = 1.0 / np.arange(1, E + 1) ** 1.2
    p /= p.sum()
    idx = np.stack([rng.choice(E, k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    li = generate_layer(cfg, DEV)
    _check_permute(cfg, li, torch.from_numpy(idx).to(DEV))


# Expert-parallel shares: only the pairs routed to experts [e_first,
# e_first + e_local) get rows; the rest get dest = -1.
@pytest.mark.parametrize("T,E,k,ns,ef,el,wdtype", [(300, 16, 4, 1, 4, 5, "bf16"), (600, 64, 8, 0, 60, 4, "fp8"),
                                                   (257, 9, 3, 1, 0, 1, "mxfp8"), (1000, 128, 8, 0, 16, 16, "bf16")])
def test_permute_share(T, E, k, ns, ef, el, wdtype):
    cfg = MoeConfig("perm_share", 10, T=T, H=256, E=E, k=k, I=128, n_shared=ns, wdtype=wdtype,
                    e_first=ef, e_local=el)
    rng = np.random.default_rng(T + E + ef)
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    li = generate_layer(cfg, DEV)
    _check_permute(cfg, li, torch.from_numpy(idx).to(DEV))


# ------------------------------------------------------------- grouped FFN ----
def _ffn_case(cfg, sizes, seed):
    """Random x_perm with crafted group sizes; returns GPU y_perm and oracle y_perm (fp32)."""
    li = generate_layer(cfg, DEV)
    rng = np.random.default_rng(seed)
    G = cfg.n_groups
    assert len(sizes) == G
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    R = int(offsets[-1])
    xr = rng.standard_normal((R, cfg.H)).astype(np.float32)
    inp = to_numpy_inputs(li)
    if cfg.wdtype == "fp8":
        codes, scales = oracle.quantize_groups_128(xr)
        x_perm = torch.from_numpy(codes).to(DEV)
        # the library takes fp8 activation scales K-block-major, [H/128, T*(k+n_shared)]
        xs = np.zeros((cfg.H // 128, cfg.R), dtype=np.float32)
        xs[:, :R] = scales.T
        x_scale = torch.from_numpy(xs).to(DEV)
        xo = oracle.fp8_e4m3.dequantize_groups_128(codes, scales)
    elif cfg.wdtype == "mxfp8":
        codes, e8 = oracle.mx_quantize_rows(xr)
        x_perm = torch.from_numpy(codes).to(DEV)
        x_scale = torch.from_numpy(e8).to(DEV)
        xo = oracle.mx_dequantize_rows(codes, e8)
    else:
        xt = torch.from_numpy(xr).to(torch.bfloat16)
        x_perm, x_scale = xt.to(DEV), None
        xo = xt.float().numpy()
    sh = moe.make_shape(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.n_shared, cfg.wdtype)
    assert R <= cfg.R
    ws = torch.empty(moe.moe_ffn_workspace_bytes(sh), dtype=torch.uint8, device=DEV)
    y = torch.zeros((cfg.R, cfg.H), dtype=torch.bfloat16, device=DEV)
    moe.moe_grouped_ffn(sh, torch.from_numpy(offsets).to(DEV), x_perm, x_scale, li.w_gate, li.w_up,
                        li.w_down, li.s_gate, li.s_up, li.s_down, y, ws)
    torch.cuda.synchronize()
    ref = oracle.grouped_ffn(xo, offsets, inp)
    return bf16_np(y)[:R], ref


@pytest.mark.parametrize("wdtype", ["bf16", "fp8", "mxfp8"])
def test_grouped_ffn_group_size_boundaries(wdtype):
    # sizes straddle the 16-row slices, the split between the streaming and
    # the tiled kernels (48 rows at this batch size) and the 128-row tiles
    sizes = [0, 1, 15, 16, 17, 31, 32, 33, 47, 48, 49, 63, 64, 65, 127, 128, 129, 0, 200, 257, 3]
    E = len(sizes)
    cfg = MoeConfig("ffn_" + wdtype, 21, T=sum(sizes), H=384, E=E, k=1, I=256, wdtype=wdtype)
    y, ref = _ffn_case(cfg, sizes, 1)
    err = rel_inf(y, ref)
    print(f"grouped ffn {wdtype}: per-row rel err {err:.3e}")
    assert err <= TOL[wdtype]


@pytest.mark.parametrize("wdtype", ["fp8", "mxfp8"])
def test_grouped_ffn_8bit_shared_group(wdtype):
    sizes = [5, 0, 66, 9, 40]        # routed rows sum to T*k = 80; group 4 = shared expert (T rows)
    cfg = MoeConfig("ffn_shared_" + wdtype, 22, T=40, H=256, E=4, k=2, I=384, n_shared=1,
                    wdtype=wdtype)
    y, ref = _ffn_case(cfg, sizes, 2)
    assert rel_inf(y, ref) <= TOL[wdtype]


# A K extent of 4096 (gate/up) and 1536 (down) walks many MX scale dwords per
# row; group sizes cover the streaming kernels and ragged 128-row tiles.
def test_grouped_ffn_mxfp8_deep_k():
    sizes = [3, 64, 65, 300, 16, 0]
    cfg = MoeConfig("ffn_mx_deep", 24, T=sum(sizes), H=4096, E=len(sizes), k=1, I=1536,
                    wdtype="mxfp8")
    y, ref = _ffn_case(cfg, sizes, 3)
    err = rel_inf(y, ref)
    print(f"grouped ffn mxfp8 H=4096: per-row rel err {err:.3e}")
    assert err <= TOL["mxfp8"]


# ----------------------------------------------------------------- combine ----
@pytest.mark.parametrize("T,H,k,ns", [(64, 4096, 8, 0), (33, 256, 2, 1), (1, 128, 1, 0), (700, 7168, 8, 1)])
def test_combine_bitexact(T, H, k, ns):
    rng = np.random.default_rng(T * 7 + k)
    R = T * (k + ns)
    y = torch.randn((R, H), generator=torch.Generator().manual_seed(T), dtype=torch.float32).to(torch.bfloat16)
    perm = rng.permutation(T * k).astype(np.int32)
    dest = perm.reshape(T, k)
    w = rng.random((T, k)).astype(np.float32)
    w /= w.sum(1, keepdims=True)
    E = max(k, 2)
    sh = moe.make_shape(T, H, E, k, 128, ns)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    offsets = np.zeros(E + ns + 1, np.int32)     # only offsets[E] (start of the shared rows) is read
    offsets[E:] = T * k
    moe.moe_combine(sh, y.to(DEV), torch.from_numpy(dest).to(DEV), torch.from_numpy(w).to(DEV),
                    torch.from_numpy(offsets).to(DEV) if ns else None, out)
    torch.cuda.synchronize()
    ref = oracle.combine(y.float().numpy(), dest, w, ns)
    assert np.array_equal(bf16_np(out), to_bf16_rne(ref))


# An expert-parallel share: pairs of other shares' experts (dest = -1) add
# nothing, and the shared rows start at offsets[L], below T*k.
@pytest.mark.parametrize("ns", [0, 1])
def test_combine_share_bitexact(ns):
    rng = np.random.default_rng(77 + ns)
    T, H, k, E, L = 90, 512, 4, 16, 5
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    counts, offsets, dest, src = oracle.counting_sort(idx, E, ns, 3, L)
    R = int(offsets[-1])
    y = torch.randn((R, H), generator=torch.Generator().manual_seed(5), dtype=torch.float32).to(torch.bfloat16)
    w = rng.random((T, k)).astype(np.float32)
    sh = moe.make_shape(T, H, E, k, 128, ns, "bf16", 3, L)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    moe.moe_combine(sh, y.to(DEV), torch.from_numpy(dest).to(DEV), torch.from_numpy(w).to(DEV),
                    torch.from_numpy(offsets).to(DEV), out)
    torch.cuda.synchronize()
    ref = oracle.combine(y.float().numpy(), dest, w, ns, shared_base=offsets[L])
    assert (dest < 0).any()
    assert np.array_equal(bf16_np(out), to_bf16_rne(ref))


# ------------------------------------------------------------- end to end ----
def _forward_check(cfg, li, sample=None):
    out, idx, w = run_forward(cfg, li)
    logits, idx2, _ = run_route(cfg, li)
    assert np.array_equal(idx.cpu().numpy(), idx2.cpu().numpy())
    lg = logits.cpu().numpy()
    inp = to_numpy_inputs(li)
    gpu_out = bf16_np(out)
    print(f"{cfg.name}: GPU layer done, oracle on the host", flush=True)
    if sample is None:
        ref = oracle.forward(inp, logits_override=lg)
        assert np.array_equal(idx.cpu().numpy(), ref.topk_idx)
        err = rel_inf(gpu_out, ref.out)
    else:
        ref = oracle.forward_tokens(inp, sample, logits_override=lg[sample])
        assert np.array_equal(idx.cpu().numpy()[sample], ref.topk_idx)
        err = rel_inf(gpu_out[sample], ref.out)
    # routing of the oracle's own logits: report near-tie flips (not a failure)
    own = oracle.topk_softmax(oracle.router_logits(oracle.bf16_bits_to_f32(inp["x_bf16"]),
                                                   inp["w_router"], inp["router_bias"]), cfg.k)[0]
    flips = int((own != idx.cpu().numpy()).any(axis=1).sum())
    n_tok = cfg.T if sample is None else len(sample)
    print(f"{cfg.name}: per-token rel err {err:.3e} over {n_tok} tokens, "
          f"routing flips vs oracle logits: {flips}")
    assert err <= TOL[cfg.wdtype]
    assert flips <= max(2, cfg.T // 500)
    return out


# Every token of every workload at full size against the whole-layer oracle
# (8192 prefill tokens, 4096 DeepSeek-like tokens through the fp8 tiled
# kernels at K = 7168, the shared expert's 4096-row group included).
@pytest.mark.parametrize("ci", range(len(CONFIGS)))
def test_forward_configs_full(ci):
    cfg = CONFIGS[ci]
    _forward_check(cfg, layer(cfg))


# MXFP8 layers at the Qwen3-235B shape, decode and prefill, every token.
@pytest.mark.parametrize("name", [c.name for c in EXTRA_CONFIGS if c.wdtype == "mxfp8"])
def test_forward_mxfp8_configs(name):
    cfg = next(c for c in EXTRA_CONFIGS if c.name == name)
    _forward_check(cfg, layer(cfg))


@pytest.mark.parametrize("ci", range(len(CONFIGS)))
def test_forward_deterministic(ci):
    cfg = CONFIGS[ci]
    li = layer(cfg)
    a, ia, wa = run_forward(cfg, li)
    b, ib, wb = run_forward(cfg, li)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(ia, ib) and torch.equal(wa, wb)


# T <= 256 with E <= 256 runs routing and dispatch in one workgroup; the
# T256/T257 pair straddles that boundary.
@pytest.mark.parametrize("case", ["T1", "T3_ragged", "E1k1", "kE", "one_hot_expert", "fp8_small",
                                  "T256_E256", "T257", "k16", "mx_small", "mx_hot", "hot_ragged_n",
                                  "fp8_hot_ragged_n", "fp8_k512", "fp8_k512_ragged_n"])
def test_forward_edge_cases(case):
    cfgs = {
        "T1": MoeConfig("T1", 30, T=1, H=256, E=8, k=2, I=256),
        "T3_ragged": MoeConfig("T3", 31, T=3, H=384, E=16, k=4, I=128, n_shared=1),
        "E1k1": MoeConfig("E1", 32, T=40, H=256, E=1, k=1, I=256),
        "kE": MoeConfig("kE", 33, T=50, H=256, E=6, k=6, I=256),
        "one_hot_expert": MoeConfig("hot", 34, T=300, H=256, E=8, k=1, I=384),
        "fp8_small": MoeConfig("f8", 35, T=77, H=512, E=12, k=3, I=256, n_shared=1, wdtype="fp8"),
        "T256_E256": MoeConfig("t256", 36, T=256, H=256, E=256, k=8, I=128, n_shared=1, zipf_s=1.1),
        "T257": MoeConfig("t257", 37, T=257, H=256, E=256, k=8, I=128, n_shared=1, zipf_s=1.1),
        "k16": MoeConfig("k16", 38, T=100, H=256, E=64, k=16, I=128),
        "mx_small": MoeConfig("mx", 39, T=77, H=512, E=12, k=3, I=256, n_shared=1, wdtype="mxfp8"),
        "mx_hot": MoeConfig("mxhot", 40, T=300, H=384, E=8, k=1, I=384, wdtype="mxfp8"),
        # one 600-row group through the tiled kernels with H = 384: the down
        # GEMM's second column tile holds 128 of its 256 columns
        "hot_ragged_n": MoeConfig("hotrn", 41, T=600, H=384, E=8, k=1, I=256),
        "fp8_hot_ragged_n": MoeConfig("f8hotrn", 42, T=600, H=384, E=8, k=1, I=256, wdtype="fp8"),
        # ~150-row groups split into two 128-row tiles, a 600-row shared
        # expert, K a multiple of 512 in both GEMMs; then H = 640, whose down
        # GEMM has a 128-column last tile.
        "fp8_k512": MoeConfig("f8k512", 43, T=600, H=1024, E=8, k=2, I=512, n_shared=1, wdtype="fp8"),
        "fp8_k512_ragged_n": MoeConfig("f8k512rn", 44, T=600, H=640, E=8, k=2, I=512, n_shared=1,
                                       wdtype="fp8"),
    }
    cfg = cfgs[case]
    li = generate_layer(cfg, DEV)
    if case in ("one_hot_expert", "mx_hot", "hot_ragged_n", "fp8_hot_ragged_n"):
        li.router_bias = torch.zeros(cfg.E, dtype=torch.float32, device=DEV)
        li.router_bias[3] = 100.0          # every token -> expert 3: 300 rows, ragged tiles
    _forward_check(cfg, li)


# Layers whose mean group is large run the streaming kernels with a capped
# grid whose workgroups walk the work list (each several items here: up to
# 8192 items for 1024 workgroups); Zipf-skewed routing leaves real small
# groups for them next to the tiled ones.
@pytest.mark.parametrize("wdtype", ["bf16", "fp8", "mxfp8"])
def test_forward_streaming_walk(wdtype):
    cfg = MoeConfig("walk_" + wdtype, 57, T=4096, H=512, E=64, k=2, I=2048, zipf_s=1.1, wdtype=wdtype)
    li = generate_layer(cfg, DEV)
    _, idx, _ = run_route(cfg, li)
    sizes = np.bincount(idx.cpu().numpy().ravel(), minlength=cfg.E)
    assert (sizes <= 48).sum() >= 4 and sizes.mean() > 96   # small groups beside large ones
    _forward_check(cfg, li)


# Large 8-bit launches run the persistent tiled kernel (one workgroup per CU
# walking its tiles, the next tile's first chunks loaded during the current
# tile's last ones, the epilogue stored from registers; MXFP8 with its scale
# stages alternating across tiles).  DeepSeek-like routing at 1024 tokens
# leaves the tiles of the 1024-row shared expert and a few routed groups
# (most workgroups get no tile or one); 1536 and 2048 tokens give about 4
# and 8 tiles per workgroup (the full layers: 17 to 37).
@pytest.mark.parametrize("wdtype", ["fp8", "mxfp8"])
@pytest.mark.parametrize("T", [1024, 1536, 2048])
def test_forward_8bit_persistent_walk(T, wdtype):
    cfg = MoeConfig(f"pers_{T}_{wdtype}", 58, T=T, H=2048, E=256, k=8, I=1024, n_shared=1, wdtype=wdtype)
    li = generate_layer(cfg, DEV)
    _, idx, _ = run_route(cfg, li)
    tiled = np.bincount(idx.cpu().numpy().ravel(), minlength=cfg.E) > 48
    assert (tiled.sum() < 16) if T == 1024 else (tiled.sum() > 64)
    _forward_check(cfg, li)


# Expert-parallel shares of the whole layer: small batches (single-workgroup
# dispatch) and large ones (tile kernels), with and without the shared
# expert, bf16 / fp8 / mxfp8; the EP8 shares of the Qwen3-235B-like layer.
SHARES = [
    MoeConfig("sh_small", 50, T=64, H=512, E=32, k=4, I=256, e_first=8, e_local=8),
    MoeConfig("sh_small_shared", 51, T=200, H=256, E=12, k=3, I=256, n_shared=1, e_first=9, e_local=3),
    MoeConfig("sh_large_fp8", 52, T=1500, H=512, E=16, k=4, I=256, n_shared=1, wdtype="fp8",
              e_first=4, e_local=4),
    MoeConfig("sh_large_mx", 53, T=700, H=384, E=8, k=2, I=256, wdtype="mxfp8", e_first=0, e_local=2),
    MoeConfig("sh_one_expert", 54, T=300, H=256, E=8, k=2, I=128, e_first=7, e_local=1),
]


@pytest.mark.parametrize("cfg", SHARES, ids=[c.name for c in SHARES])
def test_forward_share(cfg):
    _forward_check(cfg, generate_layer(cfg, DEV))


@pytest.mark.parametrize("name", [c.name for c in EXTRA_CONFIGS if c.e_local])
def test_forward_share_configs(name):
    cfg = next(c for c in EXTRA_CONFIGS if c.name == name)
    _forward_check(cfg, layer(cfg))


# Decode batches whose groups leave the chip idle take split-K in the
# streaming GEMMs (partials summed in K-range order by a reduce kernel):
# factors 2 to 8, with and without a shared expert, whole layer and shares,
# bf16, fp8 and MXFP8.
SPLITK = [
    MoeConfig("sk_q235_t4", 60, T=4, H=4096, E=128, k=8, I=1536),
    MoeConfig("sk_share_s8", 61, T=16, H=2048, E=64, k=4, I=1024, e_first=8, e_local=8),
    MoeConfig("sk_share_shared", 62, T=8, H=4096, E=16, k=2, I=1024, n_shared=1, e_first=12,
              e_local=4),
    # 8-bit streaming kernels with split-K: fp8 gate/up split 2 (a
    # DeepSeek-shaped share of 16 experts), fp8 down split 4, MXFP8 gate/up
    # split 4, MXFP8 down split 4 (gate/up partials re-quantised per 128 / 32
    # columns by the reduce)
    MoeConfig("sk_fp8_share", 63, T=16, H=7168, E=256, k=8, I=2048, wdtype="fp8", e_first=16,
              e_local=16),
    MoeConfig("sk_fp8_down", 64, T=8, H=1024, E=16, k=2, I=4096, n_shared=1, wdtype="fp8"),
    MoeConfig("sk_mx_share", 65, T=16, H=4096, E=128, k=8, I=1536, wdtype="mxfp8", e_first=16,
              e_local=16),
    MoeConfig("sk_mx_both", 66, T=8, H=1024, E=16, k=2, I=4096, n_shared=1, wdtype="mxfp8"),
]


@pytest.mark.parametrize("cfg", SPLITK, ids=[c.name for c in SPLITK])
def test_forward_split_k(cfg):
    _forward_check(cfg, generate_layer(cfg, DEV))


# Extremes of the supported shapes: 65536 tokens (256 rank tiles, groups of
# ~8k rows), K = 16384 for fp8 and MXFP8 (128 fp8 scale blocks per row),
# E = 1024 experts with k = 16.
EXTREMES = [
    MoeConfig("x_t64k", 70, T=65536, H=128, E=64, k=8, I=128),
    MoeConfig("x_h16k_fp8", 71, T=40, H=16384, E=4, k=2, I=256, n_shared=1, wdtype="fp8"),
    MoeConfig("x_h16k_mx", 73, T=30, H=16384, E=3, k=2, I=128, wdtype="mxfp8"),
    MoeConfig("x_e1024_k16", 72, T=300, H=256, E=1024, k=16, I=128),
]


@pytest.mark.parametrize("cfg", EXTREMES, ids=[c.name for c in EXTREMES])
def test_forward_extremes(cfg):
    _forward_check(cfg, generate_layer(cfg, DEV))


def test_shares_sum_to_the_layer_on_gpu():
    # Shares partitioning the experts (the shared expert on one of them) add up
    # to the whole layer: the all-reduce of the expert-parallel deployment.
    base = dict(T=400, H=512, E=24, k=4, I=256, wdtype="bf16")
    full_cfg = MoeConfig("sum_full", 55, n_shared=1, **base)
    full, _, _ = run_forward(full_cfg, generate_layer(full_cfg, DEV))
    total = torch.zeros((400, 512), dtype=torch.float32, device=DEV)
    for ef, el, ns in ((0, 10, 1), (10, 4, 0), (14, 10, 0)):
        c = MoeConfig("sum_share", 55, n_shared=ns, e_first=ef, e_local=el, **base)
        out, _, _ = run_forward(c, generate_layer(c, DEV))
        total += out.float()
    ref = full.float().cpu().numpy().astype(np.float64)
    err = rel_inf(total.cpu().numpy().astype(np.float64), ref)
    print(f"sum of shares vs layer: per-token rel err {err:.3e}")
    assert err <= 1e-2      # each share's output is rounded to bf16 once


def test_forward_zero_tokens():
    cfg = MoeConfig("T0", 36, T=0, H=256, E=8, k=2, I=256)
    sh = moe.shape_of(cfg)
    moe.moe_forward(sh, None, None, None, None, None, None, None, None, None, None, None, None, None, 0)
    counts = torch.full((8,), -1, dtype=torch.int32, device=DEV)
    offsets = torch.full((9,), -1, dtype=torch.int32, device=DEV)
    assert moe.moe_permute_workspace_bytes(sh) == 0
    moe.moe_permute(sh, None, None, counts, offsets, None, None, None, None)
    torch.cuda.synchronize()
    assert counts.cpu().tolist() == [0] * 8 and offsets.cpu().tolist() == [0] * 9
