"""Pins of the oracle's expert-parallel share ("CuTeDSL at Perplexity", MoE
Dispatch/Combine, tensor-parallel deployment: with the input replicated, a
rank's dispatch keeps the tokens routed to its own experts and its local
combine sums them before the all-reduce).

- against an fp64 per-token brute force that loops over the local experts
  only (tests/bruteforce.py), on micro shapes with and without a shared expert;
- shares that partition the experts sum to the whole layer (the all-reduce);
- dispatch: remote pairs get dest = -1, the kept pairs form a bijection onto
  the share's rows, token-ascending inside each group;
- a share holding every expert is the whole layer, bit for bit.
"""
import numpy as np
import pytest

import oracle
from synth import MoeConfig, generate_layer, to_numpy_inputs
from tests.bruteforce import layer_bruteforce


def _rel_inf(out, ref):
    num = np.abs(out - ref).max(axis=1)
    den = np.abs(ref).max(axis=1)
    return float((num / np.maximum(den, 1e-30)).max())


def _share(cfg, e_first, e_local, n_shared=None):
    ns = cfg.n_shared if n_shared is None else n_shared
    return MoeConfig(cfg.name + f"_ep{e_first}_{e_local}", cfg.seed, T=cfg.T, H=cfg.H, E=cfg.E,
                     k=cfg.k, I=cfg.I, n_shared=ns, wdtype=cfg.wdtype, zipf_s=cfg.zipf_s,
                     e_first=e_first, e_local=e_local)


@pytest.mark.parametrize("case", range(8))
def test_share_vs_bruteforce(case):
    rng = np.random.default_rng(2000 + case)
    E = int(rng.integers(2, 13))
    wd = ["bf16", "fp8", "mxfp8", "bf16"][case % 4]
    base = MoeConfig(f"epm{case}", 300 + case, T=int(rng.integers(1, 33)), H=128 * int(rng.integers(1, 3)),
                     E=E, k=int(rng.integers(1, min(E, 4) + 1)), I=128 * int(rng.integers(1, 3)),
                     n_shared=int(case % 2), wdtype=wd)
    e_local = int(rng.integers(1, E + 1))
    e_first = int(rng.integers(0, E - e_local + 1))
    cfg = _share(base, e_first, e_local)
    inp = to_numpy_inputs(generate_layer(cfg, "cpu"))
    res = oracle.forward(inp)
    ref, ref_idx, _, gap = layer_bruteforce(inp)
    ok = gap > 1e-5
    assert np.array_equal(res.topk_idx[ok], ref_idx[ok])
    # 8-bit layers: the oracle quantises h from fp32 sums, the brute force from
    # float64 sums (one e4m3 step apart at most).
    tol = 1e-4 if wd == "bf16" else 2e-2
    nz = np.abs(ref[ok]).max(axis=1) > 0
    if nz.any():
        assert _rel_inf(res.out[ok][nz], ref[ok][nz]) <= tol
    # tokens with no local pick and no shared expert give exactly zero
    assert np.all(res.out[np.abs(ref).max(axis=1) == 0] == 0)


@pytest.mark.parametrize("wdtype", ["bf16", "fp8"])
def test_shares_partitioning_the_experts_sum_to_the_layer(wdtype):
    cfg = MoeConfig("ep_sum", 41, T=48, H=256, E=12, k=3, I=128, n_shared=1, wdtype=wdtype)
    full = oracle.forward(to_numpy_inputs(generate_layer(cfg, "cpu")))
    cuts = [0, 5, 7, 12]            # three ranks; the shared expert sits on the first
    total = np.zeros_like(full.out, dtype=np.float64)
    for r in range(3):
        sh = _share(cfg, cuts[r], cuts[r + 1] - cuts[r], n_shared=1 if r == 0 else 0)
        res = oracle.forward(to_numpy_inputs(generate_layer(sh, "cpu")))
        assert np.array_equal(res.topk_idx, full.topk_idx)
        total += res.out
    # fp32 sums in another order: agreement to a few fp32 ulps of the terms
    assert _rel_inf(total, full.out.astype(np.float64)) <= 1e-5


def test_share_dispatch_tables():
    rng = np.random.default_rng(7)
    T, E, k = 200, 16, 4
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    e_first, L = 4, 6
    counts, offsets, dest, src = oracle.counting_sort(idx, E, 1, e_first, L)
    local = (idx >= e_first) & (idx < e_first + L)
    assert np.all((dest >= 0) == local)
    assert counts[:L].tolist() == [int((idx == e_first + g).sum()) for g in range(L)]
    assert counts[L] == T and offsets[L] == local.sum() and offsets[-1] == local.sum() + T
    rows = dest[local]
    assert sorted(rows.tolist()) == list(range(int(local.sum())))   # bijection onto the local rows
    for g in range(L):
        lo, hi = offsets[g], offsets[g + 1]
        toks = src[lo:hi]
        assert np.all(np.diff(toks) > 0) and np.all(idx[toks] .__eq__(e_first + g).any(axis=1))
    assert np.array_equal(src[offsets[L]:], np.arange(T))
    t, j = np.nonzero(local)
    assert np.array_equal(src[dest[t, j]], t)


def test_share_with_every_expert_is_the_layer():
    cfg = MoeConfig("ep_all", 42, T=40, H=128, E=6, k=2, I=256, n_shared=1)
    full = oracle.forward(to_numpy_inputs(generate_layer(cfg, "cpu")))
    sh = oracle.forward(to_numpy_inputs(generate_layer(_share(cfg, 0, 6), "cpu")))
    assert np.array_equal(sh.out, full.out)
    assert np.array_equal(sh.dest, full.dest) and np.array_equal(sh.src_row, full.src_row)


def test_share_forward_tokens_matches_forward():
    base = MoeConfig("ep_tok", 43, T=64, H=256, E=10, k=3, I=128, n_shared=1, wdtype="fp8")
    cfg = _share(base, 3, 4)
    inp = to_numpy_inputs(generate_layer(cfg, "cpu"))
    full = oracle.forward(inp)
    sample = np.array([0, 5, 17, 40, 63])
    part = oracle.forward_tokens(inp, sample)
    assert _rel_inf(part.out, full.out[sample]) <= 1e-6
