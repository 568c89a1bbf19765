"""moe_forward_noalloc (the entry point with the library's fixed device
scratch instead of a caller workspace) against moe_forward on the same
inputs: routing and output bit for bit (the same kernels on the same
operands), and the output against the CPU oracle within the layer tolerance.
Two calls in a row share the scratch, the second with a smaller batch, and the
results must not depend on what the first left there."""
import numpy as np
import pytest
import torch

import expert_ffn_layer_gemm_amd as moe
import oracle
from synth import MoeConfig, config_by_name, generate_layer, to_numpy_inputs
from tests.gpu_helpers import DEV, bf16_np, rel_inf, run_forward

pytestmark = pytest.mark.gpu
TOL = {"bf16": 2e-2, "fp8": 5e-2, "mxfp8": 5e-2}


def _noalloc(cfg, li, x):
    sh = moe.shape_of(cfg)
    assert moe.moe_forward_workspace_bytes(sh) <= moe.NOALLOC_SCRATCH_BYTES
    out = torch.full((cfg.T, cfg.H), float("nan"), dtype=torch.bfloat16, device=DEV)
    idx = torch.full((cfg.T, cfg.k), -7, dtype=torch.int32, device=DEV)
    w = torch.full((cfg.T, cfg.k), float("nan"), dtype=torch.float32, device=DEV)
    moe.moe_forward_noalloc(sh, x, li.w_router, li.router_bias, li.w_gate, li.w_up, li.w_down,
                            li.s_gate, li.s_up, li.s_down, out, idx, w)
    torch.cuda.synchronize()
    return out, idx, w


def _sub(li, cfg, T):
    """The same layer (weights, router) with the first T tokens."""
    small = MoeConfig(cfg.name + f"_T{T}", cfg.seed, T=T, H=cfg.H, E=cfg.E, k=cfg.k, I=cfg.I,
                      n_shared=cfg.n_shared, wdtype=cfg.wdtype, zipf_s=cfg.zipf_s,
                      e_first=cfg.e_first, e_local=cfg.e_local)
    return small, type(li)(small, li.x[:T].contiguous(), li.w_router, li.router_bias, li.w_gate,
                           li.w_up, li.w_down, li.s_gate, li.s_up, li.s_down)


def _check(cfg, li):
    out, idx, w = _noalloc(cfg, li, li.x)
    ref_out, ref_idx, ref_w = run_forward(cfg, li)
    assert torch.equal(idx, ref_idx) and torch.equal(w, ref_w)
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
    ref = oracle.forward(to_numpy_inputs(li))
    same = (idx.cpu().numpy() == ref.topk_idx).all(axis=1)
    assert same.sum() >= cfg.T - max(2, cfg.T // 500)
    err = rel_inf(bf16_np(out)[same], ref.out[same])
    print(f"{cfg.name}: noalloc == moe_forward bit for bit; vs oracle per-token rel err {err:.3e}")
    assert err <= TOL[cfg.wdtype]


CASES = [
    config_by_name("qwen3_235b_decode"),
    # groups above 48 rows: the tiled chain runs on the caller's stream here
    MoeConfig("noalloc_tiled", 81, T=300, H=512, E=8, k=2, I=256, n_shared=1),
    MoeConfig("noalloc_fp8", 82, T=200, H=512, E=16, k=4, I=256, n_shared=1, wdtype="fp8"),
]


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_noalloc_matches_forward_then_smaller_batch(cfg):
    li = generate_layer(cfg, DEV)
    _check(cfg, li)                      # first call: the full batch
    small, li_s = _sub(li, cfg, max(1, cfg.T // 4))
    _check(small, li_s)                  # second call: a smaller batch on the same scratch


def test_noalloc_rejects_oversized_shape():
    cfg = config_by_name("deepseek_v3_fp8")
    sh = moe.shape_of(cfg)
    assert moe.moe_forward_workspace_bytes(sh) > moe.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((16, 16), dtype=torch.bfloat16, device=DEV)   # never read: rejected on the host
    with pytest.raises(moe.MoeError, match="scratch"):
        moe.moe_forward_noalloc(sh, x, x, None, x, x, x, x, x, x, x, None, None)
