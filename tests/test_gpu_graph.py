"""moe_forward captured in a HIP graph (torch.cuda.CUDAGraph over the caller's
stream) and replayed: every replay must give the eager call's bits, also
after the input changes in place, because group sizes, tile lists and row
maps are rebuilt on the device by every replay (no host round trip).

The kernels are deterministic (fixed summation orders, no atomics on values),
so eager and replayed results are compared bit for bit; the first replay's
output is also checked against the CPU oracle (routing bit-exact given the
GPU's router logits, output within the layer tolerance).
"""
import numpy as np
import pytest
import torch

import expert_ffn_layer_gemm_amd as moe
import oracle
from synth import MoeConfig, config_by_name, generate_layer, to_numpy_inputs
from tests.gpu_helpers import DEV, bf16_np, layer, rel_inf, run_route

TOL = {"bf16": 2e-2, "fp8": 5e-2, "mxfp8": 5e-2}

pytestmark = pytest.mark.gpu


def _buffers(cfg):
    sh = moe.shape_of(cfg)
    ws = torch.empty(moe.moe_forward_workspace_bytes(sh), dtype=torch.uint8, device=DEV)
    out = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=DEV)
    idx = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=DEV)
    w = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=DEV)
    return sh, ws, out, idx, w


def _forward(sh, li, x, bufs, stream):
    ws, out, idx, w = bufs
    moe.moe_forward(sh, x, li.w_router, li.router_bias, li.w_gate, li.w_up, li.w_down,
                    li.s_gate, li.s_up, li.s_down, out, idx, w, ws, stream=stream)


def _eager(sh, li, x, cfg):
    _, ws, out, idx, w = _buffers(cfg)
    _forward(sh, li, x, (ws, out, idx, w), torch.cuda.current_stream())
    torch.cuda.synchronize()
    return out.clone(), idx.clone(), w.clone()


CASES = [
    config_by_name("qwen3_235b_decode"),
    # small shapes that still reach the tiled kernels (groups > 48 rows) and
    # the fp8 path with a shared expert
    MoeConfig("graph_bf16", 21, T=640, H=512, E=8, k=2, I=256),
    MoeConfig("graph_fp8", 22, T=384, H=512, E=16, k=4, I=256, n_shared=1, wdtype="fp8"),
    # skewed routing: groups on both sides of 48 rows, so the tiled chain runs
    # on the library's second stream, forked and joined inside the capture
    MoeConfig("graph_mixed", 23, T=512, H=512, E=64, k=4, I=256, zipf_s=1.1),
    MoeConfig("graph_mxfp8", 24, T=384, H=512, E=16, k=4, I=256, n_shared=1, wdtype="mxfp8"),
    # an expert-parallel share whose streaming GEMMs take split-K
    MoeConfig("graph_share_splitk", 25, T=16, H=2048, E=64, k=4, I=1024, e_first=8, e_local=8),
]


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_graph_replay_matches_eager(cfg):
    li = layer(cfg) if cfg.name == "qwen3_235b_decode" else generate_layer(cfg, DEV)
    sh, ws, out, idx, w = _buffers(cfg)
    x = li.x.clone()
    ref = _eager(sh, li, x, cfg)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _forward(sh, li, x, (ws, out, idx, w), s)        # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        _forward(sh, li, x, (ws, out, idx, w), torch.cuda.current_stream())
    torch.cuda.synchronize()

    for rep in range(3):
        out.zero_()
        idx.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        if rep == 0:
            # the replayed layer against the oracle, routed on the GPU's logits
            logits, _, _ = run_route(cfg, li)
            ref_o = oracle.forward(to_numpy_inputs(li), logits_override=logits.cpu().numpy())
            assert np.array_equal(idx.cpu().numpy(), ref_o.topk_idx), "replay routing vs oracle"
            err = rel_inf(bf16_np(out), ref_o.out)
            print(f"{cfg.name}: replay vs oracle per-token rel err {err:.3e}")
            assert err <= TOL[cfg.wdtype]
        assert torch.equal(out.view(torch.int16), ref[0].view(torch.int16)), f"replay {rep}: out"
        assert torch.equal(idx, ref[1]), f"replay {rep}: topk_idx"
        assert torch.equal(w, ref[2]), f"replay {rep}: topk_w"
        # eager work of the program between replays
        _ = (x.float() * 2).sum().item()

    # New tokens in the captured input buffer: a different routing, rebuilt on
    # the device by the replay.
    gen = torch.Generator(device=DEV).manual_seed(1234 + cfg.seed)
    x2 = torch.randn(x.shape, generator=gen, device=DEV, dtype=torch.float32).to(torch.bfloat16)
    ref2 = _eager(sh, li, x2, cfg)
    assert not torch.equal(ref2[1], ref[1])
    x.copy_(x2)
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref2[0].view(torch.int16))
    assert torch.equal(idx, ref2[1])
    assert torch.equal(w, ref2[2])
