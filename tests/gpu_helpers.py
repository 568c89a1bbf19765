"""Helpers for the GPU parity tests: allocate with torch, call the C ABI, read back."""
import numpy as np
import torch

import expert_ffn_layer_gemm_amd as moe
from synth import generate_layer

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None
_cache = {}


def layer(cfg):
    """Generated inputs of one config, kept until another config is asked for."""
    if cfg.name not in _cache:
        _cache.clear()
        torch.cuda.empty_cache()
        _cache[cfg.name] = generate_layer(cfg, DEV)
    return _cache[cfg.name]


def bf16_np(t):
    """torch bf16 tensor -> numpy fp32 (exact)."""
    u = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return (u.astype(np.uint32) << 16).view(np.float32)


def bf16_bits_np(t):
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_bf16_rne(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 round-to-nearest-even via torch's cast, back as fp32."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).float().numpy()


def rel_inf(out, ref):
    num = np.abs(out - ref).max(axis=1)
    den = np.maximum(np.abs(ref).max(axis=1), 1e-30)
    return float((num / den).max())


def run_route(cfg, li):
    sh = moe.shape_of(cfg)
    logits = torch.empty((cfg.T, cfg.E), dtype=torch.float32, device=DEV)
    idx = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=DEV)
    w = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=DEV)
    ws = torch.empty(max(moe.moe_route_workspace_bytes(sh), 16), dtype=torch.uint8, device=DEV)
    moe.moe_route(sh, li.x, li.w_router, li.router_bias, logits, idx, w, ws)
    torch.cuda.synchronize()
    return logits, idx, w


def run_permute(cfg, idx, x):
    sh = moe.shape_of(cfg)
    G, R = cfg.n_groups, cfg.R
    fp8 = cfg.wdtype in ("fp8", "mxfp8")
    counts = torch.empty(G, dtype=torch.int32, device=DEV)
    offsets = torch.empty(G + 1, dtype=torch.int32, device=DEV)
    dest = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=DEV)
    src = torch.empty(R, dtype=torch.int32, device=DEV)
    x_perm = torch.empty((R, cfg.H), dtype=torch.uint8 if fp8 else torch.bfloat16, device=DEV)
    if cfg.wdtype == "mxfp8":
        x_scale = torch.empty((R, cfg.H // 32), dtype=torch.uint8, device=DEV)
    elif fp8:
        # K-block-major: the R row scales of each 128-channel block are adjacent
        x_scale = torch.empty((cfg.H // 128, R), dtype=torch.float32, device=DEV)
    else:
        x_scale = None
    ws = torch.empty(max(moe.moe_permute_workspace_bytes(sh), 16), dtype=torch.uint8, device=DEV)
    moe.moe_permute(sh, idx, x, counts, offsets, dest, src, x_perm, x_scale, ws)
    torch.cuda.synchronize()
    return counts, offsets, dest, src, x_perm, x_scale


def run_ffn(cfg, li, offsets, x_perm, x_scale):
    sh = moe.shape_of(cfg)
    ws = torch.empty(moe.moe_ffn_workspace_bytes(sh), dtype=torch.uint8, device=DEV)
    y = torch.zeros((cfg.R, cfg.H), dtype=torch.bfloat16, device=DEV)
    moe.moe_grouped_ffn(sh, offsets, x_perm, x_scale, li.w_gate, li.w_up, li.w_down,
                        li.s_gate, li.s_up, li.s_down, y, ws)
    torch.cuda.synchronize()
    return y


def run_forward(cfg, li):
    sh = moe.shape_of(cfg)
    ws = torch.empty(moe.moe_forward_workspace_bytes(sh), dtype=torch.uint8, device=DEV)
    out = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=DEV)
    idx = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=DEV)
    w = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=DEV)
    moe.moe_forward(sh, li.x, li.w_router, li.router_bias, li.w_gate, li.w_up, li.w_down,
                    li.s_gate, li.s_up, li.s_down, out, idx, w, ws)
    torch.cuda.synchronize()
    return out, idx, w
