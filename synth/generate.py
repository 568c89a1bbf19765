"""Seeded generation of one layer's inputs and weights.

Recipe (per config):
- x ~ N(0, 1), cast fp32 -> bf16 (round to nearest even, torch's cast).
- router weight W_r [E, H] (torch Linear layout) ~ N(0, router_std), kept fp32.
- optional Zipf(s) popularity term b [E]: b_e = -s * ln(rho_e), rho a seeded
  permutation of 1..E, added to the router logits by the layer.
- expert weights per expert e (keyed separately so any single expert can be
  regenerated, and an expert-parallel share holds the same weights as the
  whole layer): W_gate[e], W_up[e] [I, H] and W_down[e] [H, I] ~ N(0, w_std),
  cast to bf16; or, for "fp8" configs, converted offline to e4m3fn codes with
  one fp32 scale per 128x128 block (scale = block amax / 448, 1 for an all-zero
  block; codes = torch's e4m3fn cast of the clamped quotient); or, for
  "mxfp8" configs, to MXFP8: e4m3fn codes with one power-of-two scale per 32
  values along K (E8M0 byte = floor(log2(amax)) - 8 + 127, 0 for an all-zero
  block; codes = torch's e4m3fn cast of the quotient clamped to +-448).  This
  static weight conversion is input preparation: the layer consumes codes +
  scales.

Every tensor is drawn from its own torch.Generator seeded by
(config seed, tensor id, expert id); tensor ids: 0 x, 1 W_r, 2 W_gate,
3 W_up, 4 W_down, 5 Zipf permutation.
"""
from dataclasses import dataclass
from typing import Optional

import torch

from .configs import MoeConfig

E4M3_MAX = 448.0


def _gen(device, seed: int, tensor_id: int, expert_id: int = 0) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed << 40) | (tensor_id << 32) | expert_id)
    return g


@dataclass
class LayerInputs:
    cfg: MoeConfig
    x: torch.Tensor                       # [T, H] bf16
    w_router: torch.Tensor                # [E, H] fp32
    router_bias: Optional[torch.Tensor]   # [E] fp32 or None
    w_gate: torch.Tensor                  # [G, I, H] bf16 | uint8 e4m3fn codes
    w_up: torch.Tensor                    # [G, I, H]
    w_down: torch.Tensor                  # [G, H, I]
    s_gate: Optional[torch.Tensor] = None  # fp8: [G, I/128, H/128] fp32; mxfp8: [G, I, H/32] uint8
    s_up: Optional[torch.Tensor] = None
    s_down: Optional[torch.Tensor] = None  # fp8: [G, H/128, I/128] fp32; mxfp8: [G, H, I/32] uint8

    def to(self, device) -> "LayerInputs":
        f = lambda t: None if t is None else t.to(device)
        return LayerInputs(self.cfg, f(self.x), f(self.w_router), f(self.router_bias),
                           f(self.w_gate), f(self.w_up), f(self.w_down),
                           f(self.s_gate), f(self.s_up), f(self.s_down))


def _fp8_blocks(w: torch.Tensor):
    """Static conversion of an fp32 [N, K] matrix to e4m3fn codes + per-128x128 scales."""
    n, k = w.shape
    blocks = w.reshape(n // 128, 128, k // 128, 128)
    amax = blocks.abs().amax(dim=(1, 3))
    scale = torch.where(amax == 0, torch.ones_like(amax), amax / E4M3_MAX)
    q = (blocks / scale[:, None, :, None]).clamp_(-E4M3_MAX, E4M3_MAX)
    codes = q.reshape(n, k).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale.contiguous()


def _mx_rows(w: torch.Tensor):
    """Static conversion of an fp32 [N, K] matrix to MXFP8: e4m3fn codes + E8M0 per 32 along K."""
    n, k = w.shape
    blocks = w.reshape(n, k // 32, 32)
    amax = blocks.abs().amax(dim=-1)
    _, ex = torch.frexp(torch.where(amax > 0, amax, torch.ones_like(amax)))
    e = torch.where(amax > 0, ex - 1 - 8, torch.full_like(ex, -127)).clamp_(-127, 127)
    q = (blocks * torch.exp2(-e.to(torch.float32))[..., None]).clamp_(-E4M3_MAX, E4M3_MAX)
    codes = q.reshape(n, k).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, (e + 127).to(torch.uint8)


def generate_expert(cfg: MoeConfig, e: int, device="cpu"):
    """Weights of one expert (gate [I,H], up [I,H], down [H,I]) as fp32 before casting."""
    out = []
    for tid, shape in ((2, (cfg.I, cfg.H)), (3, (cfg.I, cfg.H)), (4, (cfg.H, cfg.I))):
        g = _gen(device, cfg.seed, tid, e)
        out.append(torch.randn(shape, generator=g, device=device, dtype=torch.float32) * cfg.w_std)
    return out


def generate_layer(cfg: MoeConfig, device="cpu") -> LayerInputs:
    T, H, E, I = cfg.T, cfg.H, cfg.E, cfg.I
    G = cfg.n_groups
    x = torch.randn((T, H), generator=_gen(device, cfg.seed, 0), device=device,
                    dtype=torch.float32).to(torch.bfloat16)
    w_router = torch.randn((E, H), generator=_gen(device, cfg.seed, 1), device=device,
                           dtype=torch.float32) * cfg.router_std
    bias = None
    if cfg.zipf_s is not None:
        rho = torch.randperm(E, generator=_gen(device, cfg.seed, 5), device=device) + 1
        bias = (-cfg.zipf_s * torch.log(rho.to(torch.float64))).to(torch.float32)
    fp8 = cfg.wdtype == "fp8"
    mx = cfg.wdtype == "mxfp8"
    if fp8 or mx:
        assert H % 128 == 0 and I % 128 == 0, "8-bit weights need H, I multiples of 128"
    wdt = torch.uint8 if (fp8 or mx) else torch.bfloat16
    w_gate = torch.empty((G, I, H), dtype=wdt, device=device)
    w_up = torch.empty((G, I, H), dtype=wdt, device=device)
    w_down = torch.empty((G, H, I), dtype=wdt, device=device)
    s_gate = s_up = s_down = None
    if fp8:
        s_gate = torch.empty((G, I // 128, H // 128), dtype=torch.float32, device=device)
        s_up = torch.empty_like(s_gate)
        s_down = torch.empty((G, H // 128, I // 128), dtype=torch.float32, device=device)
    if mx:
        s_gate = torch.empty((G, I, H // 32), dtype=torch.uint8, device=device)
        s_up = torch.empty_like(s_gate)
        s_down = torch.empty((G, H, I // 32), dtype=torch.uint8, device=device)
    for e in range(G):
        # Local group e holds global expert e_first + e (the shared expert is
        # global id E): an expert's weights do not depend on the share.
        gid = cfg.e_first + e if e < cfg.E_loc else cfg.E + (e - cfg.E_loc)
        wg, wu, wd = generate_expert(cfg, gid, device)
        if fp8:
            w_gate[e], s_gate[e] = _fp8_blocks(wg)
            w_up[e], s_up[e] = _fp8_blocks(wu)
            w_down[e], s_down[e] = _fp8_blocks(wd)
        elif mx:
            w_gate[e], s_gate[e] = _mx_rows(wg)
            w_up[e], s_up[e] = _mx_rows(wu)
            w_down[e], s_down[e] = _mx_rows(wd)
        else:
            w_gate[e] = wg.to(torch.bfloat16)
            w_up[e] = wu.to(torch.bfloat16)
            w_down[e] = wd.to(torch.bfloat16)
        del wg, wu, wd
    return LayerInputs(cfg, x, w_router, bias, w_gate, w_up, w_down, s_gate, s_up, s_down)


def to_numpy_inputs(li: LayerInputs) -> dict:
    """Host copies in the plain formats the oracle reads (bf16 as uint16 bit patterns)."""
    def bits(t):
        if t is None:
            return None
        t = t.detach().cpu()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view("uint16")
        return t.numpy()
    return dict(x_bf16=bits(li.x), w_router=bits(li.w_router), router_bias=bits(li.router_bias),
                w_gate=bits(li.w_gate), w_up=bits(li.w_up), w_down=bits(li.w_down),
                s_gate=bits(li.s_gate), s_up=bits(li.s_up), s_down=bits(li.s_down),
                k=li.cfg.k, n_shared=li.cfg.n_shared, wdtype=li.cfg.wdtype,
                e_first=li.cfg.e_first, e_local=li.cfg.e_local)
