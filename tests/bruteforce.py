"""Float64 per-token brute force of the MoE layer (test helper, independent of oracle/).

No permutation, no grouping: for each token, pick its experts by sorting all
experts with the key (-logit, index), weight them with a float64 softmax over
the picked logits, and sum w_j * FFN_e(x_t).  FP8 quantisation (fp8 and mxfp8
layers) uses torch's e4m3fn cast as the codec and torch.frexp for the MX
scale exponent, so it shares nothing with the oracle's.
"""
import numpy as np
import torch


def _bf16_to_f64(u16):
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).double().numpy()


def _e4m3_values(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()


def _quant_dequant_rows_torch(v64):
    """Per row, per 128 columns: scale = amax/448 (fp32), codes = torch e4m3fn cast."""
    v = torch.from_numpy(v64.astype(np.float32))
    rows, C = v.shape
    g = v.reshape(rows, C // 128, 128)
    amax = g.abs().amax(-1)
    s = torch.where(amax == 0, torch.ones_like(amax), amax / 448.0)
    q = (g / s[..., None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).double()
    return (q * s[..., None].double()).reshape(rows, C).numpy()


def _mx_quant_dequant_rows_torch(v64):
    """Per row, blocks of 32 columns: X = 2^(floor(log2 amax) - 8) (torch.frexp),
    codes = torch e4m3fn cast of v / X clamped to +-448; returns codes * X."""
    v = torch.from_numpy(v64.astype(np.float32)).double()
    rows, C = v.shape
    g = v.reshape(rows, C // 32, 32)
    amax = g.abs().amax(-1)
    _, ex = torch.frexp(torch.where(amax > 0, amax, torch.ones_like(amax)))
    e = torch.where(amax > 0, ex - 9, torch.full_like(ex, -127)).clamp(-127, 127).double()
    q = torch.ldexp(g, -e[..., None]).clamp(-448.0, 448.0).float().to(torch.float8_e4m3fn).double()
    return torch.ldexp(q, e[..., None]).reshape(rows, C).numpy()


def _weights64(inp, e):
    if inp["wdtype"] == "mxfp8":
        def dqm(c, s):
            n, k = c.shape
            return (_e4m3_values(c).reshape(n, k // 32, 32)
                    * np.exp2(s.astype(np.float64) - 127.0)[..., None]).reshape(n, k)
        return (dqm(inp["w_gate"][e], inp["s_gate"][e]), dqm(inp["w_up"][e], inp["s_up"][e]),
                dqm(inp["w_down"][e], inp["s_down"][e]))
    if inp["wdtype"] == "fp8":
        def dq(c, s):
            n, k = c.shape
            return (_e4m3_values(c).reshape(n // 128, 128, k // 128, 128)
                    * s.astype(np.float64)[:, None, :, None]).reshape(n, k)
        return (dq(inp["w_gate"][e], inp["s_gate"][e]), dq(inp["w_up"][e], inp["s_up"][e]),
                dq(inp["w_down"][e], inp["s_down"][e]))
    return _bf16_to_f64(inp["w_gate"][e]), _bf16_to_f64(inp["w_up"][e]), _bf16_to_f64(inp["w_down"][e])


def layer_bruteforce(inp):
    """Returns (out [T,H] float64, topk_idx [T,k], logits float64, boundary gap per token).

    With inp["e_local"] > 0 (an expert-parallel share) only the picks of
    experts [e_first, e_first + e_local) contribute, with their full-softmax
    weights, and the weights arrays hold those experts (then the shared one).
    """
    x = _bf16_to_f64(inp["x_bf16"])
    T, H = x.shape
    Wr = inp["w_router"].astype(np.float64)          # [E, H]
    E = Wr.shape[0]
    k, ns, fp8 = inp["k"], inp["n_shared"], inp["wdtype"] == "fp8"
    mx = inp["wdtype"] == "mxfp8"
    quant = _mx_quant_dequant_rows_torch if mx else _quant_dequant_rows_torch
    logits = x @ Wr.T
    if inp.get("router_bias") is not None:
        logits = logits + inp["router_bias"].astype(np.float64)
    xin = quant(x) if (fp8 or mx) else x
    e_first = inp.get("e_first", 0)
    L = inp.get("e_local", 0) or E
    W = [_weights64(inp, e) for e in range(L + ns)]

    def ffn(e, xt):
        wg, wu, wd = W[e]
        g, u = wg @ xt, wu @ xt
        h = g / (1.0 + np.exp(-g)) * u
        if fp8 or mx:
            h = quant(h[None, :])[0]
        return wd @ h

    out = np.zeros((T, H))
    idx = np.zeros((T, k), np.int64)
    gap = np.full(T, np.inf)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-logits[t, e], e))
        idx[t] = order[:k]
        if k < E:
            gap[t] = logits[t, order[k - 1]] - logits[t, order[k]]
        sel = logits[t, idx[t]]
        p = np.exp(sel - sel.max())
        p /= p.sum()
        for j in range(k):
            if e_first <= idx[t, j] < e_first + L:
                out[t] += p[j] * ffn(idx[t, j] - e_first, xin[t])
        for s in range(ns):
            out[t] += ffn(L + s, xin[t])
    return out, idx, logits, gap
