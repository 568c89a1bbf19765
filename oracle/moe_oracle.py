"""Plain fp32 CPU oracle of one GPU's share of an MoE layer.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py): imported by tests/,
__graft_entry__.smoke() and bench.py's cpu_baseline leg, never by the product.

The layer, as the pages state it:
  1. router: logits = x W_r (+ per-expert bias), top-k per token with scores
     ("Lower latency and higher throughput with multi-node DeepSeek deployment",
     MoE Router section);
  2. dispatch: count tokens per expert, give each token a unique index in its
     expert's list, copy tokens into per-expert buffers ("CuTeDSL at
     Perplexity", MoE Dispatch/Combine, local kernel);
  3. grouped expert FFN with SwiGLU: silu(x W_gate^T) * (x W_up^T), then the
     down projection (Qwen3.5-397B on Ironwood, section 4.2.2, GMM v2 with fused
     SwiGLU);
  4. combine: weighted accumulation of the expert outputs back in token order
     ("CuTeDSL at Perplexity", local combine); a shared expert's output is added
     (DeepSeek-deployment page, Expert parallelism section).
  5. expert-parallel share ("CuTeDSL at Perplexity", MoE Dispatch/Combine,
     tensor-parallel deployment; "Hosting Qwen on Blackwell", expert-parallel
     prefill kernel): with the input replicated on every GPU, a GPU's dispatch
     keeps only the (token, slot) pairs routed to its own experts and its
     combine sums those local contributions; the sum over GPUs (an
     all-reduce) gives the layer's output.

Readings where the pages are silent:
  - top-k selects on fp32 logits; ties go to the lower expert index; +0 and -0
    tie; slots are ordered best first.
  - weights: softmax over the selected logits (equal to full softmax
    renormalised over the selected experts).
  - rows inside an expert group are token-ascending; groups are unpadded.
  - shared expert = the group after the routed ones, rows offsets[G-1] + t
    (T*k + t for the whole layer), weight 1, added after the routed sum.
  - expert-parallel share of experts [e_first, e_first + e_local): routing over
    all E experts as usual; group g holds expert e_first + g; pairs routed
    elsewhere get dest = -1 and add nothing; the shared expert, if the share
    holds it, comes after the local groups.  Output = the share's partial sum.
  - fp8 layers: x and h are quantised per row per 128 channels (scale = amax/448).
  - mxfp8 layers: weights, x and h are MXFP8 (E4M3 elements, one power-of-two
    E8M0 scale per 32 values along the contraction dimension; oracle/mx.py).

Parity status (pins in tests/test_oracle_*.py):
  router_logits  pinned (exact on small-integer inputs; W_r = 0 special case)
  topk_softmax   pinned (brute-force sorted() on tiny inputs, ties, +-0, fp64 softmax)
  counting_sort  pinned (brute-force loops, bijection / scan invariants)
  expert_ffn     pinned (closed-form SwiGLU values, fp64 brute force per token)
  combine        pinned (one-hot routing = inverse permutation, identical experts)
  expert shares  pinned (fp64 per-token brute force over local experts; shares
                 partitioning the experts sum to the whole layer; remote pairs
                 get dest = -1; tests/test_oracle_ep.py)
  forward        pinned on tiny and random micro shapes against an fp64
                 per-token brute force; at the large sizes it rests on those pins.
  mx_*           pinned (closed-form exponents, exhaustive nearest-code search,
                 exact round trips; tests/test_oracle_mx.py)
"""
import numpy as np

from .fp8_e4m3 import (quantize_groups_128, dequantize_groups_128,
                       dequantize_blocks_128x128)
from .mx import mx_quantize_rows, mx_dequantize_rows

F32 = np.float32


def bf16_bits_to_f32(u16: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to fp32."""
    return (np.asarray(u16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- router ----
def router_logits(x: np.ndarray, w_router: np.ndarray, bias=None) -> np.ndarray:
    """logits[t, e] = sum_h x[t, h] W_r[e, h] (+ b[e]), fp32; W_r is [E, H].

    The router's input to top-k (DeepSeek-deployment page, MoE Router).
    """
    l = np.matmul(x.astype(F32), w_router.astype(F32).T, dtype=F32)
    if bias is not None:
        l = (l + bias.astype(F32)[None, :]).astype(F32)
    return l


def topk_softmax(logits: np.ndarray, k: int):
    """Top-k experts per token and their renormalised softmax weights.

    DeepSeek-deployment page, MoE Router: a sort that tracks indices, giving
    the top-k indices and scores per token.  A stable sort of -logits puts the
    lower expert index first among equal logits (and treats -0 == +0 as equal).
    Weights: w_j = exp(l_j - l_0) / sum_j' exp(l_j' - l_0) over the selected.
    """
    assert np.all(np.isfinite(logits)), "router logits must be finite"
    T, E = logits.shape
    assert 1 <= k <= E
    order = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    sel = np.take_along_axis(logits, order, axis=1).astype(F32)
    ex = np.exp((sel - sel[:, :1]).astype(F32)).astype(F32)
    w = (ex / ex.sum(axis=1, keepdims=True, dtype=F32)).astype(F32)
    return order.astype(np.int32), w


# -------------------------------------------------------------- dispatch ----
def counting_sort(topk_idx: np.ndarray, E: int, n_shared: int = 0, e_first: int = 0,
                  e_local: int = 0):
    """Per-expert counts, offsets and each (token, slot)'s row in the permuted matrix.

    "CuTeDSL at Perplexity", MoE Dispatch/Combine, local kernel: count the
    tokens of each expert, give each token a unique index within its expert,
    then copy.  Unique index = number of earlier tokens routed to the same
    expert (token-ascending, unpadded groups).  The shared expert is the group
    after the routed ones, holding every token in order.

    Expert-parallel share (same page, tensor-parallel deployment: the local
    dispatch only selects the tokens assigned to experts of this rank):
    e_local > 0 keeps the experts [e_first, e_first + e_local) as groups
    0 .. e_local-1; the pairs routed elsewhere get dest = -1 and no row.

    Returns counts [L+ns], offsets [L+ns+1], dest [T, k], src_row [R] (int32),
    L = e_local or E, R = offsets[-1].
    """
    T, k = topk_idx.shape
    L = e_local or E
    flat = topk_idx.reshape(-1).astype(np.int64)
    assert flat.size == 0 or (flat.min() >= 0 and flat.max() < E), "expert index out of range"
    local = flat - e_first
    keep = (local >= 0) & (local < L)
    counts = np.bincount(local[keep], minlength=L).astype(np.int64)
    if n_shared:
        counts = np.concatenate([counts, np.full(n_shared, T, dtype=np.int64)])
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    # A stable sort by expert keeps (token, slot) order, i.e. token order
    # within each expert since a token picks an expert at most once.
    kept = np.nonzero(keep)[0]                         # flat (token, slot) positions kept
    order = kept[np.argsort(local[kept], kind="stable")]
    dest_flat = np.full(T * k, -1, dtype=np.int64)
    dest_flat[order] = np.arange(order.size)
    dest = dest_flat.reshape(T, k)
    R = int(offsets[-1])
    src_row = np.empty(R, dtype=np.int64)
    src_row[dest_flat[kept]] = kept // k
    for s in range(n_shared):
        base = int(offsets[L + s])
        src_row[base:base + T] = np.arange(T)
    return (counts.astype(np.int32), offsets.astype(np.int32),
            dest.astype(np.int32), src_row.astype(np.int32))


def permute_rows(x: np.ndarray, src_row: np.ndarray) -> np.ndarray:
    """x_perm[r] = x[src_row[r]]: the dispatch copy into expert-contiguous groups."""
    return x[src_row]


# ------------------------------------------------------------ expert FFN ----
def expert_weights_f32(inputs: dict, e: int):
    """fp32 values of expert e's (W_gate [I,H], W_up [I,H], W_down [H,I]).

    bf16 weights widen exactly; fp8 weights are code value * block scale
    (DeepSeek-deployment page, Quantization: one scale per 128x128 block);
    mxfp8 weights are code value * 2^(E8M0 - 127) per 32 values along K.
    """
    if inputs["wdtype"] == "fp8":
        return (dequantize_blocks_128x128(inputs["w_gate"][e], inputs["s_gate"][e]),
                dequantize_blocks_128x128(inputs["w_up"][e], inputs["s_up"][e]),
                dequantize_blocks_128x128(inputs["w_down"][e], inputs["s_down"][e]))
    if inputs["wdtype"] == "mxfp8":   # rows of [N, K], blocks of 32 along K
        return (mx_dequantize_rows(inputs["w_gate"][e], inputs["s_gate"][e]),
                mx_dequantize_rows(inputs["w_up"][e], inputs["s_up"][e]),
                mx_dequantize_rows(inputs["w_down"][e], inputs["s_down"][e]))
    return (bf16_bits_to_f32(inputs["w_gate"][e]), bf16_bits_to_f32(inputs["w_up"][e]),
            bf16_bits_to_f32(inputs["w_down"][e]))


def quantize_act(v: np.ndarray, wdtype: str) -> np.ndarray:
    """Values an activation matrix [rows, C] takes as a GEMM operand.

    bf16: itself.  fp8: quantised per row per 128 channels (DeepSeek-deployment
    page, Quantization).  mxfp8: MXFP8 per row, blocks of 32 (oracle/mx.py).
    """
    if wdtype == "fp8":
        return dequantize_groups_128(*quantize_groups_128(v))
    if wdtype == "mxfp8":
        return mx_dequantize_rows(*mx_quantize_rows(v))
    return v


def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z * sigmoid(z) = z / (1 + exp(-z)), fp32."""
    with np.errstate(over="ignore"):
        return (z / (F32(1.0) + np.exp(-z))).astype(F32)


def expert_ffn(X: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray,
               quantize_h=False) -> np.ndarray:
    """One expert on its rows: h = silu(X Wg^T) * (X Wu^T); y = h Wd^T (fp32).

    SwiGLU as fused into the grouped matmul (Qwen3.5-397B on Ironwood, section
    4.2.2: gate and up projections, then swiglu(gate, up)).  For fp8 layers h
    is quantised per row per 128 channels before the down projection, as the
    DeepSeek-deployment page's SiLU kernel block-quantises its output
    (Quantization section); for mxfp8 layers (quantize_h="mxfp8") h is MXFP8
    per row like every MX GEMM operand.
    """
    G = np.matmul(X, wg.T, dtype=F32)
    U = np.matmul(X, wu.T, dtype=F32)
    h = (silu(G) * U).astype(F32)
    if quantize_h:   # True (fp8, the historical flag) or a weight dtype name
        h = quantize_act(h, "fp8" if quantize_h is True else quantize_h)
    return np.matmul(h, wd.T, dtype=F32)


def grouped_ffn(x_perm: np.ndarray, offsets: np.ndarray, inputs: dict) -> np.ndarray:
    """y_perm[rows of e] = expert_ffn_e(x_perm[rows of e]) for every non-empty group."""
    R = x_perm.shape[0]
    H = inputs["w_down"].shape[1]
    y = np.zeros((R, H), dtype=F32)
    n_groups = offsets.shape[0] - 1
    for e in range(n_groups):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        wg, wu, wd = expert_weights_f32(inputs, e)
        y[lo:hi] = expert_ffn(x_perm[lo:hi], wg, wu, wd, quantize_h=_h_quant(inputs["wdtype"]))
    return y


def _h_quant(wdtype: str):
    return wdtype if wdtype in ("fp8", "mxfp8") else False


# --------------------------------------------------------------- combine ----
def combine(y_perm: np.ndarray, dest: np.ndarray, w: np.ndarray, n_shared: int = 0,
            shared_base=None) -> np.ndarray:
    """out[t] = sum_{j ascending, dest[t,j] >= 0} w[t,j] * y_perm[dest[t,j]] (+ shared rows), fp32.

    "CuTeDSL at Perplexity", local combine: weighted accumulation using the
    offsets dispatch computed; pairs routed to another GPU's experts (dest < 0)
    add nothing (same page: the local combine sums the local copies of a token
    before the all-reduce).  The shared expert's output (rows shared_base + t,
    by default T*k + t) is added with weight 1 after the routed sum
    (DeepSeek-deployment page, Expert parallelism section).  Each step is one
    fp32 product then one fp32 add.
    """
    T, k = dest.shape
    base = T * k if shared_base is None else int(shared_base)
    out = np.zeros((T, y_perm.shape[1]), dtype=F32)
    for j in range(k):
        sel = dest[:, j] >= 0
        term = (w[sel, j:j + 1].astype(F32) * y_perm[dest[sel, j]]).astype(F32)
        out[sel] = (out[sel] + term).astype(F32)
    for s in range(n_shared):
        out = (out + y_perm[base + s * T + np.arange(T)]).astype(F32)
    return out


# --------------------------------------------------------------- forward ----
class OracleResult(dict):
    """Intermediates of one oracle forward (attribute access for convenience)."""
    __getattr__ = dict.__getitem__


def forward(inputs: dict, logits_override=None) -> OracleResult:
    """The whole layer on the CPU.

    inputs: dict from synth.to_numpy_inputs (bf16 as uint16 bit patterns).
    logits_override: route from these fp32 logits instead of recomputing them
    (used to evaluate the layer under the GPU's own routing at near-ties).
    inputs["e_first"], inputs["e_local"] (optional): the expert-parallel share
    (counting_sort); the expert weights then hold the share's groups only.
    """
    x = bf16_bits_to_f32(inputs["x_bf16"])
    T, H = x.shape
    E = inputs["w_router"].shape[0]
    k, ns = inputs["k"], inputs["n_shared"]
    e_first, e_local = inputs.get("e_first", 0), inputs.get("e_local", 0)
    logits = (router_logits(x, inputs["w_router"], inputs.get("router_bias"))
              if logits_override is None else np.asarray(logits_override, dtype=F32))
    idx, w = topk_softmax(logits, k)
    counts, offsets, dest, src_row = counting_sort(idx, E, ns, e_first, e_local)
    if inputs["wdtype"] == "fp8":
        # Activations quantised on the fly per token per 128 channels
        # (DeepSeek-deployment page, Quantization section).
        xc, xs = quantize_groups_128(x)
        x_perm_codes, x_perm_scales = xc[src_row], xs[src_row]
        x_perm = dequantize_groups_128(x_perm_codes, x_perm_scales)
    elif inputs["wdtype"] == "mxfp8":
        # MXFP8 activations per token, blocks of 32 channels.
        xc, xs = mx_quantize_rows(x)
        x_perm_codes, x_perm_scales = xc[src_row], xs[src_row]
        x_perm = mx_dequantize_rows(x_perm_codes, x_perm_scales)
    else:
        x_perm_codes = x_perm_scales = None
        x_perm = permute_rows(x, src_row)
    y_perm = grouped_ffn(x_perm, offsets, inputs)
    out = combine(y_perm, dest, w, ns, shared_base=offsets[len(offsets) - 1 - ns])
    return OracleResult(logits=logits, topk_idx=idx, topk_w=w, counts=counts, offsets=offsets,
                        dest=dest, src_row=src_row, x_perm=x_perm, x_perm_codes=x_perm_codes,
                        x_perm_scales=x_perm_scales, y_perm=y_perm, out=out)



def forward_tokens(inputs: dict, tokens, logits_override=None) -> OracleResult:
    """The layer's output for a sample of tokens, evaluated one token at a time.

    Each token's output depends only on its own row: its router logits, its
    top-k and weights, and its experts' FFN of its own (for fp8: own quantised)
    row, combined in slot order with the shared expert added last.  This is
    the combine of "CuTeDSL at Perplexity" (local combine) written per token,
    without the permutation, so the large workloads can be checked on sampled
    outputs.  `logits_override` holds the logits of the sampled tokens only.
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    n = len(tokens)
    x = bf16_bits_to_f32(inputs["x_bf16"][tokens])
    k, ns = inputs["k"], inputs["n_shared"]
    E = inputs["w_router"].shape[0]
    e_first = inputs.get("e_first", 0)
    L = inputs.get("e_local", 0) or E               # routed experts of this share
    logits = (router_logits(x, inputs["w_router"], inputs.get("router_bias"))
              if logits_override is None else np.asarray(logits_override, dtype=F32))
    idx, w = topk_softmax(logits, k)
    hq = _h_quant(inputs["wdtype"])
    x = quantize_act(x, inputs["wdtype"])
    H = x.shape[1]
    y = np.zeros((n, k + ns, H), dtype=F32)       # expert output of each (token, slot)
    local = (idx >= e_first) & (idx < e_first + L)  # pairs routed to this share's experts
    for e in sorted(set(idx[local].tolist())):
        rows, slots = np.nonzero(idx == e)
        y[rows, slots] = expert_ffn(x[rows], *expert_weights_f32(inputs, e - e_first), quantize_h=hq)
    for s_ in range(ns):
        y[:, k + s_] = expert_ffn(x, *expert_weights_f32(inputs, L + s_), quantize_h=hq)
    out = np.zeros((n, H), dtype=F32)
    for j in range(k):
        sel = local[:, j]
        out[sel] = (out[sel] + (w[sel, j:j + 1] * y[sel, j]).astype(F32)).astype(F32)
    for s_ in range(ns):
        out = (out + y[:, k + s_]).astype(F32)
    return OracleResult(tokens=tokens, logits=logits, topk_idx=idx, topk_w=w, out=out)
