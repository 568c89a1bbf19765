"""Algorithmic work of the MoE layer and of each kernel launch (host logic).

Cost model of a grouped GEMM ("Lower latency and higher throughput with
multi-node DeepSeek deployment", Roofline / GroupGEMM section): g groups of
[m, k] x [k, n] cost 2*g*m*k*n FLOPs and move g*(m*k + n*k + m*n) elements.
Here every group has its own m (the realised routing), and only groups with
at least one row count: an expert that receives no token is never read,
which is the point the same page makes about the number of activated experts.

Bytes are ALGORITHMIC: what the step must read and write at least (weights
of touched experts, activations in, results out), not what a kernel happens
to move.
"""
import math
from dataclasses import dataclass

import numpy as np

# MI355X published peaks (dense, no sparsity).
PEAK_HBM_GBS = 8000.0
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "mxfp8": 5000.0, "fp32": 157.3}

# Split of the grouped-FFN schedule, the same rule as the C++ schedule
# (csrc/ffn.hpp skinny_max_rows): groups of up to 64 rows go to the
# weight-streaming kernels when T <= 64 (no group can be larger), else groups of
# up to 48 rows; larger groups go to the tiled kernels.
SKINNY_MAX_ROWS = 64


def skinny_max_rows(T: int) -> int:
    return SKINNY_MAX_ROWS if T <= SKINNY_MAX_ROWS else 48


def tokens_per_expert(T: int, k: int, E: int) -> float:
    """Mean rows per expert when T tokens each pick k of E experts."""
    return T * k / E


def ep_tokens_per_expert(batch: int, qlen: int, k: int, ep: int, E: int) -> float:
    """Mean rows per expert under expert parallelism over `ep` GPUs holding E experts
    with `batch` requests of `qlen` query tokens per GPU."""
    return batch * qlen * k * ep / E


def groupgemm_flops(g: int, m: int, k: int, n: int) -> int:
    return 2 * g * m * k * n


def groupgemm_io_elements(g: int, m: int, k: int, n: int) -> int:
    return g * (m * k + n * k + m * n)


def fp8_scale_shapes(M: int, K: int, N: int):
    """Scale shapes of a block-quantised (M, K) x (K, N) product: activation scales
    [M, ceil(K/128)] and weight scales [ceil(K/128), ceil(N/128)]."""
    kb = math.ceil(K / 128)
    return (M, kb), (kb, math.ceil(N / 128))


@dataclass
class Work:
    bytes: float
    flops: float
    groups: int


def _elt(wdtype: str) -> int:
    return 1 if wdtype in ("fp8", "mxfp8") else 2


def _scale_bytes(rows: float, cols: int, wdtype: str) -> float:
    """Scale bytes of a [rows, cols] operand quantised along cols: fp8 one fp32
    per 128 values of a row; mxfp8 one E8M0 byte per 32."""
    if wdtype == "fp8":
        return rows * (cols // 128) * 4
    if wdtype == "mxfp8":
        return rows * (cols // 32)
    return 0.0


def _weight_scale_bytes(g: int, n: int, k: int, wdtype: str) -> float:
    """Scale bytes of g weight matrices [n, k]: fp8 one fp32 per 128 x 128 block,
    mxfp8 one E8M0 byte per 32 values of a row along k."""
    if wdtype == "fp8":
        return g * (n // 128) * (k // 128) * 4
    return _scale_bytes(g * n, k, wdtype)


def kernel_groups(kernel: str, counts: np.ndarray, skinny_max: int = SKINNY_MAX_ROWS) -> np.ndarray:
    """Group sizes a grouped-FFN launch processes, from its name."""
    m = np.asarray(counts, dtype=np.int64)
    m = m[m > 0]
    if kernel.startswith("skinny_"):
        return m[m <= skinny_max]
    if kernel.startswith("tiled_"):
        return m[m > skinny_max]
    raise ValueError(f"not a grouped-FFN kernel: {kernel}")


def kernel_work(kernel: str, counts: np.ndarray, H: int, I: int, wdtype: str,
                skinny_max: int = SKINNY_MAX_ROWS) -> Work:
    """Algorithmic bytes and FLOPs of one launch of a grouped-FFN kernel
    (skinny_max: the schedule's split, skinny_max_rows(T))."""
    m = kernel_groups(kernel, counts, skinny_max).astype(np.float64)
    e = _elt(wdtype)
    rows = float(m.sum())
    g = len(m)
    if "_gateup_" in kernel:
        w = g * 2 * I * H * e + 2 * _weight_scale_bytes(g, I, H, wdtype)
        a = rows * H * e + _scale_bytes(rows, H, wdtype)
        o = rows * I * e + _scale_bytes(rows, I, wdtype)
        return Work(w + a + o, 4.0 * rows * I * H, g)
    if "_down_" in kernel:
        w = g * H * I * e + _weight_scale_bytes(g, H, I, wdtype)
        a = rows * I * e + _scale_bytes(rows, I, wdtype)
        o = rows * H * 2
        return Work(w + a + o, 2.0 * rows * H * I, g)
    raise ValueError(f"not a grouped-FFN kernel: {kernel}")


def layer_work(T: int, H: int, E: int, k: int, I: int, n_shared: int, wdtype: str,
               counts: np.ndarray) -> Work:
    """Algorithmic bytes / FLOPs of one layer call: weights of touched experts
    (and their block scales), the router weight, x in and out.  `counts` are
    the rows of the groups held here (routed, then shared); for an
    expert-parallel share they cover its experts only."""
    m = np.asarray(counts, dtype=np.int64)
    touched = int((m > 0).sum())
    e = _elt(wdtype)
    wbytes = touched * 3 * H * I * e
    wbytes += 2 * _weight_scale_bytes(touched, I, H, wdtype) + _weight_scale_bytes(touched, H, I, wdtype)
    byts = wbytes + 4 * H * E + T * H * 2 + T * H * 2
    R = int(m.sum())
    flops = 2 * T * H * E + 2 * R * 3 * H * I
    return Work(float(byts), float(flops), touched)


def roofline(work: Work, seconds: float, dtype: str):
    """Binding roofline of a launch: HBM if its arithmetic intensity is below the ridge."""
    ridge = PEAK_TFLOPS[dtype] * 1e12 / (PEAK_HBM_GBS * 1e9)
    ai = work.flops / max(work.bytes, 1.0)
    if ai < ridge:
        ach = work.bytes / seconds / 1e9
        return {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": ach / PEAK_HBM_GBS}
    ach = work.flops / seconds / 1e12
    return {"bound": "mfma", "achieved": ach, "peak": PEAK_TFLOPS[dtype], "unit": "TFLOP/s",
            "frac": ach / PEAK_TFLOPS[dtype]}
