"""The five seeded synthetic layer shapes used for parity and measurement.

Shapes and distributions:
- Qwen3-235B-like: 128 experts, top-8 ("Hosting Qwen on Blackwell", Prefillers
  section: 6000 * 8 / 128 tokens per expert); hidden 4096, intermediate 1536.
- Qwen3.5-397B-like: hidden 4096 (xxmr.cn Qwen3.5-397B on Ironwood, section
  1.1), 512 experts (section 3.1), top-10 over 1024 tokens (the [1024,10]
  routing tensors of section 3.2.1); intermediate 1024; router logits carry a
  Zipf(1.1) per-expert popularity term.
- DeepSeek-V3-like: 256 routed experts + 1 shared expert, top-8, shared output
  added ("Lower latency and higher throughput with multi-node DeepSeek
  deployment", Expert parallelism section); FP8 with 128-element activation
  groups and 128x128 weight blocks (same page, Quantization section).
"""
from dataclasses import dataclass
from typing import Optional


@dataclass(frozen=True)
class MoeConfig:
    name: str
    seed: int
    T: int          # tokens
    H: int          # hidden size (GEMM K of gate/up, N of down)
    E: int          # routed experts
    k: int          # experts per token
    I: int          # SwiGLU intermediate size
    n_shared: int = 0           # always-on shared experts (0 or 1)
    wdtype: str = "bf16"        # "bf16", "fp8" (e4m3fn codes + fp32 128x128 block scales) or
                                # "mxfp8" (e4m3fn codes + E8M0 scales per 32 along K)
    zipf_s: Optional[float] = None  # Zipf exponent of the per-expert router-logit bias
    w_std: float = 0.02
    router_std: float = 0.02
    regime: str = ""            # which roofline binds: "launch", "hbm", "mfma"
    # Expert-parallel share: this GPU holds routed experts [e_first,
    # e_first + e_local) of the E (e_local = 0: all of them) and sees every
    # token (replicated input); its output is the partial sum over its experts.
    e_first: int = 0
    e_local: int = 0

    @property
    def R(self) -> int:
        """Upper bound on the rows of the permuted activation matrix (routed + shared)."""
        return self.T * self.k + self.T * self.n_shared

    @property
    def E_loc(self) -> int:
        """Routed experts held by this GPU."""
        return self.e_local or self.E

    @property
    def n_groups(self) -> int:
        return self.E_loc + self.n_shared


CONFIGS = [
    MoeConfig("tiny", 0, T=64, H=256, E=8, k=2, I=512, regime="launch"),
    MoeConfig("qwen3_235b_decode", 1, T=64, H=4096, E=128, k=8, I=1536, regime="hbm"),
    MoeConfig("qwen3_235b_prefill", 2, T=8192, H=4096, E=128, k=8, I=1536, regime="mfma"),
    MoeConfig("qwen35_397b_zipf", 3, T=1024, H=4096, E=512, k=10, I=1024, zipf_s=1.1, regime="hbm"),
    MoeConfig("deepseek_v3_fp8", 4, T=4096, H=7168, E=256, k=8, I=2048, n_shared=1,
              wdtype="fp8", regime="hbm"),
]


# Further workloads (not among the five above): the Qwen3-235B-like layer with
# MXFP8 experts, as "Hosting Qwen on Blackwell" (Quantization) deploys it, and
# expert-parallel shares (one GPU's experts, every token:
# "CuTeDSL at Perplexity", MoE Dispatch/Combine, tensor-parallel deployment):
# EP8 at the decode batch (16 experts, about 4 rows each) and EP4 at the
# prefill chunk ("Hosting Qwen on Blackwell" runs its prefill EP on 4 GPUs).
EXTRA_CONFIGS = [
    MoeConfig("qwen3_235b_decode_mxfp8", 5, T=64, H=4096, E=128, k=8, I=1536, wdtype="mxfp8",
              regime="hbm"),
    MoeConfig("qwen3_235b_prefill_mxfp8", 6, T=8192, H=4096, E=128, k=8, I=1536, wdtype="mxfp8",
              regime="mfma"),
    MoeConfig("qwen3_235b_decode_ep8", 7, T=64, H=4096, E=128, k=8, I=1536, e_first=16, e_local=16,
              regime="hbm"),
    MoeConfig("qwen3_235b_prefill_ep4", 8, T=8192, H=4096, E=128, k=8, I=1536, e_first=32,
              e_local=32, regime="mfma"),
    # 8-bit decode shares: the DeepSeek-like layer's 16 routed experts of an
    # EP16 deployment at a 64-token decode batch (fp8), and the MXFP8
    # Qwen3-235B-like layer's EP8 share.
    MoeConfig("deepseek_v3_decode_ep16", 9, T=64, H=7168, E=256, k=8, I=2048, wdtype="fp8",
              e_first=32, e_local=16, regime="hbm"),
    MoeConfig("qwen3_235b_decode_mxfp8_ep8", 10, T=64, H=4096, E=128, k=8, I=1536, wdtype="mxfp8",
              e_first=16, e_local=16, regime="hbm"),
]


def config_by_name(name: str) -> MoeConfig:
    for c in CONFIGS + EXTRA_CONFIGS:
        if c.name == name:
            return c
    raise KeyError(f"unknown config {name!r}; known: {[c.name for c in CONFIGS]}")
