"""The five decode workloads (plus their fp8 and kappa-stress variants) as plain data.

Dimensions follow the two models on the pages:
  * the running model of "DeepSeek-V2 from Scratch" (section "The Running Model"):
    d=512, n_h=8, d_h=64, d_c=128, d_c'=96, d_h^R=32;
  * the DeepSeek-V2 production shape (same page, section 7, and the summary page's
    "MLA: joint low-rank compression"): d=5120, n_h=128, d_h=128, d_c=512, d_c'=1536, d_h^R=64.
"""
from dataclasses import dataclass, field, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class Dims:
    d: int        # hidden size
    n_h: int      # attention heads
    d_h: int      # per-head content dimension
    d_c: int      # KV latent width
    d_cq: int     # query latent width (d_c')
    d_r: int      # decoupled rotary width (d_h^R)
    rope_base: float = 10000.0
    # YaRN extension of the decoupled RoPE (factor <= 1: off); parameters are the caller's
    yarn_factor: float = 1.0
    yarn_orig_len: int = 0
    yarn_alpha: float = 0.0
    yarn_beta: float = 0.0

    @property
    def row(self) -> int:
        """Elements per cached token: latent followed by the rotary key."""
        return self.d_c + self.d_r


RUNNING_DIMS = Dims(d=512, n_h=8, d_h=64, d_c=128, d_cq=96, d_r=32)
V2_DIMS = Dims(d=5120, n_h=128, d_h=128, d_c=512, d_cq=1536, d_r=64)

# storage type names used across the repository
STORAGE = ("f32", "f16", "bf16", "fp8_e4m3", "fp6_e2m3")


@dataclass(frozen=True)
class Config:
    key: str
    title: str
    dims: Dims
    wdtype: str                  # weights and hidden states
    cdtype: str                  # latent cache rows
    batch: int
    lens: Tuple                  # ("fixed", T) or ("uniform", lo, hi) inclusive
    layout: str = "contiguous"   # or "paged"
    page_size: int = 64
    sigma_h: float = 0.02
    sigma_w: float = 0.02
    kappa: float = 1.0           # scale on W^UQ and W^QR (score-stress variants)
    seed: int = 1000

    @property
    def sigma_row(self) -> float:
        """Std of a prefix cache element: a projection of h by an N(0, sigma_w) matrix has
        std sigma_w * sigma_h * sqrt(d); a rotation keeps that std for the rotary part."""
        return self.sigma_w * self.sigma_h * (self.dims.d ** 0.5)

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


CONFIGS = {
    "0": Config("0", "running-model decode, fp32, B=1, T=64", RUNNING_DIMS, "f32", "f32",
                1, ("fixed", 64), seed=1000),
    "1": Config("1", "running-model decode, fp16 storage, B=32, T=4096", RUNNING_DIMS, "f16", "f16",
                32, ("fixed", 4096), seed=1001),
    "2": Config("2", "DeepSeek-V2 shape decode, bf16, B=64, T=4096, contiguous", V2_DIMS, "bf16", "bf16",
                64, ("fixed", 4096), sigma_h=1.0, sigma_w=0.006, seed=1002),
    "3": Config("3", "DeepSeek-V2 shape, ragged T~U[1024,32768], 64-token pages, bf16", V2_DIMS, "bf16", "bf16",
                128, ("uniform", 1024, 32768), layout="paged", sigma_h=1.0, sigma_w=0.006, seed=1003),
    "4": Config("4", "DeepSeek-V2 shape long context, B=4, T=131072, bf16 cache", V2_DIMS, "bf16", "bf16",
                4, ("fixed", 131072), sigma_h=1.0, sigma_w=0.006, seed=1004),
    "4f8": Config("4f8", "DeepSeek-V2 shape long context, B=4, T=131072, fp8 e4m3 cache + per-token scale",
                  V2_DIMS, "bf16", "fp8_e4m3", 4, ("fixed", 131072), sigma_h=1.0, sigma_w=0.006, seed=1005),
    # the ~6-bit cache: e2m3 codes packed 6 bits each (432 bytes per row) + one float32 scale per token
    "4f6": Config("4f6", "DeepSeek-V2 shape long context, B=4, T=131072, fp6 e2m3 cache (6 bits + per-token scale)",
                  V2_DIMS, "bf16", "fp6_e2m3", 4, ("fixed", 131072), sigma_h=1.0, sigma_w=0.006, seed=1006),
}

# kappa for the score-stress variants: W^UQ and W^QR are scaled by kappa so that the scaled scores
# have a standard deviation near 2 (at the configs' own distributions the softmax is close to
# uniform, so parity on u alone would barely test the score path). With all entries independent:
#   std(c^Q) = s_w s_h sqrt(d);  std(q^C) = std(q^R) = kappa s_w std(c^Q) sqrt(d_cq)
#   std(c^KV) = std(k^R) = s_w s_h sqrt(d);  std(k^C) = s_w std(c^KV) sqrt(d_c)
#   std(score) = sqrt(d_h std(q^C)^2 std(k^C)^2 + d_r std(q^R)^2 std(k^R)^2) / sqrt(d_h + d_r)
# which is 0.0255 kappa at the V2 shape and 9.7e-6 kappa for the running model.
STRESS_KAPPA = {"0": 2.2e5, "1": 2.2e5, "2": 80.0, "3": 80.0, "4": 80.0, "4f8": 80.0, "4f6": 80.0}


def get_config(key: str, stress: bool = False, **overrides) -> Config:
    cfg = CONFIGS[key]
    if stress:
        cfg = cfg.with_(kappa=STRESS_KAPPA[key])
    if overrides:
        cfg = cfg.with_(**overrides)
    return cfg
