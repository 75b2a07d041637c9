"""Cache-size arithmetic of the pages — TEST INFRASTRUCTURE ONLY.

Elements cached per token per layer ([Scratch] = "DeepSeek-V2 from Scratch", sections 1, 2, 4.5, 7;
the summary page's "MLA: joint low-rank compression"; the visual page's "How much smaller the
cache gets"):
  MHA: keys and values of every head, 2 n_h d_h
  GQA with g groups: 2 g d_h; MQA is g = 1
  MLA, latent only (the first attempt in section 2): d_c
  MLA with the decoupled rotary key: d_c + d_h^R
  GQA-equivalent group count of MLA: (d_c + d_h^R) / (2 d_h)
"""


def cache_counts(n_h, d_h, d_c, d_r, layers=1, bytes_per_elem=2, gqa_groups=2):
    per = {
        "mha": 2 * n_h * d_h,
        "gqa": 2 * gqa_groups * d_h,
        "mqa": 2 * d_h,
        "mla_latent_only": d_c,
        "mla": d_c + d_r,
    }
    out = {k + "_per_layer": v for k, v in per.items()}
    out.update({k + "_total": v * layers for k, v in per.items()})
    out.update({k + "_bytes": v * layers * bytes_per_elem for k, v in per.items()})
    out["mla_over_mha"] = per["mla"] / per["mha"]
    out["gqa_equivalent_groups"] = (d_c + d_r) / (2 * d_h)
    return out
