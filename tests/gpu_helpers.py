"""Shared helpers of the GPU parity tests: run a case through the C ABI, run the oracle on the
same stored bytes, compare."""
import numpy as np
import torch

import mla_latent_kv_25_amd as mla
from oracle import OracleDims, decode_step_explicit, quantize_rows_e4m3

TOL = {  # (rel-L2, max-abs) on u
    "f32": (1e-4, 1e-4),
    "f16": (5e-3, 2e-2),
    "bf16": (5e-3, 2e-2),
    "fp8_e4m3": (5e-3, 2e-2),
    "fp6_e2m3": (5e-3, 2e-2),
}


def build_cache(case):
    """Device cache filled with the case's prefix rows (fp8: quantised by the library)."""
    cfg, dims = case.cfg, case.dims
    if cfg.layout == "contiguous":
        cache = mla.LatentCache.contiguous(case.B, case.t_cap, dims.row, cfg.cdtype)
    else:
        cache = mla.LatentCache.paged(case.num_pages, cfg.page_size, dims.row, cfg.cdtype, case.block_table)
    if cfg.cdtype not in ("fp8_e4m3", "fp6_e2m3"):
        cache.rows.copy_(case.rows)
        return cache
    # fp8 / fp6: the library's encoder writes codes + scales from the float32 source rows
    d = mla.Dims.of(dims)
    n_rows = (case.seq_lens - 1).to(torch.int32).contiguous()
    if cfg.layout == "contiguous":
        mla.cache_store(d, cache, n_rows, case.t_cap, case.rows32.contiguous(), case.t_cap)
    else:
        src = torch.stack([torch.nn.functional.pad(case.prefix_rows(b), (0, 0, 0, case.t_cap - int(case.seq_lens[b]) + 1))
                           for b in range(case.B)]).contiguous()
        mla.cache_store(d, cache, n_rows, case.t_cap, src, case.t_cap)
    return cache


def run_gpu(case, num_splits=0, cache=None):
    dims = case.dims
    cache = cache if cache is not None else build_cache(case)
    step = mla.DecodeStep(dims, case.B, num_splits)
    step.run(case.h, case.weights, cache, case.seq_lens)
    torch.cuda.synchronize()
    return step, cache


def oracle_prefix(case, b):
    """The stored prefix rows of sequence b as the oracle reads them (float64)."""
    pre = case.prefix_rows(b)
    if case.cfg.cdtype == "fp8_e4m3":
        codes, scales = quantize_rows_e4m3(pre.float().cpu().numpy())
        from oracle import e4m3_decode
        return e4m3_decode(codes) * scales.astype(np.float64)[:, None]
    if case.cfg.cdtype == "fp6_e2m3":
        from oracle import e2m3_decode, quantize_rows_e2m3
        codes, scales = quantize_rows_e2m3(pre.float().cpu().numpy())
        return e2m3_decode(codes) * scales.astype(np.float64)[:, None]
    return pre.double().cpu().numpy()


def weights64(case):
    return {k: v.double().cpu().numpy() for k, v in case.weights.items()}


def run_oracle(case, seqs=None, heads=None, want_u=True):
    W = weights64(case)
    od = OracleDims.of(case.dims)
    seqs = range(case.B) if seqs is None else seqs
    out = {}
    for b in seqs:
        out[b] = decode_step_explicit(W, case.h[b].double().cpu().numpy(), oracle_prefix(case, b), od,
                                      case.cfg.cdtype, heads=heads, want_u=want_u)
    return out


def rel_l2(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def check_u(u_gpu, u_ref, cdtype, label=""):
    rl, ma = rel_l2(u_gpu, u_ref), float(np.max(np.abs(np.asarray(u_gpu) - u_ref)))
    tr, ta = TOL[cdtype]
    print(f"{label} u rel-L2 {rl:.3e} max-abs {ma:.3e} (|ref|max {np.max(np.abs(u_ref)):.3e})", flush=True)
    assert rl <= tr and ma <= ta, (label, rl, ma)
    return rl, ma
