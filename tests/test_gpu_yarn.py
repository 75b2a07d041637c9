"""GPU: the YaRN-extended decoupled RoPE (mla_dims yarn_* fields) against the oracle.

The rotation stage is compared on positions far past the original context, and whole decode
steps (V2 shape with a bf16 cache and κ-stress; the running model in float32) are compared with
the oracle's explicit step using the same frequencies and score temperature.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import mla_latent_kv_25_amd as mla  # noqa: E402
from oracle import rope  # noqa: E402
from synth import get_config, make_case  # noqa: E402

from gpu_helpers import TOL, check_u, rel_l2, run_gpu, run_oracle  # noqa: E402

YARN = dict(yarn_factor=40.0, yarn_orig_len=4096, yarn_alpha=1.0, yarn_beta=32.0)


def _yarn_cfg(key, stress=False):
    cfg = get_config(key, stress=stress)
    return cfg.with_(dims=replace(cfg.dims, **YARN))


def test_yarn_rope_stage():
    """q^R of every head and the shared k^R, rotated in place by mla_rope, at positions up to 2^17."""
    dims = replace(get_config("2").dims, **YARN)
    d = mla.Dims.of(dims)
    lens = torch.tensor([1, 100, 4096, 70001, 131072], dtype=torch.int32, device="cuda")
    B = lens.numel()
    g = torch.Generator(device="cpu").manual_seed(5)
    q_pe = torch.randn((B, dims.n_h, dims.d_r), generator=g).cuda()
    kv = torch.randn((B, dims.d_c + dims.d_r), generator=g).cuda()
    q0, k0 = q_pe.double().cpu().numpy(), kv.double().cpu().numpy()
    mla.rope(d, lens, q_pe, kv)
    torch.cuda.synchronize()
    yarn = (YARN["yarn_factor"], YARN["yarn_orig_len"], YARN["yarn_alpha"], YARN["yarn_beta"])
    for b in range(B):
        pos = int(lens[b]) - 1
        q_ref = rope(q0[b], pos, dims.rope_base, yarn)
        k_ref = rope(k0[b, dims.d_c:], pos, dims.rope_base, yarn)
        eq = rel_l2(q_pe[b].double().cpu().numpy(), q_ref)
        ek = rel_l2(kv[b, dims.d_c:].double().cpu().numpy(), k_ref)
        print(f"pos {pos}: q^R rel-L2 {eq:.2e}, k^R rel-L2 {ek:.2e}", flush=True)
        assert eq < 1e-6 and ek < 1e-6
        # the latent part is untouched
        assert torch.equal(kv[b, :dims.d_c].cpu(), torch.from_numpy(k0[b, :dims.d_c]).float())


@pytest.mark.parametrize("key,B,T,stress", [
    ("0", 1, [64], False),
    ("2", 3, [300, 1, 77], True),
    ("3", 2, [700, 129], True),
])
def test_yarn_decode_step(key, B, T, stress):
    cfg = _yarn_cfg(key, stress)
    case = make_case(cfg, device="cuda", B=B, T=T)
    print(f"case cfg={key} B={B} T={T} cdtype={cfg.cdtype} yarn={YARN}", flush=True)
    step, _ = run_gpu(case, 0)
    ref = run_oracle(case)
    u_ref = np.stack([ref[b]["u"] for b in range(B)])
    check_u(step.u.double().cpu().numpy(), u_ref, cfg.cdtype, f"yarn cfg{key}")
    lse_ref = np.stack([ref[b]["lse"] for b in range(B)])
    err = float(np.max(np.abs(step.lse.double().cpu().numpy() - lse_ref)))
    assert err <= (1e-4 if cfg.cdtype == "f32" else TOL[cfg.cdtype][1]), err
