"""GPU: mla_combine_absorb_out (the combine fused with the per-head W^UV product) against the
oracle, and against mla_combine + mla_absorb_out on the same decode workspace.

Cases: DeepSeek-V2 shape with bf16, fp8 and fp6 caches (f16 partials), ragged and single-token
contexts, more ranges than tokens, batches that leave the last 32-sequence slice partly empty,
and the full config-2 batch (B = 64) on short contexts.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import mla_latent_kv_25_amd as mla  # noqa: E402
from synth import get_config, make_case  # noqa: E402

from gpu_helpers import build_cache, check_u, rel_l2, run_oracle  # noqa: E402

CASES = [
    # (config, B, lengths, layout override, stress, num_splits)
    ("2", 3, [300, 1, 77], None, True, 4),
    ("2", 2, [3, 40], None, True, 64),
    ("3", 4, [700, 129, 31, 1500], None, True, 7),
    ("4f8", 3, [900, 64, 2], "paged", True, 5),
    ("4f6", 2, [2000, 33], None, True, 3),
    ("2", 33, None, None, False, 0),
]


@pytest.mark.parametrize("key,B,T,layout,stress,splits", CASES,
                         ids=[f"cfg{c[0]}-B{c[1]}-S{c[5]}" for c in CASES])
def test_fused_combine_absorb_out(key, B, T, layout, stress, splits):
    T = T if T is not None else [int(x) for x in np.random.default_rng(5).integers(1, 400, size=B)]
    cfg = get_config(key, stress=stress)
    case = make_case(cfg, device="cuda", B=B, T=T, layout=layout)
    print(f"fused case cfg={key} B={B} T={T[:6]} splits={splits}", flush=True)
    c1, c2 = build_cache(case), build_cache(case)
    s1 = mla.DecodeStep(case.dims, B, splits)
    s2 = mla.DecodeStep(case.dims, B, splits, fused=True)
    u1 = s1.run(case.h, case.weights, c1, case.seq_lens).clone()
    u2 = s2.run(case.h, case.weights, c2, case.seq_lens).clone()
    torch.cuda.synchronize()
    # the per-head outputs o (start of the absorb_out workspace): float32 in the two-call path,
    # bf16 in the fused one; the same sums in another order agree to the bf16 rounding
    nho = B * case.dims.n_h * case.dims.d_h
    o1 = s1.ws_o[: 4 * nho].view(torch.float32).double()
    o2 = s2.ws_o[: 2 * nho].view(torch.bfloat16).double()
    slack = 2.0 ** -8 * o1.abs() + 1e-5 * float(o1.abs().max())
    assert bool(((o2 - o1).abs() <= slack).all()), float(((o2 - o1).abs() - slack).max())
    # u then differs by that rounding only
    assert rel_l2(u2.double().cpu().numpy(), u1.double().cpu().numpy()) < 2e-3
    assert float((s1.lse - s2.lse).abs().max()) <= 1e-6
    if B <= 4:
        ref = run_oracle(case)
        check_u(u2.double().cpu().numpy(), np.stack([ref[b]["u"] for b in range(B)]), case.cfg.cdtype,
                f"fused cfg{key}")


def test_fused_without_lse():
    """lse is optional: NULL skips it and leaves u unchanged."""
    case = make_case(get_config("2"), device="cuda", B=2, T=[50, 9])
    c = build_cache(case)
    s = mla.DecodeStep(case.dims, 2, 3, fused=True)
    u_ref = s.run(case.h, case.weights, c, case.seq_lens).clone()
    u = torch.empty_like(u_ref)
    mla.combine_absorb_out(s.dims, 3, s.ws_d, case.weights["W_uv"], case.weights["W_o"], s.ws_o, u, None)
    torch.cuda.synchronize()
    assert torch.equal(u, u_ref)


def test_fused_zero_length_sequences():
    """Sequences at length 0 (outside the contract, but defined): the fused call gives them u = 0 and
    lse = -inf, as mla_combine + mla_absorb_out do, and the others the two-call results."""
    T = [1, 300, 1, 77, 5, 1]
    empty = [0, 2, 5]
    case = make_case(get_config("2", stress=True), device="cuda", B=len(T), T=T, layout="paged")
    cache = build_cache(case)
    s1 = mla.DecodeStep(case.dims, len(T), 7)
    s1.run(case.h, case.weights, cache, case.seq_lens)
    lens = case.seq_lens.clone()
    lens[empty] = 0
    mla.decode_attn(s1.dims, s1.q_lat, s1.q_pe, cache, lens, 7, s1.ws_d)
    u_f = torch.full_like(s1.u, 7.0)
    lse_f = torch.full_like(s1.lse, 7.0)
    mla.combine_absorb_out(s1.dims, 7, s1.ws_d, case.weights["W_uv"], case.weights["W_o"], s1.ws_o, u_f, lse_f)
    o_lat = torch.empty_like(s1.o_lat)
    lse_u = torch.empty_like(s1.lse)
    u_u = torch.empty_like(s1.u)
    mla.combine(s1.dims, 7, lens, s1.ws_d, o_lat, lse_u)
    mla.absorb_out(s1.dims, o_lat, case.weights["W_uv"], case.weights["W_o"], s1.ws_o, u_u)
    torch.cuda.synchronize()
    for b in range(len(T)):
        if b in empty:
            assert torch.all(u_f[b] == 0) and torch.all(torch.isneginf(lse_f[b])), b
        else:
            assert rel_l2(u_f[b].double().cpu().numpy(), u_u[b].double().cpu().numpy()) < 2e-3, b
            assert float((lse_f[b] - lse_u[b]).abs().max()) <= 1e-6, b
