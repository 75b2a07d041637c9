"""The no-allocation entry point (mla_absorb_out_noalloc) against mla_absorb_out through the C ABI.

Two calls in a row share the library's static scratch; the second has a smaller batch, so stale
contents of the first call's partial sums must not leak into it. Each result is compared with the
workspace entry point's on the same inputs (the same kernels, so the bar is bitwise equality,
well inside the float32 / bf16 parity bars of the rest of the suite)."""
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import mla_latent_kv_25_amd as mla  # noqa: E402
from synth import get_config, make_case  # noqa: E402


def _inputs(key, B):
    case = make_case(get_config(key), device="cuda", B=B, T=2)
    g = torch.Generator(device="cuda")
    g.manual_seed(4242 + B)
    o_lat = torch.randn((B, case.dims.n_h, case.dims.d_c), generator=g, device="cuda", dtype=torch.float32)
    return case, o_lat


@pytest.mark.parametrize("key", ["2", "1", "0"])
def test_absorb_out_noalloc_matches_workspace_call(key):
    for B in (64, 16) if key != "0" else (5, 2):
        case, o_lat = _inputs(key, B)
        print(f"case cfg={key} B={B} entry=mla_absorb_out_noalloc", flush=True)
        step = mla.DecodeStep(case.dims, B, 0)
        W = case.weights
        u_ref = torch.empty((B, case.dims.d), dtype=torch.float32, device="cuda")
        u_na = torch.full((B, case.dims.d), float("nan"), dtype=torch.float32, device="cuda")
        mla.absorb_out(step.dims, o_lat, W["W_uv"], W["W_o"], step.ws_o, u_ref)
        mla.absorb_out_noalloc(step.dims, o_lat, W["W_uv"], W["W_o"], u_na)
        torch.cuda.synchronize()
        assert torch.isfinite(u_na).all()
        assert torch.equal(u_na, u_ref), float((u_na - u_ref).abs().max())


def test_absorb_out_noalloc_rejects_oversized_batch():
    case = make_case(get_config("2"), device="cuda", B=1, T=2)
    d = mla.Dims.of(case.dims)
    B = 256
    o_lat = torch.zeros((B, 128, 512), dtype=torch.float32, device="cuda")
    u = torch.zeros((B, 5120), dtype=torch.float32, device="cuda")
    with pytest.raises(mla.MLAError, match="scratch"):
        mla.absorb_out_noalloc(d, o_lat, case.weights["W_uv"], case.weights["W_o"], u)
