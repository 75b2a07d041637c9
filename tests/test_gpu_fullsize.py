"""GPU parity at the full workload sizes, in the launch configuration bench.py times (one range per
compute unit), on sampled outputs the oracle can compute one by one.

Every config runs its whole decode step on the GPU through the C ABI. The oracle is then run on a
few sampled sequences, with explicit K/V reconstruction: the first, the last and one in between,
or the shortest and longest of a ragged batch. For the long contexts only a few sampled heads
are checked (o_lat, lse), because u needs every head.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from oracle import OracleDims, decode_step_explicit  # noqa: E402
from synth import get_config, make_case  # noqa: E402

from gpu_helpers import TOL, check_u, oracle_prefix, rel_l2, run_gpu, weights64  # noqa: E402


def _oracle(case, b, heads=None, want_u=True):
    W = weights64(case)
    od = OracleDims.of(case.dims)
    return decode_step_explicit(W, case.h[b].double().cpu().numpy(), oracle_prefix(case, b), od,
                                case.cfg.cdtype, heads=heads, want_u=want_u)


def _check_heads(step, case, b, ref, heads, label):
    cd = case.cfg.cdtype
    tol_o = 1e-4 if cd == "f32" else 5e-3
    tol_l = 1e-4 if cd == "f32" else 2e-2
    o = step.o_lat[b, heads].double().cpu().numpy()
    lse = step.lse[b, heads].double().cpu().numpy()
    eo = rel_l2(o, ref["o_lat"])
    el = float(np.max(np.abs(lse - ref["lse"])))
    hs = f"{len(heads)} heads" if len(heads) > 8 else f"heads {heads}"
    print(f"{label} b={b} T={int(case.seq_lens[b])} {hs}: o_lat rel-L2 {eo:.3e}, lse max-abs {el:.3e}", flush=True)
    assert eo <= tol_o and el <= tol_l, (label, b, eo, el)


@pytest.mark.parametrize("stress", [False, True], ids=["plain", "stress"])
def test_fullsize_config2(stress):
    """B=64, T=4096, contiguous bf16: u, o_lat and lse of three sampled sequences."""
    case = make_case(get_config("2", stress=stress), device="cuda")
    step, _ = run_gpu(case, 0)
    for b in (0, 37, case.B - 1):
        ref = _oracle(case, b)
        check_u(step.u[b].double().cpu().numpy(), ref["u"], case.cfg.cdtype, f"cfg2 b={b}")
        _check_heads(step, case, b, {"o_lat": ref["o_lat"], "lse": ref["lse"]}, list(range(case.dims.n_h)), "cfg2")


def test_fullsize_config1():
    """B=32, T=4096, running dims, fp16 storage: u of two sampled sequences."""
    case = make_case(get_config("1"), device="cuda")
    step, _ = run_gpu(case, 0)
    for b in (0, case.B - 1):
        ref = _oracle(case, b)
        check_u(step.u[b].double().cpu().numpy(), ref["u"], case.cfg.cdtype, f"cfg1 b={b}")


def test_fullsize_config3():
    """B=128 ragged T in [1024, 32768], 64-token pages: shortest and longest sequence."""
    case = make_case(get_config("3"), device="cuda")
    step, _ = run_gpu(case, 0)
    lens = case.seq_lens.cpu().numpy()
    b_short, b_long = int(np.argmin(lens)), int(np.argmax(lens))
    ref = _oracle(case, b_short)
    check_u(step.u[b_short].double().cpu().numpy(), ref["u"], case.cfg.cdtype, f"cfg3 b={b_short}")
    heads = [0, 57, 127]
    ref = _oracle(case, b_long, heads=heads, want_u=False)
    _check_heads(step, case, b_long, ref, heads, "cfg3")


@pytest.mark.parametrize("key", ["4", "4f8"])
def test_fullsize_config4(key):
    """B=4, T=131072 (bf16 and fp8 e4m3 caches): sampled heads of two sequences."""
    case = make_case(get_config(key), device="cuda")
    step, _ = run_gpu(case, 0)
    heads = [0, 101]
    for b in (0, case.B - 1):
        ref = _oracle(case, b, heads=heads, want_u=False)
        _check_heads(step, case, b, ref, heads, f"cfg{key}")
