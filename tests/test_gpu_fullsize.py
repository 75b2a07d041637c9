"""GPU parity at the full workload sizes, in the launch configuration bench.py times (one range per
compute unit), on sampled outputs the oracle can compute one by one.

Every config runs its whole decode step on the GPU through the C ABI (config 2 also with the fused
combine + W^UV call the bench uses). The oracle is then run, with
explicit K/V reconstruction and every head, on sampled sequences: the first, the last and one in
between of config 2; the shortest, the longest and ten more seeded picks of the ragged config 3;
two whole 131,072-token sequences of config 4 (bf16, fp8 and fp6 caches). Each sampled sequence is
compared on u (the step's output) and on o_lat and lse of all its heads.
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


@pytest.mark.parametrize("stress", [False, True], ids=["plain", "stress"])
def test_fullsize_config2_fused(stress):
    """The bench's own step at config 2 (mla_combine_absorb_out in place of the last two calls): u
    of three sampled sequences against the oracle, and every sequence's u and lse against the
    two-call step on the same decode workspace contents."""
    import mla_latent_kv_25_amd as mla
    from gpu_helpers import build_cache
    case = make_case(get_config("2", stress=stress), device="cuda")
    step, cache = run_gpu(case, 0)
    fused = mla.DecodeStep(case.dims, case.B, 0, fused=True)
    fused.run(case.h, case.weights, build_cache(case), case.seq_lens)
    torch.cuda.synchronize()
    assert rel_l2(fused.u.double().cpu().numpy(), step.u.double().cpu().numpy()) < 2e-3
    assert float((fused.lse - step.lse).abs().max()) <= 1e-5
    for b in (0, 37, case.B - 1):
        ref = _oracle(case, b)
        check_u(fused.u[b].double().cpu().numpy(), ref["u"], case.cfg.cdtype, f"cfg2 fused b={b}")


def test_fullsize_config1():
    """B=32, T=4096, running dims, fp16 storage: u of two sampled sequences."""
    case = make_case(get_config("1"), device="cuda")
    step, _ = run_gpu(case, 0)
    for b in (0, case.B - 1):
        ref = _oracle(case, b)
        check_u(step.u[b].double().cpu().numpy(), ref["u"], case.cfg.cdtype, f"cfg1 b={b}")


def config3_sample(lens, n_extra=10, seed=7):
    """Sequences of config 3 checked against the oracle: the shortest, the longest and n_extra more
    drawn without replacement from the rest with a fixed seed."""
    lens = np.asarray(lens)
    b_short, b_long = int(np.argmin(lens)), int(np.argmax(lens))
    rest = [b for b in range(len(lens)) if b not in (b_short, b_long)]
    rng = np.random.default_rng(seed)
    extra = sorted(int(b) for b in rng.choice(rest, size=min(n_extra, len(rest)), replace=False))
    return [b_short, b_long] + extra


def test_fullsize_config3():
    """B=128 ragged T in [1024, 32768], 64-token pages: u, o_lat and lse of 12 sampled sequences
    (the shortest, the longest and ten seeded picks), every head."""
    case = make_case(get_config("3"), device="cuda")
    step, _ = run_gpu(case, 0)
    lens = case.seq_lens.cpu().numpy()
    sample = config3_sample(lens)
    print(f"cfg3 sample {sample} (T = {[int(lens[b]) for b in sample]})", flush=True)
    for b in sample:
        ref = _oracle(case, b)
        check_u(step.u[b].double().cpu().numpy(), ref["u"], case.cfg.cdtype, f"cfg3 b={b}")
        _check_heads(step, case, b, ref, list(range(case.dims.n_h)), "cfg3")


@pytest.mark.parametrize("key", ["4", "4f8", "4f6"])
def test_fullsize_config4(key):
    """B=4, T=131072 (bf16, fp8 e4m3 and fp6 e2m3 caches), split over 64 ranges per sequence: u,
    o_lat and lse of every head of the first and the last sequence."""
    case = make_case(get_config(key), device="cuda")
    step, _ = run_gpu(case, 0)
    for b in (0, case.B - 1):
        ref = _oracle(case, b)
        check_u(step.u[b].double().cpu().numpy(), ref["u"], case.cfg.cdtype, f"cfg{key} b={b}")
        _check_heads(step, case, b, ref, list(range(case.dims.n_h)), f"cfg{key}")
