"""GPU: chunked prefill through the decode calls (mla_prefill_tables + the five entry points over
B * C causal pseudo-sequences) against the oracle's chunk prefill (the chunk's decode steps in
order, each appending its rounded row), on the same stored prefix.

Cases: V2 shape with bf16 and fp8 caches (MFMA kernels), the running model with fp32 and fp16
caches (generic kernel), empty and ragged prefixes, chunks of 1 to 33 tokens crossing pages.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import mla_latent_kv_25_amd as mla  # noqa: E402
from oracle import OracleDims, prefill_chunk  # noqa: E402
from synth import get_config, make_prefill_case  # noqa: E402

from gpu_helpers import build_cache, check_u, oracle_prefix, rel_l2, weights64  # noqa: E402

CASES = [
    # (config, p0 per sequence, C, stress, num_splits)
    ("2", [100, 0], 7, True, 0),
    ("2", [40, 1, 300], 33, True, 5),
    ("3", [70, 129], 1, True, 3),
    ("4f8", [50, 3], 9, True, 0),
    ("4f6", [50, 3], 9, True, 0),
    ("0", [20, 0, 63], 5, True, 4),
    ("1", [10, 200], 12, False, 0),
]


@pytest.mark.parametrize("key,p0,C,stress,splits", CASES,
                         ids=[f"cfg{c[0]}-p0{'-'.join(map(str, c[1]))}-C{c[2]}-S{c[4]}" for c in CASES])
def test_prefill_parity(key, p0, C, stress, splits):
    case = make_prefill_case(get_config(key, stress=stress), p0, C, device="cuda")
    print(f"case cfg={key} p0={p0} C={C} cdtype={case.cfg.cdtype} splits={splits}", flush=True)
    cache = build_cache(case)
    B = len(p0)
    pf = mla.PrefillStep(case.dims, B, C, int(case.block_table.shape[1]), splits)
    u = pf.run(case.h_chunk, case.weights, cache, case.p0)
    torch.cuda.synchronize()
    W = weights64(case)
    od = OracleDims.of(case.dims)
    for b in range(B):
        prefix = oracle_prefix(case, b)[: p0[b]]
        outs = prefill_chunk(W, case.h_chunk[b].double().cpu().numpy(), prefix, od, case.cfg.cdtype)
        u_ref = np.stack([o["u"] for o in outs])
        check_u(u[b].double().cpu().numpy(), u_ref, case.cfg.cdtype, f"prefill cfg{key} b={b}")
        lse_ref = np.stack([o["lse"] for o in outs])
        lse = pf.step.lse.view(B, C, -1)[b].double().cpu().numpy()
        assert float(np.max(np.abs(lse - lse_ref))) <= (1e-4 if case.cfg.cdtype == "f32" else 2e-2)


def test_prefill_rows_match_decode_steps():
    """The rows a prefill chunk appends equal those of C single-token decode steps (bitwise)."""
    key, p0, C = "2", [30, 5], 6
    case = make_prefill_case(get_config(key, stress=True), p0, C, device="cuda")
    B = len(p0)
    c1 = build_cache(case)
    pf = mla.PrefillStep(case.dims, B, C, int(case.block_table.shape[1]), 0)
    u_pf = pf.run(case.h_chunk, case.weights, c1, case.p0).clone()
    torch.cuda.synchronize()
    c2 = build_cache(case)
    step = mla.DecodeStep(case.dims, B, 0)
    for t in range(C):
        lens = (case.p0 + t + 1).to(torch.int32).contiguous()
        u_t = step.run(case.h_chunk[:, t].contiguous(), case.weights, c2, lens)
        torch.cuda.synchronize()
        assert rel_l2(u_pf[:, t].double().cpu().numpy(), u_t.double().cpu().numpy()) < 1e-5
    assert torch.equal(c1.rows, c2.rows)


def test_prefill_benchmark_shape_sampled():
    """The bench's prefill workload (B=16 x 2048 stored rows, C=64, bf16 paged, one range per CU):
    sampled chunk tokens of two sequences against the oracle."""
    key, P0, C, B = "3", 2048, 64, 16
    case = make_prefill_case(get_config(key), [P0] * B, C, device="cuda")
    cache = build_cache(case)
    pf = mla.PrefillStep(case.dims, B, C, int(case.block_table.shape[1]), 0)
    u = pf.run(case.h_chunk, case.weights, cache, case.p0)
    torch.cuda.synchronize()
    W = weights64(case)
    od = OracleDims.of(case.dims)
    for b in (0, B - 1):
        prefix = oracle_prefix(case, b)[:P0]
        H = case.h_chunk[b].double().cpu().numpy()
        # tokens 0 and 1 of the chunk (token 1 reads token 0's appended row)
        outs = prefill_chunk(W, H[:2], prefix, od, case.cfg.cdtype)
        for t in range(2):
            check_u(u[b, t].double().cpu().numpy(), outs[t]["u"], case.cfg.cdtype, f"prefill bench b={b} t={t}")
