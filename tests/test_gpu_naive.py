"""GPU: the naive-form chunked prefill (absorb_q_naive -> rope -> prefill_naive_attn -> output_proj:
keys and values expanded per head from the latent rows, attention per head on them) against the
oracle's chunk prefill, and against the absorbed form on the same inputs.

Cases: DeepSeek-V2 shape, bf16 weights and paged bf16 cache; empty, ragged and page-crossing
prefixes; chunks of 1 to 260 tokens (one to three 128-query blocks per (sequence, head), ragged tails).
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
    # (config, p0 per sequence, C, stress)
    ("2", [100, 0], 7, True),
    ("2", [40, 1, 300], 33, True),
    ("3", [70, 129], 65, False),
    ("3", [0], 1, False),
    ("2", [5], 130, True),
    # three 128-query blocks, the last one ragged (4 queries)
    ("2", [3, 40], 260, False),
]


def _run_naive(case, C, max_ctx=None):
    B = int(case.p0.numel())
    max_ctx = int(case.p0.max().item()) + C if max_ctx is None else max_ctx
    cache = build_cache(case)
    pf = mla.PrefillStep(case.dims, B, C, int(case.block_table.shape[1]), naive=True, max_ctx=max_ctx)
    u = pf.run(case.h_chunk, case.weights, cache, case.p0)
    torch.cuda.synchronize()
    return pf, u, cache


@pytest.mark.parametrize("key,p0,C,stress", CASES,
                         ids=[f"cfg{c[0]}-p0{'-'.join(map(str, c[1]))}-C{c[2]}" for c in CASES])
def test_naive_prefill_parity(key, p0, C, stress):
    case = make_prefill_case(get_config(key, stress=stress), p0, C, device="cuda")
    print(f"naive case cfg={key} p0={p0} C={C}", flush=True)
    pf, u, _ = _run_naive(case, C)
    B = len(p0)
    W = weights64(case)
    od = OracleDims.of(case.dims)
    o_gpu = pf.o.view(B, C, -1).double().cpu().numpy()
    for b in range(B):
        prefix = oracle_prefix(case, b)[: p0[b]]
        outs = prefill_chunk(W, case.h_chunk[b].double().cpu().numpy(), prefix, od, case.cfg.cdtype)
        check_u(u[b].double().cpu().numpy(), np.stack([o["u"] for o in outs]), case.cfg.cdtype,
                f"naive cfg{key} b={b}")
        # per-head outputs o_{t,i} before W^O
        o_ref = np.stack([o["o"].reshape(-1) for o in outs])
        print(f"  o rel-L2 {rel_l2(o_gpu[b], o_ref):.3e}", flush=True)
        assert rel_l2(o_gpu[b], o_ref) <= 5e-3, rel_l2(o_gpu[b], o_ref)


def test_naive_equals_absorbed_and_appends_same_rows():
    """Both execution forms append bit-identical rows (same query/KV pathway and rope kernels) and
    agree on u up to the rounding of their different arithmetic."""
    key, p0, C = "3", [33, 0, 200], 40
    case = make_prefill_case(get_config(key), p0, C, device="cuda")
    B = len(p0)
    _, u_n, c_n = _run_naive(case, C, max_ctx=max(p0) + C + 10)   # slack rows are zero-filled, masked
    u_n = u_n.clone()
    c_a = build_cache(case)
    pa = mla.PrefillStep(case.dims, B, C, int(case.block_table.shape[1]))
    u_a = pa.run(case.h_chunk, case.weights, c_a, case.p0)
    torch.cuda.synchronize()
    assert torch.equal(c_n.rows, c_a.rows)
    assert rel_l2(u_n.double().cpu().numpy(), u_a.double().cpu().numpy()) < 5e-3


def test_naive_benchmark_shape_sampled():
    """The prefill workload (B=16 x 2048 stored rows, C=64, bf16 paged) in the naive form: sampled
    chunk tokens of two sequences against the oracle, and the rest against the absorbed form."""
    key, P0, C, B = "3", 2048, 64, 16
    case = make_prefill_case(get_config(key), [P0] * B, C, device="cuda")
    pf, u, _ = _run_naive(case, C)
    u = u.clone()
    W = weights64(case)
    od = OracleDims.of(case.dims)
    for b in (0, B - 1):
        prefix = oracle_prefix(case, b)[:P0]
        outs = prefill_chunk(W, case.h_chunk[b].double().cpu().numpy()[:2], prefix, od, case.cfg.cdtype)
        for t in range(2):
            check_u(u[b, t].double().cpu().numpy(), outs[t]["u"], case.cfg.cdtype, f"naive bench b={b} t={t}")
    c_a = build_cache(case)
    pa = mla.PrefillStep(case.dims, B, C, int(case.block_table.shape[1]))
    u_a = pa.run(case.h_chunk, case.weights, c_a, case.p0)
    torch.cuda.synchronize()
    assert rel_l2(u.double().cpu().numpy(), u_a.double().cpu().numpy()) < 5e-3


def test_naive_attention_contiguous_cache_equals_paged():
    """mla_prefill_naive_attn on a contiguous copy of the paged cache (same rows, in order) gives
    the same per-head outputs bit for bit: the gather is the only layout-dependent step."""
    key, p0, C = "3", [150, 20], 40
    case = make_prefill_case(get_config(key), p0, C, device="cuda")
    B = len(p0)
    pf, _, cache = _run_naive(case, C)
    o_paged = pf.o.clone()
    ps, t_cap = cache.page_size, cache.t_cap
    j = torch.arange(t_cap, device="cuda")
    rows = cache.rows.view(-1, case.dims.row)
    # unassigned pages (-1) lie past every sequence's rows, which the gather never reads: page 0 there
    pages = [cache.block_table[b, j // ps].long().clamp_min(0) for b in range(B)]
    contig = torch.stack([rows[pages[b] * ps + j % ps] for b in range(B)]).contiguous()
    cc = mla.LatentCache(contig, cache.dtype, t_cap)
    o = torch.empty_like(o_paged)
    mla.prefill_naive_attn(pf.dims, B, C, pf.q_c, pf.step.q_pe, cc, case.p0, pf.max_ctx, case.weights["W_uk"],
                           case.weights["W_uv"], pf.ws_n, o)
    torch.cuda.synchronize()
    assert torch.equal(o, o_paged)
