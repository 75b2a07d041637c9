"""GPU parity: the HIP path through the C ABI against the CPU oracle on the same seeded inputs.

Small cases span several 32-token tiles, ragged tails, single-token contexts, paged and
contiguous layouts, every cache dtype and the kappa score-stress variants; invariants check split
counts, layouts, row order, batch independence and run-to-run determinism.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU boxes only to be deselected by -m "not gpu"
    pytest.skip("no GPU", allow_module_level=True)

import mla_latent_kv_25_amd as mla  # noqa: E402
from oracle import OracleDims, absorbed_query, bf16_decode, bf16_encode, e4m3_decode, output_projection  # noqa: E402
from oracle import quantize_rows_e4m3  # noqa: E402
from synth import get_config, make_case  # noqa: E402

from gpu_helpers import TOL, build_cache, check_u, rel_l2, run_gpu, run_oracle, weights64  # noqa: E402

SMALL_CASES = [
    # (config, B, lengths, layout override, stress, num_splits)
    ("0", 1, [64], None, False, 1),
    ("0", 3, [64, 1, 33], None, True, 4),
    ("0", 2, [64, 17], None, False, 256),
    ("1", 4, [4096, 1, 100, 2049], None, False, 0),
    ("1", 3, [500, 1000, 3], None, True, 16),
    # few-head MFMA kernel: paged rows, and more ranges than tokens
    ("1", 3, [500, 1000, 3], "paged", True, 16),
    ("1", 2, [3, 40], None, True, 64),
    ("1", 3, [70, 33, 1], "paged", False, 37),
    ("2", 3, [300, 1, 77], None, False, 4),
    ("2", 3, [300, 1, 77], None, True, 4),
    ("2", 2, [1000, 65], "paged", True, 5),
    ("3", 4, [1030, 64, 1, 2000], None, False, 0),
    ("3", 4, [700, 129, 31, 1500], None, True, 7),
    ("4", 2, [3000, 129], None, False, 8),
    ("4f8", 2, [3000, 129], None, False, 8),
    ("4f8", 2, [2000, 33], None, True, 3),
    ("4f8", 3, [900, 64, 2], "paged", True, 5),
    # more ranges than tokens: most ranges are empty, the rest hold one or two tokens
    ("2", 2, [3, 40], None, True, 64),
    ("4f8", 2, [5, 20], "paged", True, 48),
    # fp6 e2m3 cache (packed rows converted to the fp8 tile layout in LDS)
    ("4f6", 2, [3000, 129], None, False, 8),
    ("4f6", 2, [2000, 33], None, True, 3),
    ("4f6", 3, [900, 64, 2], "paged", True, 5),
    ("4f6", 2, [5, 20], "paged", True, 48),
]


def _case(key, B, T, layout=None, stress=False, seed=None):
    cfg = get_config(key, stress=stress)
    return make_case(cfg, device="cuda", B=B, T=T, layout=layout, seed=seed)


@pytest.mark.parametrize("key,B,T,layout,stress,splits", SMALL_CASES,
                         ids=[f"cfg{c[0]}-B{c[1]}-{c[3] or 'cfg'}-{'stress' if c[4] else 'plain'}-S{c[5]}"
                              for c in SMALL_CASES])
def test_small_parity(key, B, T, layout, stress, splits):
    case = _case(key, B, T, layout, stress)
    print(f"case cfg={key} B={B} T={T} layout={case.cfg.layout} cdtype={case.cfg.cdtype} stress={stress} "
          f"splits={splits}", flush=True)
    step, _ = run_gpu(case, splits)
    ref = run_oracle(case)
    u_ref = np.stack([ref[b]["u"] for b in range(B)])
    check_u(step.u.double().cpu().numpy(), u_ref, case.cfg.cdtype, f"cfg{key}")
    o_ref = np.stack([ref[b]["o_lat"] for b in range(B)])
    lse_ref = np.stack([ref[b]["lse"] for b in range(B)])
    o_err = rel_l2(step.o_lat.double().cpu().numpy(), o_ref)
    lse_err = float(np.max(np.abs(step.lse.double().cpu().numpy() - lse_ref)))
    print(f"  o_lat rel-L2 {o_err:.3e}  lse max-abs {lse_err:.3e}", flush=True)
    tol_o = 1e-4 if case.cfg.cdtype == "f32" else 5e-3
    assert o_err <= tol_o and lse_err <= (1e-4 if case.cfg.cdtype == "f32" else 2e-2)


@pytest.mark.parametrize("key", ["0", "1", "2", "4f8", "4f6"])
def test_tiny_contexts(key):
    """Contexts of 1-4 tokens (T = 1 is the closed form: one weight of 1)."""
    case = _case(key, 4, [1, 2, 3, 4], stress=True)
    step, _ = run_gpu(case, 2)
    ref = run_oracle(case)
    check_u(step.u.double().cpu().numpy(), np.stack([ref[b]["u"] for b in range(4)]), case.cfg.cdtype, f"tiny{key}")


def test_stage_outputs():
    """absorb_q / rope outputs and absorb_out against the oracle's stage definitions."""
    for key in ("0", "2"):
        case = _case(key, 3, [40, 1, 7], stress=True)
        step, cache = run_gpu(case, 2)
        W = weights64(case)
        od = OracleDims.of(case.dims)
        for b in range(3):
            q_lat, q_pe, row = absorbed_query(W, case.h[b].double().cpu().numpy(), int(case.seq_lens[b]) - 1, od)
            e1 = rel_l2(step.q_lat[b].double().cpu().numpy(), q_lat)
            e2 = rel_l2(step.q_pe[b].double().cpu().numpy(), q_pe)
            e3 = rel_l2(step.kv_new[b].double().cpu().numpy(), row)
            print(f"cfg{key} b{b} q_lat {e1:.2e} q_pe {e2:.2e} kv_new {e3:.2e}", flush=True)
            assert max(e1, e2, e3) < (1e-5 if key == "0" else 2e-4)
        # output stage on a drawn o_lat (not taken from the GPU pipeline)
        g = torch.Generator(device="cpu").manual_seed(5)
        o_lat = torch.randn((3, case.dims.n_h, case.dims.d_c), generator=g).cuda() * 0.3
        d = mla.Dims.of(case.dims)
        ws = torch.empty(mla.absorb_out_workspace_bytes(d, 3), dtype=torch.uint8, device="cuda")
        u = torch.empty((3, case.dims.d), dtype=torch.float32, device="cuda")
        mla.absorb_out(d, o_lat, case.weights["W_uv"], case.weights["W_o"], ws, u)
        torch.cuda.synchronize()
        for b in range(3):
            ref = output_projection(W, o_lat[b].double().cpu().numpy(), od)
            e = rel_l2(u[b].double().cpu().numpy(), ref)
            print(f"cfg{key} absorb_out b{b} {e:.2e}", flush=True)
            assert e < (1e-5 if key == "0" else 2e-4)


@pytest.mark.parametrize("B", [33, 100, 130, 300])
def test_stage_outputs_wide_batch(B):
    """Projection stages at batch widths that use every column-block count of the MFMA GEMMs
    (33: two blocks with a ragged one, 100: four, 130: two 128-column tiles in one launch, the
    second holding 2 rows; 300: three tiles, a ragged 44-row one, with K split over the tiles; from
    256 rows on, the per-head outputs are rounded to bf16 between W^UV and W^O, and the reference
    rounds them the same way)."""
    case = _case("2", B, [5] * B)
    d = mla.Dims.of(case.dims)
    step = mla.DecodeStep(case.dims, B, 0)
    mla.absorb_q(d, case.h, case.weights, step.ws_q, step.q_lat, step.q_pe, step.kv_new)
    g = torch.Generator(device="cpu").manual_seed(11)
    o_lat = (torch.randn((B, case.dims.n_h, case.dims.d_c), generator=g) * 0.3).cuda()
    mla.absorb_out(d, o_lat, case.weights["W_uv"], case.weights["W_o"], step.ws_o, step.u)
    torch.cuda.synchronize()
    W = weights64(case)
    od = OracleDims.of(case.dims)
    worst, worst_round = 0.0, 0.0
    Wuv = W["W_uv"].reshape(case.dims.n_h, case.dims.d_h, case.dims.d_c)
    for b in range(B):
        q_lat, _, row = absorbed_query(W, case.h[b].double().cpu().numpy(), 4, od)
        ol = o_lat[b].double().cpu().numpy()
        if B >= 256:
            # wide batches round the per-head outputs o_i = W^UV_i o_lat_i to bf16 before W^O (the
            # header's contract): the reference applies the same rounding
            o = np.stack([Wuv[i] @ ol[i] for i in range(case.dims.n_h)]).reshape(-1)
            u_ref = W["W_o"] @ bf16_decode(bf16_encode(o))
            # and that rounding stays within its budget (unit roundoff 2^-9 per element of o)
            worst_round = max(worst_round, rel_l2(step.u[b].double().cpu().numpy(), output_projection(W, ol, od)))
        else:
            u_ref = output_projection(W, ol, od)
        e = max(rel_l2(step.q_lat[b].double().cpu().numpy(), q_lat),
                rel_l2(step.kv_new[b, :case.dims.d_c].double().cpu().numpy(), row[:case.dims.d_c]),
                rel_l2(step.u[b].double().cpu().numpy(), u_ref))
        worst = max(worst, e)
    print(f"B={B} worst stage rel-L2 {worst:.2e}, u against unrounded o {worst_round:.2e}", flush=True)
    assert worst < 2e-4
    assert worst_round < 2.0 ** -8


def test_split_count_invariance():
    case = _case("2", 3, [700, 33, 250], stress=True)
    outs = []
    for S in (1, 3, 16, 64):
        step, _ = run_gpu(case, S)
        outs.append((step.u.clone(), step.o_lat.clone(), step.lse.clone()))
    for u, o, l in outs[1:]:
        assert rel_l2(u.double().cpu().numpy(), outs[0][0].double().cpu().numpy()) < 2e-3
        assert float((l - outs[0][2]).abs().max()) < 1e-3


@pytest.mark.parametrize("key", ["0", "1", "2", "4f8", "4f6"])
def test_zero_length_sequences(key):
    """decode_attn + combine with some sequences at length 0 (first, middle and last), called on
    the queries and cache of a normal step: those sequences get o_lat = 0 and lse = -inf, and the
    others match the normal step up to the range split (the batch's total changes)."""
    T = [1, 300, 1, 77, 5, 1]
    empty = [0, 2, 5]
    case = _case(key, len(T), T, layout="paged" if key in ("2", "4f8", "4f6") else None, stress=True)
    print(f"case cfg={key} T={T} zeroed={empty}", flush=True)
    step, cache = run_gpu(case, 7)
    lens = case.seq_lens.clone()
    lens[empty] = 0
    o_lat = torch.full_like(step.o_lat, 7.0)
    lse = torch.full_like(step.lse, 7.0)
    mla.decode_attn(step.dims, step.q_lat, step.q_pe, cache, lens, 7, step.ws_d)
    mla.combine(step.dims, 7, lens, step.ws_d, o_lat, lse)
    torch.cuda.synchronize()
    for b in range(len(T)):
        if b in empty:
            assert torch.all(o_lat[b] == 0) and torch.all(torch.isneginf(lse[b])), b
        else:
            e = rel_l2(o_lat[b].double().cpu().numpy(), step.o_lat[b].double().cpu().numpy())
            le = float((lse[b] - step.lse[b]).abs().max())
            print(f"  b{b}: o_lat rel-L2 {e:.2e}, lse max-abs {le:.2e}", flush=True)
            assert e < (1e-5 if key == "0" else 2e-3) and le < (1e-5 if key == "0" else 1e-3)


@pytest.mark.parametrize("key,layout", [("2", "contiguous"), ("2", "paged"), ("4f8", "contiguous"), ("4f6", "paged"),
                                        ("0", "contiguous")])
def test_rope_zero_length_writes_nothing(key, layout):
    """mla_rope with sequences of length 0 (outside the contract; the first and the last of the
    batch): their q_pe and kv_new rows stay as they were and nothing is stored for them. In a
    contiguous cache, position -1 of sequence 0 would be the row before the buffer, and in a paged
    cache slot -1 of its first page. The only cache rows that change are the rows the other
    sequences append at their positions."""
    T = [5, 300, 9]
    empty = [0, 2]
    case = _case(key, 3, T, layout=layout)
    print(f"case cfg={key} layout={layout} T={T} zeroed={empty}", flush=True)
    cache = build_cache(case)
    step = mla.DecodeStep(case.dims, 3, 4)
    mla.absorb_q(step.dims, case.h, case.weights, step.ws_q, step.q_lat, step.q_pe, step.kv_new)
    torch.cuda.synchronize()
    lens = case.seq_lens.clone()
    lens[empty] = 0
    rows0, qpe0, kv0 = cache.rows.clone(), step.q_pe.clone(), step.kv_new.clone()
    sc0 = cache.scales.clone() if cache.scales is not None else None
    mla.rope(step.dims, lens, step.q_pe, step.kv_new, cache)
    torch.cuda.synchronize()
    for b in empty:
        assert torch.equal(step.q_pe[b], qpe0[b]) and torch.equal(step.kv_new[b], kv0[b]), b
    assert not torch.equal(step.q_pe[1], qpe0[1])  # the non-empty sequence was rotated
    changed = (cache.rows != rows0).reshape(-1, cache.rows.shape[-1]).any(dim=1)
    if sc0 is not None:
        changed |= (cache.scales != sc0).reshape(-1)
    pos = T[1] - 1
    if layout == "contiguous":
        allowed = 1 * case.t_cap + pos
    else:
        ps = case.cfg.page_size
        allowed = int(case.block_table[1, pos // ps]) * ps + pos % ps
    idx = torch.nonzero(changed).flatten().tolist()
    assert set(idx) <= {allowed}, idx


def test_paged_equals_contiguous():
    for key in ("2", "4f8", "4f6"):
        pc = _case(key, 3, [300, 64, 129], layout="paged", stress=True)
        cc = _case(key, 3, [300, 64, 129], layout="contiguous", stress=True)
        for b in range(3):
            assert torch.equal(pc.prefix_rows(b), cc.prefix_rows(b))
        sp, _ = run_gpu(pc, 5)
        sc, _ = run_gpu(cc, 5)
        assert torch.equal(sp.u, sc.u), float((sp.u - sc.u).abs().max())


def test_row_permutation_invariance():
    """Rows hold already-rotated keys, so attention over them is a set function of the rows."""
    case = _case("2", 1, [257], stress=True)
    step, _ = run_gpu(case, 3)
    u0 = step.u.clone()
    perm = torch.randperm(256, generator=torch.Generator().manual_seed(3)).cuda()
    case.rows[0, :256] = case.rows[0, :256][perm]
    step2, _ = run_gpu(case, 3)
    assert rel_l2(step2.u.double().cpu().numpy(), u0.double().cpu().numpy()) < 3e-3


def test_batch_independence_and_determinism():
    case = _case("3", 4, [1030, 64, 1, 600], stress=True)
    s1, _ = run_gpu(case, 6)
    s2, _ = run_gpu(case, 6)
    assert torch.equal(s1.u, s2.u) and torch.equal(s1.o_lat, s2.o_lat)   # bitwise reproducible
    alone = make_case(case.cfg, device="cuda", B=4, T=[1030, 64, 1, 600])
    assert torch.equal(alone.rows, case.rows)
    # sequence 1 alone in a batch of its own
    one = make_case(case.cfg, device="cuda", B=4, T=[1030, 64, 1, 600])
    one.h = one.h[1:2].contiguous()
    one.seq_lens = one.seq_lens[1:2].contiguous()
    one.block_table = one.block_table[1:2].contiguous()
    s3, _ = run_gpu(one, 1)
    assert rel_l2(s3.u[0].double().cpu().numpy(), s1.u[1].double().cpu().numpy()) < 2e-3


def test_fp6_cache_store_bit_exact():
    """The library's fp6 encoder (mla_cache_store) writes the oracle's packed bytes and scales."""
    from oracle import pack_e2m3, quantize_rows_e2m3
    for layout in ("contiguous", "paged"):
        case = _case("4f6", 3, [200, 1, 70], layout=layout)
        cache = build_cache(case)
        torch.cuda.synchronize()
        for b in range(3):
            n = int(case.seq_lens[b]) - 1
            src = case.prefix_rows(b).float().cpu().numpy()
            codes, scales = quantize_rows_e2m3(src)
            packed = pack_e2m3(codes)
            if layout == "contiguous":
                g_rows = cache.rows[b, :n].cpu().numpy()
                g_sc = cache.scales[b, :n].cpu().numpy()
            else:
                ps = case.cfg.page_size
                pages = case.block_table[b, : (n + ps) // ps].long()
                g_rows = cache.rows[pages].reshape(-1, cache.rows.shape[-1])[:n].cpu().numpy()
                g_sc = cache.scales[pages].reshape(-1)[:n].cpu().numpy()
            assert np.array_equal(g_rows, packed), (layout, b)
            assert np.array_equal(g_sc.view(np.uint32), scales.view(np.uint32)), (layout, b)


@pytest.mark.parametrize("key,B,T,splits", [("1", 4, [500, 1, 100, 2049], 16), ("0", 3, [64, 1, 33], 4)])
def test_fp6_generic_kernel(key, B, T, splits):
    """An fp6 cache at the running model's dims (float32 generic kernel, 6-bit codes read in place)."""
    cfg = get_config(key, stress=True)
    for layout in ("contiguous", "paged"):
        case = make_case(cfg, device="cuda", B=B, T=T, layout=layout, cdtype="fp6_e2m3")
        print(f"case cfg={key} fp6 layout={layout} T={T} splits={splits}", flush=True)
        step, _ = run_gpu(case, splits)
        ref = run_oracle(case)
        u_ref = np.stack([ref[b]["u"] for b in range(B)])
        check_u(step.u.double().cpu().numpy(), u_ref, "fp6_e2m3", f"cfg{key} fp6 {layout}")


@pytest.mark.parametrize("layout", ["contiguous", "paged"])
def test_small_heads_bf16(layout):
    """A bf16 cache at the running model's dims (the few-head MFMA kernel in its bf16 form)."""
    cfg = get_config("1", stress=True)
    B, T = 3, [1200, 65, 2]
    case = make_case(cfg, device="cuda", B=B, T=T, layout=layout, cdtype="bf16")
    print(f"case cfg=1 bf16 layout={layout} T={T} splits=0", flush=True)
    step, _ = run_gpu(case, 0)
    ref = run_oracle(case)
    u_ref = np.stack([ref[b]["u"] for b in range(B)])
    check_u(step.u.double().cpu().numpy(), u_ref, "bf16", f"cfg1 bf16 {layout}")
    o_ref = np.stack([ref[b]["o_lat"] for b in range(B)])
    o_err = rel_l2(step.o_lat.double().cpu().numpy(), o_ref)
    print(f"  o_lat rel-L2 {o_err:.3e}", flush=True)
    assert o_err <= 5e-3


def test_fp8_cache_store_bit_exact():
    for layout in ("contiguous", "paged"):
        case = _case("4f8", 3, [200, 1, 70], layout=layout)
        cache = build_cache(case)
        torch.cuda.synchronize()
        for b in range(3):
            n = int(case.seq_lens[b]) - 1
            src = case.prefix_rows(b).float().cpu().numpy()
            codes, scales = quantize_rows_e4m3(src)
            if layout == "contiguous":
                g_codes = cache.rows[b, :n].cpu().numpy()
                g_sc = cache.scales[b, :n].cpu().numpy()
            else:
                ps = case.cfg.page_size
                pages = case.block_table[b, : (n + ps) // ps].long()
                g_codes = cache.rows[pages].reshape(-1, case.dims.row)[:n].cpu().numpy()
                g_sc = cache.scales[pages].reshape(-1)[:n].cpu().numpy()
            assert np.array_equal(g_codes, codes), (layout, b)
            assert np.array_equal(g_sc.view(np.uint32), scales.view(np.uint32)), (layout, b)


def test_appended_row_storage():
    """The row mla_rope appends is the oracle's row rounded to the storage type: float32 to
    rounding, bf16 within one code step for elements whose float32 value sits on a rounding
    boundary, fp8 codes within one step and the scale within float32 rounding."""
    for key in ("0", "2", "4f8", "4f6"):
        case = _case(key, 3, [40, 1, 7], stress=True)
        step, cache = run_gpu(case, 2)
        ref = run_oracle(case, want_u=False, heads=[0])
        for b in range(3):
            pos = int(case.seq_lens[b]) - 1
            row_ref = ref[b]["row_new"]
            if case.cfg.cdtype == "f32":
                g = cache.rows[b, pos].double().cpu().numpy()
                assert rel_l2(g, row_ref) < 1e-6 and np.max(np.abs(g - row_ref)) < 1e-6 * np.max(np.abs(row_ref))
            elif case.cfg.cdtype == "bf16":
                g = cache.rows[b, pos].view(torch.int16).cpu().numpy().view(np.uint16).astype(np.int64)
                r = bf16_encode(row_ref).astype(np.int64)
                assert np.max(np.abs(g - r)) <= 1 and np.mean(g != r) < 0.02
            elif case.cfg.cdtype == "fp6_e2m3":
                from oracle import e2m3_decode, quantize_rows_e2m3, unpack_e2m3
                g = unpack_e2m3(cache.rows[b, pos].cpu().numpy(), case.dims.row)
                codes, scale = quantize_rows_e2m3(row_ref.astype(np.float32)[None, :])
                assert abs(float(cache.scales[b, pos]) - float(scale[0])) <= 1e-6 * float(scale[0])
                dv = np.abs(e2m3_decode(g) - e2m3_decode(codes[0]))
                assert np.mean(g != codes[0]) < 0.02
                assert np.all(dv <= np.abs(e2m3_decode(codes[0])) * 2.0 ** -3 + 2.0 ** -3)
            else:
                g = cache.rows[b, pos].cpu().numpy()
                codes, scale = quantize_rows_e4m3(row_ref.astype(np.float32)[None, :])
                assert abs(float(cache.scales[b, pos]) - float(scale[0])) <= 1e-6 * float(scale[0])
                dv = np.abs(e4m3_decode(g) - e4m3_decode(codes[0]))
                assert np.mean(g != codes[0]) < 0.02
                assert np.all(dv <= np.abs(e4m3_decode(codes[0])) * 2.0 ** -3 + 2.0 ** -9)


def spike_budget(case, ref, mult, rel=2.0 ** -7):
    """Error budget of the late-spike case, from the oracle's own
    query and stored rows. The V2-shape MFMA kernels hold the query as bf16 (or as two e4m3 parts
    with the same 8 significant bits) and the probabilities as bf16: each is rounded with a relative
    error of at most 2^-8, so
      score s_ij:  |ds_ij| <= 2^-8 * scale * sum_k |q_ik c_jk|, and lse_i moves by at most max_j |ds_ij|;
      u:           one dominating row carries its rounded weight into every output, |du| <= 2^-8 |u|,
                   plus 2^-11 for the float16 partial rows.
    The bars are the absolute bf16 bars (max-abs 2e-2) plus twice these terms (rel = 2^-7), and they grow with
    the spike: 8x more from x8 to x64. The few-head kernel over an fp16 cache rounds the query and
    the probabilities to fp16 (unit roundoff 2^-11): rel = 2^-10."""
    import numpy as np
    from oracle import OracleDims, absorbed_query, score_scale
    dims = OracleDims.of(case.dims)
    W = weights64(case)
    scale = float(score_scale(dims))
    lse_bar, u_bar = [], []
    for b in range(case.B):
        T = int(case.seq_lens[b])
        q_lat, q_pe, _ = absorbed_query(W, case.h[b].double().cpu().numpy(), T - 1, dims)
        q = np.abs(np.concatenate([q_lat, q_pe], axis=1))                       # [n_h, 576]
        from gpu_helpers import oracle_prefix
        rows = np.abs(np.vstack([oracle_prefix(case, b), ref[b]["read_new"][None, :]]))  # [T, 576]
        lse_bar.append(2e-2 + rel * scale * (rows @ q.T).max(axis=0))   # per head
        u_bar.append(2e-2 + rel * float(np.max(np.abs(ref[b]["u"]))))
    return np.stack(lse_bar), np.array(u_bar)


@pytest.mark.parametrize("key,mult", [("0", 64), ("1", 64), ("2", 8), ("2", 64), ("4f8", 8), ("4f8", 64),
                                      ("4f6", 64)])
def test_late_score_spike(key, mult):
    """A cached row far along a range with a score far above everything before it: the attention
    kernels take the first tile's maximum as their softmax reference, and a score more than 2^64
    above it sends the range through a second pass with a higher reference. One row per sequence
    is scaled by `mult` (exact in every storage type, and the fp8 scale follows it); with 4 ranges
    over T = [1000, 300], both rows sit in later tiles of their ranges. At x64 the spike dominates
    some heads by far more than 2^64 (second pass), at x8 it does not; u is up to ~50x larger than in
    the standard workloads. The MFMA kernels (configs 1, 2, 4f8, 4f6) are held to the error budget of
    spike_budget, the float32 generic kernel (config 0) to the plain bars."""
    import numpy as np
    case = _case(key, 2, [1000, 300], stress=True)
    src = case.row_source()
    assert case.cfg.layout == "contiguous"
    for b, pos in ((0, 900), (1, 250)):
        src[b, pos] = src[b, pos] * mult
    print(f"case cfg={key} B=2 T=[1000, 300] spike rows (0, 900), (1, 250) x{mult} splits=4", flush=True)
    step, _ = run_gpu(case, 4)
    ref = run_oracle(case)
    u_ref = np.stack([ref[b]["u"] for b in range(2)])
    lse_ref = np.stack([ref[b]["lse"] for b in range(2)])
    u_gpu = step.u.double().cpu().numpy()
    lse_err = np.abs(step.lse.double().cpu().numpy() - lse_ref)
    rl = rel_l2(u_gpu, u_ref)
    u_err = np.max(np.abs(u_gpu - u_ref), axis=1)
    tr, ta = TOL[case.cfg.cdtype]
    print(f"spike cfg{key} x{mult}: u rel-L2 {rl:.3e}, max-abs per seq {u_err}, |u|max {np.max(np.abs(u_ref)):.3e}; "
          f"lse max-abs {lse_err.max():.3e} (largest lse {lse_ref.max():.1f})", flush=True)
    assert rl <= tr, rl
    if mult == 64:  # the second pass is reached
        assert float(np.max(lse_ref)) > 100.0, float(np.max(lse_ref))
    if case.cfg.cdtype == "f32":
        # float32 arithmetic on the stored values throughout: the absolute bars plus a float32
        # budget of 2^-16 relative (unit roundoff 2^-24 grown by sums of up to a few thousand terms)
        assert np.all(u_err <= ta + 2.0 ** -16 * np.max(np.abs(u_ref), axis=1)), u_err
        lse_tol = 1e-4 + 2.0 ** -16 * np.abs(lse_ref)
        assert np.all(lse_err <= lse_tol), float(np.max(lse_err - lse_tol))
        return
    lse_bar, u_bar = spike_budget(case, ref, mult, 2.0 ** -10 if case.cfg.cdtype == "f16" else 2.0 ** -7)
    print(f"  budget: u max-abs <= {u_bar}, lse max-abs <= {lse_bar.min():.3e} .. {lse_bar.max():.3e}; "
          f"worst lse use {float(np.max(lse_err / lse_bar)):.2f} of its bar", flush=True)
    assert np.all(u_err <= u_bar), (u_err, u_bar)
    assert np.all(lse_err <= lse_bar), float(np.max(lse_err - lse_bar))


@pytest.mark.parametrize("key,ps", [("2", 32), ("2", 256), ("4f8", 32), ("4f8", 128), ("4f6", 32), ("4f6", 256),
                                    ("1", 16), ("1", 32), ("1", 128), ("0", 8)])
def test_page_sizes(key, ps):
    """Paged caches with other page sizes than the configs' 64: the MFMA kernels take any power of
    two >= 32 (a 32-token tile spans at most two pages), the generic kernel any size. Ragged
    lengths put range starts at every offset inside a page."""
    cfg = get_config(key, stress=True).with_(page_size=ps)
    case = make_case(cfg, device="cuda", B=3, T=[300, 70, 5], layout="paged")
    print(f"case cfg={key} page_size={ps} B=3 T=[300, 70, 5] splits=7", flush=True)
    step, _ = run_gpu(case, 7)
    ref = run_oracle(case)
    u_ref = np.stack([ref[b]["u"] for b in range(3)])
    check_u(step.u.double().cpu().numpy(), u_ref, case.cfg.cdtype, f"paged ps={ps} cfg{key}")


@pytest.mark.parametrize("key", ["2", "4f8", "4f6", "1"])
def test_paged_long_ranges(key):
    """Ranges that span more than 64 pages: with 32-token pages and two ranges over the 6800 tokens, each
    range covers about 106 pages, whose ids the kernels look up tile by tile as the range crosses
    page after page."""
    cfg = get_config(key, stress=True).with_(page_size=32)
    case = make_case(cfg, device="cuda", B=2, T=[4500, 2300], layout="paged")
    print(f"case cfg={key} page_size=32 B=2 T=[4500, 2300] splits=2", flush=True)
    step, _ = run_gpu(case, 2)
    ref = run_oracle(case)
    u_ref = np.stack([ref[b]["u"] for b in range(2)])
    check_u(step.u.double().cpu().numpy(), u_ref, case.cfg.cdtype, f"paged long range cfg{key}")
