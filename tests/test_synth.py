"""The seeded workload generator: determinism, layouts, and the stress-variant score spread."""
import numpy as np
import torch

from oracle import OracleDims, decode_step_explicit
from synth import RUNNING_DIMS, V2_DIMS, get_config, make_case


def test_deterministic_and_shapes():
    cfg = get_config("0")
    a, b = make_case(cfg), make_case(cfg)
    for k in a.weights:
        assert torch.equal(a.weights[k], b.weights[k])
        assert a.weights[k].dtype == torch.float32
    assert torch.equal(a.h, b.h) and torch.equal(a.rows, b.rows)
    assert a.weights["W_o"].shape == (512, 512) and a.weights["W_qr"].shape == (256, 96)
    assert a.rows.shape == (1, 64, 160) and int(a.seq_lens[0]) == 64
    assert torch.all(a.rows[0, 63] == 0)            # the current token's slot is left empty
    c = make_case(get_config("1"), B=3, T=[5, 1, 9])
    assert c.weights["W_uk"].dtype == torch.float16 and c.rows.shape == (3, 9, 160)
    assert torch.all(c.rows[1] == 0)


def test_paged_layout_matches_contiguous_rows():
    cfg = get_config("3")
    lens = [70, 1, 64, 65, 200]
    p = make_case(cfg, B=5, T=lens)
    c = make_case(cfg, B=5, T=lens, layout="contiguous")
    bt = p.block_table
    assert bt.shape == (5, 4)
    used = bt[bt >= 0]
    assert sorted(used.tolist()) == list(range(p.num_pages))
    assert p.num_pages == sum((t + 63) // 64 for t in lens)
    for b, t in enumerate(lens):
        assert int((bt[b] >= 0).sum()) == (t + 63) // 64
        assert torch.equal(p.prefix_rows(b), c.prefix_rows(b))
        assert p.prefix_rows(b).shape == (t - 1, 576)


def test_ragged_lengths_in_range():
    cfg = get_config("3")
    g = torch.Generator().manual_seed(1)
    from synth.gen import _lengths
    L = _lengths(cfg, 4096, g, None)
    assert int(L.min()) >= 1024 and int(L.max()) <= 32768
    assert abs(float(L.float().mean()) - (1024 + 32768) / 2) < 600


def _score_std(cfg, T=256, B=2):
    case = make_case(cfg, B=B, T=T)
    dims = OracleDims.of(cfg.dims)
    W = {k: v.double().numpy() for k, v in case.weights.items()}
    out = []
    for b in range(B):
        pre = case.prefix_rows(b).double().numpy()
        e = decode_step_explicit(W, case.h[b].double().numpy(), pre, dims, cfg.cdtype, heads=[0, 1],
                                 want_u=False)
        out.append(e["score_std"])
    return float(np.mean(out))


def test_stress_kappa_spreads_scores():
    for key in ("0", "2"):
        s0 = _score_std(get_config(key))
        s1 = _score_std(get_config(key, stress=True))
        assert s0 < 0.1, (key, s0)          # near-uniform softmax at the configs' own draws
        assert 1.0 < s1 < 4.0, (key, s1)    # stress variant: std around 2
