"""GPU: a decode step captured as a HIP graph (torch.cuda.CUDAGraph; bench.py --graph replays the
step this way) gives the eager result on every replay, with eager work and synchronisations
between the replays. The step's kernels record no memset nodes."""
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import mla_latent_kv_25_amd as mla  # noqa: E402
from synth import get_config, make_case  # noqa: E402

from gpu_helpers import build_cache  # noqa: E402


@pytest.mark.parametrize("key,fused", [("2", True), ("2", False), ("1", False)])
def test_graph_replay_matches_eager(key, fused):
    cfg = get_config(key)
    T = [700, 33, 1, 250] if key == "2" else [300, 4096, 1, 77]
    case = make_case(cfg, device="cuda", B=len(T), T=T)
    cache = build_cache(case)
    step = mla.DecodeStep(case.dims, len(T), 0, fused=fused)
    u_ref = step.run(case.h, case.weights, cache, case.seq_lens).clone()
    lse_ref = step.lse.clone()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step.run(case.h, case.weights, cache, case.seq_lens)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step.run(case.h, case.weights, cache, case.seq_lens)
    for rep in range(3):
        step.u.fill_(7.0)
        step.lse.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(step.u, u_ref), rep
        assert torch.equal(step.lse, lse_ref), rep
        # eager work between replays
        x = torch.randn(1 << 20, device="cuda")
        torch.cuda.synchronize()
        del x
