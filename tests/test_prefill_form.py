"""Host logic: which chunked-prefill form PrefillStep(naive="auto") picks (CPU only)."""
from types import SimpleNamespace

import torch

from mla_latent_kv_25_amd.binding import NAIVE_MIN_CHUNK, choose_prefill_form, naive_form_available

V2 = SimpleNamespace(d=5120, n_h=128, d_h=128, d_c=512, d_cq=1536, d_r=64)
RUN = SimpleNamespace(d=512, n_h=8, d_h=64, d_c=128, d_cq=96, d_r=32)


def test_naive_form_needs_its_kernel_shapes_and_types():
    assert naive_form_available(V2, torch.bfloat16, "bf16")
    assert not naive_form_available(RUN, torch.bfloat16, "bf16")            # no kernels at d_h = 64
    assert not naive_form_available(V2, torch.float16, "bf16")              # bf16 weights only
    assert not naive_form_available(V2, torch.bfloat16, "fp8_e4m3")         # bf16 cache only
    assert not naive_form_available(SimpleNamespace(**{**V2.__dict__, "d_cq": 1000}), torch.bfloat16, "bf16")


def test_auto_form_follows_the_measured_crossover():
    assert not choose_prefill_form(V2, 64, torch.bfloat16, "bf16")
    assert not choose_prefill_form(V2, NAIVE_MIN_CHUNK - 1, torch.bfloat16, "bf16")
    assert choose_prefill_form(V2, NAIVE_MIN_CHUNK, torch.bfloat16, "bf16")
    assert choose_prefill_form(V2, 512, torch.bfloat16, "bf16")
    assert not choose_prefill_form(V2, 512, torch.bfloat16, "fp8_e4m3")
    assert not choose_prefill_form(RUN, 512, torch.float32, "f32")
