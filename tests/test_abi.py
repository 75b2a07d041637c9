"""The C-ABI library: it loads, exports every symbol include/mla.h declares, and rejects invalid
arguments on the host before enqueueing anything (no GPU needed: every call here fails
validation, or is a no-op, before any HIP call)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    from mla_latent_kv_25_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from mla_latent_kv_25_amd.build import build
        build()
    return binding.lib()


def _declared():
    src = open(os.path.join(ROOT, "include", "mla.h")).read()
    return sorted(set(re.findall(r"MLA_API\s+[\w\s\*]+?\b(mla_\w+)\s*\(", src)))


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert len(names) == 25, names
    for n in names:
        assert hasattr(L, n), n
    from mla_latent_kv_25_amd.binding import EXPORTS
    assert sorted(EXPORTS) == names
    assert L.mla_version().decode().startswith("mla_latent_kv_25_amd")


def _dims(**kw):
    from mla_latent_kv_25_amd.binding import Dims
    d = dict(d=512, n_h=8, d_h=64, d_c=128, d_cq=96, d_r=32, rope_base=10000.0, sm_scale=0.0)
    d.update(kw)
    return Dims(**d)


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first in every use below


def test_status_strings(L):
    assert L.mla_status_str(0) == b"MLA_OK"
    assert L.mla_status_str(3) == b"MLA_E_WORKSPACE"


def test_dims_validation(L):
    assert L.mla_rope(None, 1, None, None, None, None, None) == 1
    assert b"dims is NULL" in L.mla_last_error()
    for bad in (dict(n_h=0), dict(d_r=30), dict(d_c=100), dict(rope_base=1.0), dict(d=-5),
                dict(yarn_factor=40.0, yarn_orig_len=0, yarn_alpha=1.0, yarn_beta=32.0),
                dict(yarn_factor=40.0, yarn_orig_len=4096, yarn_alpha=32.0, yarn_beta=1.0),
                dict(yarn_factor=float("nan"))):
        d = _dims(**bad)
        assert L.mla_rope(ctypes.byref(d), 1, FAKE, FAKE, FAKE, None, None) == 1, bad


def test_absorb_q_validation(L):
    d = _dims()
    # bad weight dtype (fp8 is a cache-only format)
    assert L.mla_absorb_q(ctypes.byref(d), 2, 3, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                          FAKE, FAKE, FAKE, None) == 1
    # null tensor
    assert L.mla_absorb_q(ctypes.byref(d), 2, 0, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                          FAKE, FAKE, FAKE, None) == 1
    # workspace too small
    need = L.mla_absorb_q_workspace_bytes(ctypes.byref(d), 2)
    assert need > 0
    assert L.mla_absorb_q(ctypes.byref(d), 2, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1,
                          FAKE, FAKE, FAKE, None) == 3
    assert b"workspace" in L.mla_last_error()
    # empty batch: nothing to do
    assert L.mla_absorb_q(ctypes.byref(d), 0, 0, None, None, None, None, None, None, None, None, 0,
                          None, None, None, None) == 0
    assert L.mla_absorb_q(ctypes.byref(d), -1, 0, None, None, None, None, None, None, None, None, 0,
                          None, None, None, None) == 1


def _cache(**kw):
    from mla_latent_kv_25_amd.binding import CCache
    c = dict(rows=0x1000, scales=None, dtype=2, page_size=0, t_cap=64, block_table=None, max_pages=0, num_pages=0)
    c.update(kw)
    return CCache(**c)


def test_cache_validation(L):
    d = _dims()
    cases = [
        (_cache(rows=None), b"rows is NULL"),
        (_cache(dtype=9), b"bad cache dtype"),
        (_cache(dtype=3), b"scales"),                       # fp8 without scales
        (_cache(scales=0x2000), b"scales"),                 # scales on a bf16 cache
        (_cache(t_cap=0), b"t_cap"),
        (_cache(page_size=64, t_cap=128), b"block table"),
        (_cache(page_size=64, t_cap=100, block_table=0x3000, max_pages=2, num_pages=4), b"max_pages * page_size"),
    ]
    for c, msg in cases:
        assert L.mla_decode_attn(ctypes.byref(d), 1, FAKE, FAKE, ctypes.byref(c), FAKE, 4, FAKE, 1 << 30, None) == 1
        assert msg in L.mla_last_error(), (msg, L.mla_last_error())


def test_decode_validation(L):
    d = _dims()
    c = _cache()
    assert L.mla_decode_attn(ctypes.byref(d), 1, FAKE, FAKE, ctypes.byref(c), FAKE, -1, FAKE, 1 << 30, None) == 1
    assert L.mla_decode_attn(ctypes.byref(d), 1, FAKE, FAKE, ctypes.byref(c), FAKE, 1025, FAKE, 1 << 40, None) == 1
    need = L.mla_decode_workspace_bytes(ctypes.byref(d), 3, 8)
    # (8 + 3 - 1) pieces of n_h * (d_c + 1) floats plus the prefix sums
    assert need >= (8 + 3 - 1) * 8 * (128 + 1) * 4 + 4 * 8
    assert L.mla_decode_attn(ctypes.byref(d), 3, FAKE, FAKE, ctypes.byref(c), FAKE, 8, FAKE, need - 1, None) == 3
    assert L.mla_combine(ctypes.byref(d), 3, 8, FAKE, FAKE, need - 1, FAKE, None, None) == 3
    # the MFMA path needs power-of-two pages of at least 32 rows at the V2 shape
    v2 = _dims(d=5120, n_h=128, d_h=128, d_c=512, d_cq=1536, d_r=64)
    pc = _cache(page_size=48, t_cap=96, block_table=0x3000, max_pages=2, num_pages=2)
    assert L.mla_decode_attn(ctypes.byref(v2), 1, FAKE, FAKE, ctypes.byref(pc), FAKE, 4, FAKE, 1 << 40, None) == 2
    # no kernel for a float32 cache at the V2 shape
    fc = _cache(dtype=0)
    assert L.mla_decode_attn(ctypes.byref(v2), 1, FAKE, FAKE, ctypes.byref(fc), FAKE, 4, FAKE, 1 << 40, None) == 2


def test_absorb_out_and_store_validation(L):
    d = _dims()
    assert L.mla_absorb_out(ctypes.byref(d), 2, 0, None, FAKE, FAKE, FAKE, 1 << 30, FAKE, None) == 1
    need = L.mla_absorb_out_workspace_bytes(ctypes.byref(d), 2)
    assert L.mla_absorb_out(ctypes.byref(d), 2, 0, FAKE, FAKE, FAKE, FAKE, need - 1, FAKE, None) == 3
    c = _cache()
    assert L.mla_cache_store(ctypes.byref(d), ctypes.byref(c), 1, FAKE, 65, FAKE, 65, None) == 1  # > t_cap
    assert L.mla_cache_store(ctypes.byref(d), ctypes.byref(c), 1, FAKE, 10, FAKE, 5, None) == 1   # stride
    assert L.mla_cache_store(ctypes.byref(d), ctypes.byref(c), 0, None, 0, None, 0, None) == 0


def test_absorb_out_noalloc_validation(L):
    """The no-allocation variant rejects bad arguments, and any batch whose workspace would not fit
    the library's static scratch, before touching the device."""
    d = _dims()
    assert L.mla_absorb_out_noalloc(ctypes.byref(d), 2, 0, None, FAKE, FAKE, FAKE, None) == 1
    assert L.mla_absorb_out_noalloc(ctypes.byref(d), 2, 7, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert L.mla_absorb_out_noalloc(ctypes.byref(d), 0, 0, None, None, None, None, None) == 0
    v2 = _dims(d=5120, n_h=128, d_h=128, d_c=512, d_cq=1536, d_r=64)
    limit = 32 << 20
    assert L.mla_absorb_out_workspace_bytes(ctypes.byref(v2), 255) <= limit
    assert L.mla_absorb_out_workspace_bytes(ctypes.byref(v2), 256) > limit
    assert L.mla_absorb_out_noalloc(ctypes.byref(v2), 256, 2, FAKE, FAKE, FAKE, FAKE, None) == 3
    assert b"scratch" in L.mla_last_error()


def test_precombined_validation(L):
    d = _dims()
    odd = ctypes.c_void_p(0x1004)
    assert L.mla_precombine(None, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert L.mla_precombine(ctypes.byref(d), 7, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1   # dtype
    assert L.mla_precombine(ctypes.byref(d), 0, None, None, None, None, None, None, None) == 0   # nothing asked
    assert L.mla_precombine(ctypes.byref(d), 0, None, FAKE, None, None, FAKE, None, None) == 1   # W_uq missing
    assert b"W_uq" in L.mla_last_error()
    assert L.mla_precombine(ctypes.byref(d), 0, None, None, FAKE, None, None, FAKE, None) == 1   # W_o missing
    assert L.mla_precombine(ctypes.byref(d), 0, FAKE, FAKE, None, None, odd, None, None) == 1
    assert b"aligned" in L.mla_last_error()
    need_q = L.mla_absorb_q_workspace_bytes(ctypes.byref(d), 2)
    args = [FAKE] * 6
    assert L.mla_absorb_q_pre(ctypes.byref(d), 2, 0, *args[:2], None, *args[:3], FAKE, need_q, FAKE, FAKE, FAKE,
                              None) == 1                                                        # Wq_pre NULL
    assert L.mla_absorb_q_pre(ctypes.byref(d), 2, 0, *args, FAKE, need_q - 1, FAKE, FAKE, FAKE, None) == 3
    assert L.mla_absorb_q_pre(ctypes.byref(d), 0, 0, *[None] * 6, None, 0, None, None, None, None) == 0
    need_o = L.mla_absorb_out_pre_workspace_bytes(ctypes.byref(d), 2)
    assert need_o > 0
    assert L.mla_absorb_out_pre(ctypes.byref(d), 2, 0, None, FAKE, FAKE, need_o, FAKE, None) == 1
    assert L.mla_absorb_out_pre(ctypes.byref(d), 2, 0, FAKE, FAKE, FAKE, need_o - 1, FAKE, None) == 3
    assert L.mla_absorb_out_pre(ctypes.byref(d), 2, 3, FAKE, FAKE, FAKE, need_o, FAKE, None) == 1  # fp8 weights
    assert L.mla_absorb_out_pre(ctypes.byref(d), 0, 0, None, None, None, 0, None, None) == 0


def test_prefill_tables_validation(L):
    paged = _cache(page_size=64, t_cap=128, block_table=0x3000, max_pages=2, num_pages=4)
    assert L.mla_prefill_tables(None, 2, 4, FAKE, FAKE, FAKE, None) == 1
    assert L.mla_prefill_tables(ctypes.byref(_cache()), 2, 4, FAKE, FAKE, FAKE, None) == 1   # contiguous
    assert b"paged" in L.mla_last_error()
    assert L.mla_prefill_tables(ctypes.byref(paged), 2, 0, FAKE, FAKE, FAKE, None) == 1     # C >= 1
    assert L.mla_prefill_tables(ctypes.byref(paged), 2, 4, None, FAKE, FAKE, None) == 1
    assert L.mla_prefill_tables(ctypes.byref(paged), 2, 4, ctypes.c_void_p(0x1002), FAKE, FAKE, None) == 1
    assert L.mla_prefill_tables(ctypes.byref(paged), 0, 4, None, None, None, None) == 0     # empty batch


def test_naive_prefill_validation(L):
    """The naive-form prefill calls check their arguments, and refuse shapes and types they have no
    kernels for, before touching the device."""
    v2 = _dims(d=5120, n_h=128, d_h=128, d_c=512, d_cq=1536, d_r=64)
    run = _dims()
    paged = _cache(page_size=64, t_cap=4096, block_table=0x3000, max_pages=64, num_pages=64)
    W = [FAKE] * 5
    need_q = L.mla_absorb_q_workspace_bytes(ctypes.byref(v2), 4)
    # absorb_q_naive: bf16 weights at the V2 head shape only
    assert L.mla_absorb_q_naive(ctypes.byref(run), 4, 2, FAKE, *W, FAKE, 1 << 40, FAKE, FAKE, FAKE, None) == 2
    assert L.mla_absorb_q_naive(ctypes.byref(v2), 4, 0, FAKE, *W, FAKE, 1 << 40, FAKE, FAKE, FAKE, None) == 2
    assert L.mla_absorb_q_naive(ctypes.byref(v2), 4, 2, None, *W, FAKE, 1 << 40, FAKE, FAKE, FAKE, None) == 1
    assert L.mla_absorb_q_naive(ctypes.byref(v2), 4, 2, FAKE, *W, FAKE, need_q - 1, FAKE, FAKE, FAKE, None) == 3
    assert L.mla_absorb_q_naive(ctypes.byref(v2), 0, 2, *[None] * 6, None, 0, None, None, None, None) == 0
    # workspace: gathered rows (d_c + d_r bf16) plus expanded K and V (2 n_h d_h bf16) per context row
    need = L.mla_prefill_naive_workspace_bytes(ctypes.byref(v2), 2, 1000)
    assert need >= 2 * 1000 * (576 * 2 + 2 * 16384 * 2)
    assert L.mla_prefill_naive_workspace_bytes(ctypes.byref(v2), 0, 1000) == 0
    attn = L.mla_prefill_naive_attn
    ok = (FAKE, FAKE, ctypes.byref(paged), FAKE)
    assert attn(ctypes.byref(v2), 2, 64, 2, *ok, 1000, FAKE, FAKE, FAKE, need - 1, FAKE, None) == 3
    assert attn(ctypes.byref(v2), 2, 64, 2, *ok, 5000, FAKE, FAKE, FAKE, 1 << 40, FAKE, None) == 1  # > capacity
    assert b"capacity" in L.mla_last_error()
    assert attn(ctypes.byref(v2), 2, 64, 2, *ok, 32, FAKE, FAKE, FAKE, 1 << 40, FAKE, None) == 1    # max_ctx < C
    assert attn(ctypes.byref(v2), 2, 0, 2, *ok, 1000, FAKE, FAKE, FAKE, 1 << 40, FAKE, None) == 1   # C >= 1
    fp8 = _cache(dtype=3, scales=0x2000, page_size=64, t_cap=4096, block_table=0x3000, max_pages=64, num_pages=64)
    assert attn(ctypes.byref(v2), 2, 64, 2, FAKE, FAKE, ctypes.byref(fp8), FAKE, 1000, FAKE, FAKE, FAKE, 1 << 40,
                FAKE, None) == 2                                                                    # bf16 cache only
    assert attn(ctypes.byref(run), 2, 64, 2, *ok, 1000, FAKE, FAKE, FAKE, 1 << 40, FAKE, None) == 2
    assert attn(ctypes.byref(v2), 2, 64, 2, FAKE, FAKE, ctypes.byref(paged), None, 1000, FAKE, FAKE, FAKE, 1 << 40,
                FAKE, None) == 1                                                                    # p0 NULL
    assert attn(ctypes.byref(v2), 0, 64, 2, None, None, ctypes.byref(paged), None, 1000, None, None, None, 0, None,
                None) == 0
    # output projection
    need_o = L.mla_output_proj_workspace_bytes(ctypes.byref(v2), 512)
    assert L.mla_output_proj(ctypes.byref(v2), 512, 2, 2, None, FAKE, FAKE, need_o, FAKE, None) == 1
    if need_o > 0:
        assert L.mla_output_proj(ctypes.byref(v2), 512, 2, 2, FAKE, FAKE, FAKE, need_o - 1, FAKE, None) == 3
    assert L.mla_output_proj(ctypes.byref(v2), 512, 0, 0, FAKE, FAKE, FAKE, need_o, FAKE, None) == 2
    assert L.mla_output_proj(ctypes.byref(v2), 512, 2, 1, FAKE, FAKE, FAKE, need_o, FAKE, None) == 1  # f16 o
    assert L.mla_output_proj(ctypes.byref(v2), 0, 2, 0, None, None, None, 0, None, None) == 0


def test_combine_absorb_out_validation(L):
    """The fused combine + absorb_out call checks both workspaces and refuses the shapes it has no
    kernel for (the caller then uses mla_combine + mla_absorb_out)."""
    v2 = _dims(d=5120, n_h=128, d_h=128, d_c=512, d_cq=1536, d_r=64)
    run = _dims()
    f = L.mla_combine_absorb_out
    need_d = L.mla_decode_workspace_bytes(ctypes.byref(v2), 4, 8)
    need_o = L.mla_absorb_out_workspace_bytes(ctypes.byref(v2), 4)
    assert f(ctypes.byref(run), 4, 2, 8, FAKE, 1 << 40, FAKE, FAKE, FAKE, 1 << 40, FAKE, None, None) == 2
    assert f(ctypes.byref(v2), 4, 0, 8, FAKE, 1 << 40, FAKE, FAKE, FAKE, 1 << 40, FAKE, None, None) == 2
    assert f(ctypes.byref(v2), 4, 2, 8, FAKE, need_d - 1, FAKE, FAKE, FAKE, need_o, FAKE, None, None) == 3
    assert f(ctypes.byref(v2), 4, 2, 8, FAKE, need_d, FAKE, FAKE, FAKE, need_o - 1, FAKE, None, None) == 3
    assert f(ctypes.byref(v2), 4, 2, 8, None, need_d, FAKE, FAKE, FAKE, need_o, FAKE, None, None) == 1
    assert f(ctypes.byref(v2), 4, 2, 8, FAKE, need_d, FAKE, FAKE, FAKE, need_o, FAKE, ctypes.c_void_p(0x1002),
             None) == 1                                                                             # lse alignment
    assert f(ctypes.byref(v2), 4, 2, 2000, FAKE, need_d, FAKE, FAKE, FAKE, need_o, FAKE, None, None) == 1
    assert f(ctypes.byref(v2), 0, 2, 8, None, 0, None, None, None, 0, None, None, None) == 0


def test_alignment_validation(L):
    """Kernels use 16-byte vector accesses: misaligned tensor pointers are rejected up front."""
    d = _dims()
    odd = ctypes.c_void_p(0x1004)
    assert L.mla_rope(ctypes.byref(d), 1, FAKE, odd, FAKE, None, None) == 1
    assert b"aligned" in L.mla_last_error()
    c = _cache(rows=0x1008)
    assert L.mla_decode_attn(ctypes.byref(d), 1, FAKE, FAKE, ctypes.byref(c), FAKE, 4, FAKE, 1 << 30, None) == 1
    assert b"aligned" in L.mla_last_error()
    need = L.mla_absorb_out_workspace_bytes(ctypes.byref(d), 2)
    assert L.mla_absorb_out(ctypes.byref(d), 2, 0, FAKE, FAKE, FAKE, odd, need, FAKE, None) == 1
    assert b"aligned" in L.mla_last_error()


def test_stream_read_validation(L):
    sink = ctypes.c_void_p(0x2000)
    assert L.mla_stream_read(None, 16, sink, None) == 1
    assert L.mla_stream_read(FAKE, 0, sink, None) == 1
    assert L.mla_stream_read(FAKE, 24, sink, None) == 1
    assert b"multiple of 16" in L.mla_last_error()
    assert L.mla_stream_read(ctypes.c_void_p(0x1008), 32, sink, None) == 1
    assert L.mla_stream_read(FAKE, 32, None, None) == 1
