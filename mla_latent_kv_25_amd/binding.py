"""ctypes binding of libmla.so: argument marshalling only.

Each function here has the name of a C entry point of include/mla.h (without the `mla_` prefix)
and does nothing but check tensor placement/dtype/contiguity, pass raw pointers and the current
HIP stream, and raise MLAError on a non-zero status. Every step of the computation runs in the
library's kernels; there is no fallback. PyTorch is used only for device memory and streams.
"""
import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla.so")

F32, F16, BF16, FP8_E4M3 = 0, 1, 2, 3
DTYPE_CODE = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}
FP6_E2M3 = 4
STORAGE_CODE = {"f32": F32, "f16": F16, "bf16": BF16, "fp8_e4m3": FP8_E4M3, "fp6_e2m3": FP6_E2M3}
# bytes of one cached row of `row` elements in each storage type
def row_bytes(dtype: str, row: int) -> int:
    return {"f32": 4 * row, "f16": 2 * row, "bf16": 2 * row, "fp8_e4m3": row, "fp6_e2m3": row * 6 // 8}[dtype]


class MLAError(RuntimeError):
    pass


class Dims(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("n_h", ctypes.c_int32), ("d_h", ctypes.c_int32),
                ("d_c", ctypes.c_int32), ("d_cq", ctypes.c_int32), ("d_r", ctypes.c_int32),
                ("rope_base", ctypes.c_double), ("sm_scale", ctypes.c_float),
                ("yarn_factor", ctypes.c_float), ("yarn_orig_len", ctypes.c_int32),
                ("yarn_alpha", ctypes.c_float), ("yarn_beta", ctypes.c_float)]

    @classmethod
    def of(cls, dims, sm_scale: float = 0.0) -> "Dims":
        """From any object with the dimension attributes; YaRN fields are optional (off)."""
        return cls(dims.d, dims.n_h, dims.d_h, dims.d_c, dims.d_cq, dims.d_r, float(dims.rope_base), sm_scale,
                   float(getattr(dims, "yarn_factor", 1.0)), int(getattr(dims, "yarn_orig_len", 0)),
                   float(getattr(dims, "yarn_alpha", 0.0)), float(getattr(dims, "yarn_beta", 0.0)))


class CCache(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("t_cap", ctypes.c_int64), ("block_table", ctypes.c_void_p),
                ("max_pages", ctypes.c_int32), ("num_pages", ctypes.c_int32)]


_lib = None


def lib():
    """Load libmla.so once. Raises ImportError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                          "or `python mla_latent_kv_25_amd/build.py`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ, ST = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p
    D, C = ctypes.POINTER(Dims), ctypes.POINTER(CCache)
    sig = {
        "mla_absorb_q_workspace_bytes": (SZ, [D, I32]),
        "mla_absorb_q": (I32, [D, I32, I32, P, P, P, P, P, P, P, P, SZ, P, P, P, ST]),
        "mla_rope": (I32, [D, I32, P, P, P, C, ST]),
        "mla_decode_workspace_bytes": (SZ, [D, I32, I32]),
        "mla_decode_attn": (I32, [D, I32, P, P, C, P, I32, P, SZ, ST]),
        "mla_combine": (I32, [D, I32, I32, P, P, SZ, P, P, ST]),
        "mla_absorb_out_workspace_bytes": (SZ, [D, I32]),
        "mla_absorb_out": (I32, [D, I32, I32, P, P, P, P, SZ, P, ST]),
        "mla_absorb_out_noalloc": (I32, [D, I32, I32, P, P, P, P, ST]),
        "mla_prefill_tables": (I32, [C, I32, I32, P, P, P, ST]),
        "mla_precombine": (I32, [D, I32, P, P, P, P, P, P, ST]),
        "mla_absorb_q_pre": (I32, [D, I32, I32, P, P, P, P, P, P, P, SZ, P, P, P, ST]),
        "mla_absorb_out_pre_workspace_bytes": (SZ, [D, I32]),
        "mla_absorb_out_pre": (I32, [D, I32, I32, P, P, P, SZ, P, ST]),
        "mla_cache_store": (I32, [D, C, I32, P, I32, P, I64, ST]),
        "mla_combine_absorb_out": (I32, [D, I32, I32, I32, P, SZ, P, P, P, SZ, P, P, ST]),
        "mla_absorb_q_naive": (I32, [D, I32, I32, P, P, P, P, P, P, P, SZ, P, P, P, ST]),
        "mla_prefill_naive_workspace_bytes": (SZ, [D, I32, I32]),
        "mla_prefill_naive_attn": (I32, [D, I32, I32, I32, P, P, C, P, I32, P, P, P, SZ, P, ST]),
        "mla_output_proj_workspace_bytes": (SZ, [D, I32]),
        "mla_output_proj": (I32, [D, I32, I32, I32, P, P, P, SZ, P, ST]),
        "mla_stream_read": (I32, [P, SZ, P, ST]),
        "mla_status_str": (ctypes.c_char_p, [I32]),
        "mla_last_error": (ctypes.c_char_p, []),
        "mla_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


EXPORTS = ("mla_absorb_q_workspace_bytes", "mla_absorb_q", "mla_rope", "mla_decode_workspace_bytes",
           "mla_decode_attn", "mla_combine", "mla_absorb_out_workspace_bytes", "mla_absorb_out",
           "mla_absorb_out_noalloc",
           "mla_prefill_tables", "mla_precombine", "mla_absorb_q_pre", "mla_absorb_out_pre_workspace_bytes",
           "mla_absorb_out_pre", "mla_cache_store", "mla_combine_absorb_out", "mla_absorb_q_naive", "mla_prefill_naive_workspace_bytes",
           "mla_prefill_naive_attn", "mla_output_proj_workspace_bytes", "mla_output_proj", "mla_stream_read",
           "mla_status_str", "mla_last_error", "mla_version")


def _check(status: int):
    if status != 0:
        L = lib()
        raise MLAError(f"{L.mla_status_str(status).decode()}: {L.mla_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor], dtype=None, name="tensor"):
    if t is None:
        return None
    if not t.is_cuda:
        raise MLAError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise MLAError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise MLAError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


# ------------------------------------------------------------------------------------------------
@dataclass
class LatentCache:
    """Device buffers of one layer's latent cache (see mla_cache in include/mla.h)."""
    rows: torch.Tensor                       # [B, t_cap, row] or [P, page, row]; uint8 codes for fp8,
                                             # [.., row * 6 / 8] packed bytes for fp6
    dtype: str                               # "f32" | "f16" | "bf16" | "fp8_e4m3"
    t_cap: int
    scales: Optional[torch.Tensor] = None    # fp8: float32 per row
    block_table: Optional[torch.Tensor] = None
    page_size: int = 0

    @classmethod
    def contiguous(cls, B, t_cap, row, dtype, device="cuda"):
        if dtype in ("fp8_e4m3", "fp6_e2m3"):
            return cls(torch.zeros((B, t_cap, row_bytes(dtype, row)), dtype=torch.uint8, device=device), dtype, t_cap,
                       scales=torch.ones((B, t_cap), dtype=torch.float32, device=device))
        tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
        return cls(torch.zeros((B, t_cap, row), dtype=tdt, device=device), dtype, t_cap)

    @classmethod
    def paged(cls, num_pages, page_size, row, dtype, block_table, device="cuda"):
        max_pages = int(block_table.shape[1])
        if dtype in ("fp8_e4m3", "fp6_e2m3"):
            return cls(torch.zeros((num_pages, page_size, row_bytes(dtype, row)), dtype=torch.uint8, device=device), dtype,
                       max_pages * page_size, scales=torch.ones((num_pages, page_size), dtype=torch.float32,
                                                               device=device),
                       block_table=block_table, page_size=page_size)
        tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
        return cls(torch.zeros((num_pages, page_size, row), dtype=tdt, device=device), dtype,
                   max_pages * page_size, block_table=block_table, page_size=page_size)

    def c(self) -> CCache:
        bt = self.block_table
        return CCache(_ptr(self.rows, name="cache rows"), _ptr(self.scales, torch.float32, "cache scales"),
                      STORAGE_CODE[self.dtype], self.page_size, self.t_cap,
                      _ptr(bt, torch.int32, "block_table") if bt is not None else None,
                      int(bt.shape[1]) if bt is not None else 0,
                      int(self.rows.shape[0]) if self.page_size else 0)


# ------------------------------------------------------------------------------------------------
def absorb_q_workspace_bytes(dims: Dims, B: int) -> int:
    return lib().mla_absorb_q_workspace_bytes(ctypes.byref(dims), B)


def decode_workspace_bytes(dims: Dims, B: int, num_splits: int) -> int:
    return lib().mla_decode_workspace_bytes(ctypes.byref(dims), B, num_splits)


def absorb_out_workspace_bytes(dims: Dims, B: int) -> int:
    return lib().mla_absorb_out_workspace_bytes(ctypes.byref(dims), B)


def absorb_q(dims: Dims, h, W, workspace, q_lat, q_pe, kv_new):
    """W: dict with W_dq, W_uq, W_qr, W_uk, W_dkv, W_kr (same dtype as h)."""
    wdt = DTYPE_CODE[h.dtype]
    _check(lib().mla_absorb_q(ctypes.byref(dims), h.shape[0], wdt, _ptr(h, name="h"),
                              *[_ptr(W[k], h.dtype, k) for k in ("W_dq", "W_uq", "W_qr", "W_uk", "W_dkv", "W_kr")],
                              _ptr(workspace, name="workspace"), workspace.numel() * workspace.element_size(),
                              _ptr(q_lat, torch.float32, "q_lat"), _ptr(q_pe, torch.float32, "q_pe"),
                              _ptr(kv_new, torch.float32, "kv_new"), _stream()))


def rope(dims: Dims, seq_lens, q_pe, kv_new, cache: Optional[LatentCache] = None):
    cc = cache.c() if cache is not None else None
    _check(lib().mla_rope(ctypes.byref(dims), seq_lens.shape[0], _ptr(seq_lens, torch.int32, "seq_lens"),
                          _ptr(q_pe, torch.float32, "q_pe"), _ptr(kv_new, torch.float32, "kv_new"),
                          ctypes.byref(cc) if cc is not None else None, _stream()))


def decode_attn(dims: Dims, q_lat, q_pe, cache: LatentCache, seq_lens, num_splits: int, workspace):
    cc = cache.c()
    _check(lib().mla_decode_attn(ctypes.byref(dims), seq_lens.shape[0], _ptr(q_lat, torch.float32, "q_lat"),
                                 _ptr(q_pe, torch.float32, "q_pe"), ctypes.byref(cc),
                                 _ptr(seq_lens, torch.int32, "seq_lens"), num_splits,
                                 _ptr(workspace, name="workspace"),
                                 workspace.numel() * workspace.element_size(), _stream()))


def combine(dims: Dims, num_splits: int, seq_lens, workspace, o_lat, lse=None):
    _check(lib().mla_combine(ctypes.byref(dims), seq_lens.shape[0], num_splits,
                             _ptr(seq_lens, torch.int32, "seq_lens"), _ptr(workspace, name="workspace"),
                             workspace.numel() * workspace.element_size(), _ptr(o_lat, torch.float32, "o_lat"),
                             _ptr(lse, torch.float32, "lse"), _stream()))


def absorb_out(dims: Dims, o_lat, W_uv, W_o, workspace, u):
    wdt = DTYPE_CODE[W_uv.dtype]
    _check(lib().mla_absorb_out(ctypes.byref(dims), o_lat.shape[0], wdt, _ptr(o_lat, torch.float32, "o_lat"),
                                _ptr(W_uv, name="W_uv"), _ptr(W_o, W_uv.dtype, "W_o"),
                                _ptr(workspace, name="workspace"), workspace.numel() * workspace.element_size(),
                                _ptr(u, torch.float32, "u"), _stream()))


def combine_absorb_out(dims: Dims, num_splits: int, dec_workspace, W_uv, W_o, workspace, u, lse=None):
    """mla_combine + mla_absorb_out fused: u [B, d] (and lse [B, n_h] if given) from the pieces."""
    _check(lib().mla_combine_absorb_out(ctypes.byref(dims), u.shape[0], DTYPE_CODE[W_uv.dtype], num_splits,
                                        _ptr(dec_workspace, name="dec_workspace"), dec_workspace.numel(),
                                        _ptr(W_uv, name="W_uv"), _ptr(W_o, W_uv.dtype, "W_o"),
                                        _ptr(workspace, name="workspace"), workspace.numel(),
                                        _ptr(u, torch.float32, "u"), _ptr(lse, torch.float32, "lse"), _stream()))


def absorb_out_noalloc(dims: Dims, o_lat, W_uv, W_o, u):
    """absorb_out with the library's static scratch in place of a workspace (no allocation)."""
    wdt = DTYPE_CODE[W_uv.dtype]
    _check(lib().mla_absorb_out_noalloc(ctypes.byref(dims), o_lat.shape[0], wdt, _ptr(o_lat, torch.float32, "o_lat"),
                                        _ptr(W_uv, name="W_uv"), _ptr(W_o, W_uv.dtype, "W_o"),
                                        _ptr(u, torch.float32, "u"), _stream()))


def precombine(dims: Dims, W, Wq_pre=None, Wo_pre=None):
    """Build the pre-combined W~^Q [n_h*d_c, d_cq] and / or W~^O [d, n_h*d_c] (weight dtype) from
    W["W_uq"], W["W_uk"] / W["W_uv"], W["W_o"]."""
    dt = W["W_uq"].dtype
    _check(lib().mla_precombine(ctypes.byref(dims), DTYPE_CODE[dt],
                                *[_ptr(W[k], dt, k) for k in ("W_uq", "W_uk", "W_uv", "W_o")],
                                _ptr(Wq_pre, dt, "Wq_pre"), _ptr(Wo_pre, dt, "Wo_pre"), _stream()))


def absorb_q_pre(dims: Dims, h, W, Wq_pre, workspace, q_lat, q_pe, kv_new):
    """absorb_q with the pre-combined W~^Q (W_uq and W_uk unused)."""
    wdt = DTYPE_CODE[h.dtype]
    _check(lib().mla_absorb_q_pre(ctypes.byref(dims), h.shape[0], wdt, _ptr(h, name="h"),
                                  _ptr(W["W_dq"], h.dtype, "W_dq"), _ptr(Wq_pre, h.dtype, "Wq_pre"),
                                  _ptr(W["W_qr"], h.dtype, "W_qr"), _ptr(W["W_dkv"], h.dtype, "W_dkv"),
                                  _ptr(W["W_kr"], h.dtype, "W_kr"),
                                  _ptr(workspace, name="workspace"), workspace.numel() * workspace.element_size(),
                                  _ptr(q_lat, torch.float32, "q_lat"), _ptr(q_pe, torch.float32, "q_pe"),
                                  _ptr(kv_new, torch.float32, "kv_new"), _stream()))


def absorb_out_pre_workspace_bytes(dims: Dims, B: int) -> int:
    return lib().mla_absorb_out_pre_workspace_bytes(ctypes.byref(dims), B)


def absorb_out_pre(dims: Dims, o_lat, Wo_pre, workspace, u):
    wdt = DTYPE_CODE[Wo_pre.dtype]
    _check(lib().mla_absorb_out_pre(ctypes.byref(dims), o_lat.shape[0], wdt, _ptr(o_lat, torch.float32, "o_lat"),
                                    _ptr(Wo_pre, name="Wo_pre"), _ptr(workspace, name="workspace"),
                                    workspace.numel() * workspace.element_size(), _ptr(u, torch.float32, "u"),
                                    _stream()))


def prefill_tables(cache: LatentCache, B: int, C: int, p0, seq_lens_out, block_table_out):
    """Lengths and block tables of the B * C causal pseudo-sequences of a C-token prefill chunk."""
    cc = cache.c()
    _check(lib().mla_prefill_tables(ctypes.byref(cc), B, C, _ptr(p0, torch.int32, "p0"),
                                    _ptr(seq_lens_out, torch.int32, "seq_lens_out"),
                                    _ptr(block_table_out, torch.int32, "block_table_out"), _stream()))


def cache_store(dims: Dims, cache: LatentCache, n_rows, max_rows: int, src, src_stride: int):
    cc = cache.c()
    _check(lib().mla_cache_store(ctypes.byref(dims), ctypes.byref(cc), n_rows.shape[0],
                                 _ptr(n_rows, torch.int32, "n_rows"), max_rows,
                                 _ptr(src, torch.float32, "src"), src_stride, _stream()))


def absorb_q_naive(dims: Dims, h, W, workspace, q_c, q_pe, kv_new):
    """Query and KV pathways without the W^UK absorption: q_c [B, n_h, d_h] float32."""
    wdt = DTYPE_CODE[h.dtype]
    _check(lib().mla_absorb_q_naive(ctypes.byref(dims), h.shape[0], wdt, _ptr(h, name="h"),
                                    _ptr(W["W_dq"], h.dtype, "W_dq"), _ptr(W["W_uq"], h.dtype, "W_uq"),
                                    _ptr(W["W_qr"], h.dtype, "W_qr"), _ptr(W["W_dkv"], h.dtype, "W_dkv"),
                                    _ptr(W["W_kr"], h.dtype, "W_kr"), _ptr(workspace, name="workspace"),
                                    workspace.numel(), _ptr(q_c, torch.float32, "q_c"),
                                    _ptr(q_pe, torch.float32, "q_pe"), _ptr(kv_new, torch.float32, "kv_new"),
                                    _stream()))


def prefill_naive_workspace_bytes(dims: Dims, B: int, max_ctx: int) -> int:
    return lib().mla_prefill_naive_workspace_bytes(ctypes.byref(dims), B, max_ctx)


def prefill_naive_attn(dims: Dims, B: int, C: int, q_c, q_pe, cache: LatentCache, p0, max_ctx: int, W_uk, W_uv,
                       workspace, o):
    """Causal attention of a C-token chunk per sequence on the expanded keys and values."""
    cc = cache.c()
    _check(lib().mla_prefill_naive_attn(ctypes.byref(dims), B, C, DTYPE_CODE[W_uk.dtype],
                                        _ptr(q_c, torch.float32, "q_c"), _ptr(q_pe, torch.float32, "q_pe"),
                                        ctypes.byref(cc), _ptr(p0, torch.int32, "p0"), max_ctx,
                                        _ptr(W_uk, name="W_uk"), _ptr(W_uv, W_uk.dtype, "W_uv"),
                                        _ptr(workspace, name="workspace"), workspace.numel(),
                                        _ptr(o, torch.bfloat16, "o"), _stream()))


def output_proj_workspace_bytes(dims: Dims, N: int) -> int:
    return lib().mla_output_proj_workspace_bytes(ctypes.byref(dims), N)


def output_proj(dims: Dims, o, W_o, workspace, u):
    """u = W^O o for o [N, n_h * d_h] float32 or bf16."""
    if o.dtype not in (torch.float32, torch.bfloat16):
        raise MLAError("o must be float32 or bfloat16")
    _check(lib().mla_output_proj(ctypes.byref(dims), o.shape[0], DTYPE_CODE[W_o.dtype], DTYPE_CODE[o.dtype],
                                 _ptr(o, name="o"),
                                 _ptr(W_o, name="W_o"), _ptr(workspace, name="workspace") if workspace is not None
                                 else None, 0 if workspace is None else workspace.numel(),
                                 _ptr(u, torch.float32, "u"), _stream()))


STREAM_SINK_WORDS = 4096  # MLA_STREAM_SINK_WORDS


def stream_read(src, sink):
    """mla_stream_read: read every byte of the device tensor `src` once (the read-stream ceiling
    measurement); `sink` is a device int32/uint32 tensor of STREAM_SINK_WORDS words."""
    if sink.numel() < STREAM_SINK_WORDS or sink.element_size() != 4:
        raise MLAError(f"sink must hold {STREAM_SINK_WORDS} 32-bit words")
    _check(lib().mla_stream_read(_ptr(src, None, "src"), src.numel() * src.element_size(),
                                 _ptr(sink, None, "sink"), _stream()))


def version() -> str:
    return lib().mla_version().decode()


# ------------------------------------------------------------------------------------------------
def fused_output_suits(B: int, num_splits: int, device="cuda") -> bool:
    """Whether mla_combine_absorb_out is the faster output call for B sequences over num_splits
    ranges (0: the library's default of one range per CU at the DeepSeek-V2 shape). Its workgroups
    (one head, 32 sequences) fetch up to six pieces of a sequence in one round trip and walk longer
    piece lists one piece at a time; with more than about four ranges per sequence (long contexts
    over a few sequences) mla_combine + mla_absorb_out are faster (B = 4 x 131072 tokens: 61 against
    123 us)."""
    G = num_splits or torch.cuda.get_device_properties(device).multi_processor_count
    return G <= 4 * B


class DecodeStep:
    """Buffers for the five calls of one decode step, allocated once (torch), reused per step.
    fused=True runs combine and absorb_out as the one call mla_combine_absorb_out (bf16 weights; other
    weight types take the two calls); fused="auto" does so where fused_output_suits says it is faster."""

    def __init__(self, dims, B: int, num_splits: int, device="cuda", sm_scale: float = 0.0, fused=False):
        self.dims = Dims.of(dims, sm_scale)
        self.B = B
        self.num_splits = num_splits
        self.fused = fused_output_suits(B, num_splits, device) if fused == "auto" else bool(fused)
        f32 = dict(dtype=torch.float32, device=device)
        self.q_lat = torch.empty((B, dims.n_h, dims.d_c), **f32)
        self.q_pe = torch.empty((B, dims.n_h, dims.d_r), **f32)
        self.kv_new = torch.empty((B, dims.d_c + dims.d_r), **f32)
        self.o_lat = torch.empty((B, dims.n_h, dims.d_c), **f32)
        self.lse = torch.empty((B, dims.n_h), **f32)
        self.u = torch.empty((B, dims.d), **f32)
        u8 = dict(dtype=torch.uint8, device=device)
        self.ws_q = torch.empty(max(1, absorb_q_workspace_bytes(self.dims, B)), **u8)
        self.ws_d = torch.empty(max(1, decode_workspace_bytes(self.dims, B, num_splits)), **u8)
        self.ws_o = torch.empty(max(1, absorb_out_workspace_bytes(self.dims, B)), **u8)

    def run(self, h, W, cache: LatentCache, seq_lens):
        """absorb_q -> rope (append) -> decode_attn -> combine -> absorb_out; returns u [B, d]."""
        absorb_q(self.dims, h, W, self.ws_q, self.q_lat, self.q_pe, self.kv_new)
        rope(self.dims, seq_lens, self.q_pe, self.kv_new, cache)
        decode_attn(self.dims, self.q_lat, self.q_pe, cache, seq_lens, self.num_splits, self.ws_d)
        if self.fused and W["W_uv"].dtype == torch.bfloat16:
            combine_absorb_out(self.dims, self.num_splits, self.ws_d, W["W_uv"], W["W_o"], self.ws_o, self.u, self.lse)
        else:
            combine(self.dims, self.num_splits, seq_lens, self.ws_d, self.o_lat, self.lse)
            absorb_out(self.dims, self.o_lat, W["W_uv"], W["W_o"], self.ws_o, self.u)
        return self.u


class PrecombinedStep(DecodeStep):
    """The decode step in the pre-combined form: W~^Q and W~^O are built once (precombine), then
    each step runs absorb_q_pre -> rope -> decode_attn -> combine -> absorb_out_pre."""

    def __init__(self, dims, B: int, num_splits: int, W, device="cuda", sm_scale: float = 0.0):
        super().__init__(dims, B, num_splits, device, sm_scale)
        dt = W["W_uq"].dtype
        self.Wq_pre = torch.empty((dims.n_h * dims.d_c, dims.d_cq), dtype=dt, device=device)
        self.Wo_pre = torch.empty((dims.d, dims.n_h * dims.d_c), dtype=dt, device=device)
        precombine(self.dims, W, self.Wq_pre, self.Wo_pre)
        self.ws_op = torch.empty(max(1, absorb_out_pre_workspace_bytes(self.dims, B)), dtype=torch.uint8,
                                 device=device)

    def run(self, h, W, cache: LatentCache, seq_lens):
        absorb_q_pre(self.dims, h, W, self.Wq_pre, self.ws_q, self.q_lat, self.q_pe, self.kv_new)
        rope(self.dims, seq_lens, self.q_pe, self.kv_new, cache)
        decode_attn(self.dims, self.q_lat, self.q_pe, cache, seq_lens, self.num_splits, self.ws_d)
        combine(self.dims, self.num_splits, seq_lens, self.ws_d, self.o_lat, self.lse)
        absorb_out_pre(self.dims, self.o_lat, self.Wo_pre, self.ws_op, self.u)
        return self.u


# Chunk length from which the naive form is the faster one (measured crossover at the DeepSeek-V2
# shape, 16 sequences of 2048 stored rows, bf16: between C = 128 and C = 256)
NAIVE_MIN_CHUNK = 160


def naive_form_available(dims, weight_dtype, cache_dtype: str) -> bool:
    """Whether the naive-form calls have kernels for these dims and types (mla_absorb_q_naive,
    mla_prefill_naive_attn, mla_output_proj): d_h 128, d_c 512, d_r 64, the MFMA GEMM shapes
    (d and d_cq multiples of 256, n_h d_h a multiple of 256), bf16 weights and a bf16 cache."""
    return (dims.d_h == 128 and dims.d_c == 512 and dims.d_r == 64 and dims.d % 256 == 0 and dims.d_cq % 256 == 0
            and (dims.n_h * dims.d_h) % 256 == 0 and weight_dtype == torch.bfloat16 and cache_dtype == "bf16")


def choose_prefill_form(dims, C: int, weight_dtype, cache_dtype: str) -> bool:
    """True for the naive form: from NAIVE_MIN_CHUNK chunk tokens on, where it has kernels."""
    return C >= NAIVE_MIN_CHUNK and naive_form_available(dims, weight_dtype, cache_dtype)


class PrefillStep:
    """Chunked prefill: C new tokens per sequence (positions p0[b] .. p0[b] + C - 1) as B * C causal
    pseudo-sequences sharing their sequence's pages (mla_prefill_tables). Every chunk token's row is
    appended, and each token gets its causal output u.
      absorbed form (naive=False): the five decode calls over the pseudo-sequences;
      naive form (naive=True): absorb_q_naive -> rope -> prefill_naive_attn -> output_proj, with
      keys and values expanded for contexts of up to max_ctx rows (p0[b] + C <= max_ctx);
      naive="auto": the naive form from NAIVE_MIN_CHUNK tokens on where it has kernels (weight and
      cache types given as weight_dtype / cache_dtype), the absorbed form otherwise."""

    def __init__(self, dims, B: int, C: int, max_pages: int, num_splits: int = 0, device="cuda",
                 sm_scale: float = 0.0, naive=False, max_ctx: Optional[int] = None,
                 weight_dtype=torch.bfloat16, cache_dtype: str = "bf16"):
        self.B, self.C = B, C
        if naive == "auto":
            naive = max_ctx is not None and choose_prefill_form(dims, C, weight_dtype, cache_dtype)
        self.naive = bool(naive)
        # separate combine and absorb_out: at B * C pseudo-sequences the fused call re-reads W^UV_i
        # per 32 of them and is no faster (C = 64: 571 against 560 us)
        self.step = DecodeStep(dims, B * C, num_splits, device, sm_scale)
        self.dims = self.step.dims
        self.seq_lens = torch.empty(B * C, dtype=torch.int32, device=device)
        self.block_table = torch.empty((B * C, max_pages), dtype=torch.int32, device=device)
        if self.naive:
            if max_ctx is None:
                raise MLAError("the naive form needs max_ctx (bound on p0[b] + C)")
            self.max_ctx = max_ctx
            f32 = dict(dtype=torch.float32, device=device)
            self.q_c = torch.empty((B * C, dims.n_h, dims.d_h), **f32)
            self.o = torch.empty((B * C, dims.n_h * dims.d_h), dtype=torch.bfloat16, device=device)
            u8 = dict(dtype=torch.uint8, device=device)
            self.ws_n = torch.empty(max(1, prefill_naive_workspace_bytes(self.dims, B, max_ctx)), **u8)
            self.ws_p = torch.empty(max(1, output_proj_workspace_bytes(self.dims, B * C)), **u8)

    def run(self, h_chunk, W, cache: LatentCache, p0):
        """h_chunk [B, C, d] (weight dtype); cache: paged, holding p0[b] rows of sequence b."""
        if cache.page_size <= 0:
            raise MLAError("chunked prefill needs a paged cache")
        prefill_tables(cache, self.B, self.C, p0, self.seq_lens, self.block_table)
        view = LatentCache(cache.rows, cache.dtype, cache.t_cap, cache.scales, self.block_table, cache.page_size)
        h = h_chunk.reshape(self.B * self.C, -1).contiguous()
        if not self.naive:
            u = self.step.run(h, W, view, self.seq_lens)
            return u.view(self.B, self.C, -1)
        st = self.step
        absorb_q_naive(self.dims, h, W, st.ws_q, self.q_c, st.q_pe, st.kv_new)
        rope(self.dims, self.seq_lens, st.q_pe, st.kv_new, view)
        prefill_naive_attn(self.dims, self.B, self.C, self.q_c, st.q_pe, cache, p0, self.max_ctx, W["W_uk"],
                           W["W_uv"], self.ws_n, self.o)
        output_proj(self.dims, self.o, W["W_o"], self.ws_p, st.u)
        return st.u.view(self.B, self.C, -1)
