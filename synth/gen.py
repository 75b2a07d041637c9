"""Seeded draws for one decode step of one attention layer.

Draw order (fixed, one torch.Generator per case): W^DQ, W^UQ, W^QR, W^DKV, W^KR, W^UK, W^UV, W^O,
then h (the query token of every sequence), then the context lengths, then the page permutation,
then the prefix cache rows sequence by sequence.

The prefix rows (positions 0 .. T_b-2) are state handed to the decode step. They are drawn
directly as N(0, sigma_row) values; the rotary half is already "post-rotation" data, which any
Gaussian vector with independent entries is, because a rotation maps that distribution to itself.
Row T_b-1 (the current token) is left empty: the decode step computes and appends it.

Weights are stored as [out, in] so that y = W x, matching the pages' notation.
"""
from dataclasses import dataclass
from typing import Dict, Optional

import torch

from .configs import Config

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
WEIGHT_NAMES = ("W_dq", "W_uq", "W_qr", "W_dkv", "W_kr", "W_uk", "W_uv", "W_o")


def weight_shapes(dims) -> Dict[str, tuple]:
    return {
        "W_dq": (dims.d_cq, dims.d),
        "W_uq": (dims.n_h * dims.d_h, dims.d_cq),
        "W_qr": (dims.n_h * dims.d_r, dims.d_cq),
        "W_dkv": (dims.d_c, dims.d),
        "W_kr": (dims.d_r, dims.d),
        "W_uk": (dims.n_h * dims.d_h, dims.d_c),
        "W_uv": (dims.n_h * dims.d_h, dims.d_c),
        "W_o": (dims.d, dims.n_h * dims.d_h),
    }


@dataclass
class Case:
    cfg: Config
    weights: Dict[str, torch.Tensor]     # storage dtype (cfg.wdtype)
    h: torch.Tensor                      # [B, d] storage dtype
    seq_lens: torch.Tensor               # [B] int32, includes the current token
    t_cap: int                           # contiguous capacity (max T_b)
    # cache payload. For f32/f16/bf16: `rows` holds the stored rows (contiguous [B, t_cap, row] or
    # paged pool [P, page, row]). For fp8 / fp6: `rows32` holds float32 source rows in the same
    # layout and each side quantises them with its own encoder.
    rows: Optional[torch.Tensor] = None
    rows32: Optional[torch.Tensor] = None
    block_table: Optional[torch.Tensor] = None   # [B, max_pages] int32, -1 = unused
    num_pages: int = 0
    # chunked prefill (make_prefill_case): C new tokens per sequence after p0[b] stored rows
    h_chunk: Optional[torch.Tensor] = None       # [B, C, d] storage dtype
    p0: Optional[torch.Tensor] = None            # [B] int32
    chunk: int = 0

    @property
    def B(self) -> int:
        return int(self.h.shape[0])

    @property
    def dims(self):
        return self.cfg.dims

    def row_source(self) -> torch.Tensor:
        return self.rows32 if self.rows32 is not None else self.rows

    def prefix_rows(self, b: int) -> torch.Tensor:
        """Rows 0..T_b-2 of sequence b, in the stored/source dtype, gathered in token order."""
        T = int(self.seq_lens[b])
        src = self.row_source()
        if self.cfg.layout == "contiguous":
            return src[b, : T - 1]
        ps = self.cfg.page_size
        n_pages = (T + ps - 1) // ps
        pages = self.block_table[b, :n_pages].to(torch.long).to(src.device)
        return src[pages].reshape(n_pages * ps, -1)[: T - 1]


def _lengths(cfg: Config, B: int, g: torch.Generator, T_override) -> torch.Tensor:
    if T_override is not None:
        if isinstance(T_override, int):
            return torch.full((B,), T_override, dtype=torch.int32)
        t = torch.as_tensor(T_override, dtype=torch.int32)
        assert t.numel() == B
        return t.clone()
    kind = cfg.lens[0]
    if kind == "fixed":
        return torch.full((B,), int(cfg.lens[1]), dtype=torch.int32)
    lo, hi = int(cfg.lens[1]), int(cfg.lens[2])
    return torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64).to(torch.int32)


def make_case(cfg: Config, device="cpu", B: Optional[int] = None, T=None, seed: Optional[int] = None,
              layout: Optional[str] = None, cdtype: Optional[str] = None) -> Case:
    """Draw one seeded decode case. `B`, `T` (int or per-sequence list), `layout` and `cdtype`
    override the config (used for small parity cases with the config's distributions)."""
    if layout is not None or cdtype is not None:
        cfg = cfg.with_(layout=layout or cfg.layout, cdtype=cdtype or cfg.cdtype)
    dims = cfg.dims
    B = cfg.batch if B is None else B
    g = torch.Generator(device="cpu")
    g.manual_seed(cfg.seed if seed is None else seed)
    wdt = TORCH_DTYPE[cfg.wdtype]

    weights = {}
    for name, shape in weight_shapes(dims).items():
        w = torch.randn(shape, generator=g, dtype=torch.float32) * cfg.sigma_w
        if name in ("W_uq", "W_qr"):
            w = w * cfg.kappa
        weights[name] = w.to(wdt).to(device)
    h = (torch.randn((B, dims.d), generator=g, dtype=torch.float32) * cfg.sigma_h).to(wdt).to(device)
    seq_lens = _lengths(cfg, B, g, T)
    assert int(seq_lens.min()) >= 1
    t_cap = int(seq_lens.max())

    case = Case(cfg=cfg, weights=weights, h=h, seq_lens=seq_lens.to(device), t_cap=t_cap)
    row = dims.row
    src_dt = torch.float32 if cfg.cdtype in ("f32", "fp8_e4m3", "fp6_e2m3") else TORCH_DTYPE[cfg.cdtype]

    # prefix rows are drawn on the target device (the large configs hold billions of values)
    gd = torch.Generator(device=device)
    gd.manual_seed((cfg.seed if seed is None else seed) * 7919 + 17)
    if cfg.layout == "contiguous":
        buf = torch.zeros((B, t_cap, row), dtype=src_dt, device=device)
        for b in range(B):
            n = int(seq_lens[b]) - 1
            if n > 0:
                buf[b, :n] = (torch.randn((n, row), generator=gd, device=device) * cfg.sigma_row).to(src_dt)
    else:
        ps = cfg.page_size
        pages_per = [(int(t) + ps - 1) // ps for t in seq_lens.tolist()]
        P = sum(pages_per)
        perm = torch.randperm(P, generator=g).to(torch.int32)
        max_pages = max(pages_per)
        bt = torch.full((B, max_pages), -1, dtype=torch.int32)
        k = 0
        for b in range(B):
            bt[b, : pages_per[b]] = perm[k: k + pages_per[b]]
            k += pages_per[b]
        buf = torch.zeros((P, ps, row), dtype=src_dt, device=device)
        for b in range(B):
            n = int(seq_lens[b]) - 1
            if n <= 0:
                continue
            vals = (torch.randn((n, row), generator=gd, device=device) * cfg.sigma_row).to(src_dt)
            npg = (n + ps - 1) // ps
            padded = torch.zeros((npg * ps, row), dtype=src_dt, device=device)
            padded[:n] = vals
            idx = bt[b, :npg].to(torch.long).to(device)
            buf[idx] = padded.view(npg, ps, row)
        case.block_table = bt.to(device)
        case.num_pages = P
    if cfg.cdtype in ("fp8_e4m3", "fp6_e2m3"):
        case.rows32 = buf
    else:
        case.rows = buf
    return case


def make_prefill_case(cfg: Config, p0, C: int, device="cpu", seed: Optional[int] = None):
    """A chunked-prefill case: sequence b holds p0[b] stored rows (the config's prefix-row draw,
    paged layout) and receives C new tokens whose hidden states h_chunk [B, C, d] are drawn like
    the decode step's h. Pages cover p0[b] + C rows."""
    cfg = cfg.with_(layout="paged")
    B = len(p0)
    case = make_case(cfg, device=device, B=B, T=[int(p) + C for p in p0], seed=seed)
    g = torch.Generator(device="cpu")
    g.manual_seed((cfg.seed if seed is None else seed) * 104729 + 3)
    wdt = TORCH_DTYPE[cfg.wdtype]
    case.h_chunk = (torch.randn((B, C, cfg.dims.d), generator=g, dtype=torch.float32) * cfg.sigma_h).to(wdt).to(device)
    case.p0 = torch.tensor([int(p) for p in p0], dtype=torch.int32, device=device)
    case.chunk = C
    return case
