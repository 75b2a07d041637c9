"""Reference decode step of Multi-head Latent Attention — TEST INFRASTRUCTURE ONLY.

Plain numpy in float64. The oracle does NOT use the absorption trick: it rebuilds every past
token's per-head content key and value from the cached latent and runs ordinary multi-head
attention with the decoupled rotary part, exactly as the pages write the method out:

  [Scratch] = "DeepSeek-V2 from Scratch: Multi-head Latent Attention and DeepSeekMoE"
              (prathamp.com), sections 1-7;
  [Visual]  = "DeepSeek-V2" (sghael visual-learn), "Why position needs separate handling";
  [Summary] = noblerworks summary of the DeepSeek-V2 paper, "The matrix-absorption trick".

Where the pages are silent the oracle takes these readings:
  * rotary embedding: consecutive pairs (x_2m, x_2m+1) rotated by pos * base^(-2m/d_r), base
    10000; applied to every head's d_h^R slice of the rotary query and to the shared rotary key;
  * positions are 0-based, cache row j holds position j, the current token sits at T_b - 1 and
    attends to itself (the pages' sums run to j = t inclusive);
  * head i owns row block i of W^UQ, W^QR, W^UK, W^UV and column block i of W^O;
  * the attention weight carries a head index (it depends on the head's query);
  * the softmax scale is 1/sqrt(d_h + d_h^R) in every formulation, including the absorbed one;
  * the appended row is rounded to the storage type before attention reads it.

Pins (tests/test_oracle_pins.py): the absorbed formulation below agrees to 1e-10; a special case
reduces to torch's scaled-dot-product attention; T = 1 closed form; hand-derived tiny case
(tests/golden); rotary invariants and a complex-number formulation; decode step by step equals
causal attention over the whole prefix; the pages' printed softmax example.
"""
from dataclasses import dataclass

import numpy as np

from .encodings import store_rows, load_rows


@dataclass(frozen=True)
class OracleDims:
    d: int
    n_h: int
    d_h: int
    d_c: int
    d_cq: int
    d_r: int
    rope_base: float = 10000.0
    # YaRN extension of the decoupled RoPE: factor s (<= 1: off), original context length L and
    # the ramp bounds alpha < beta, in turns over L
    yarn_factor: float = 1.0
    yarn_orig_len: int = 0
    yarn_alpha: float = 0.0
    yarn_beta: float = 0.0

    @classmethod
    def of(cls, dims) -> "OracleDims":
        return cls(dims.d, dims.n_h, dims.d_h, dims.d_c, dims.d_cq, dims.d_r, float(dims.rope_base),
                   float(getattr(dims, "yarn_factor", 1.0)), int(getattr(dims, "yarn_orig_len", 0)),
                   float(getattr(dims, "yarn_alpha", 0.0)), float(getattr(dims, "yarn_beta", 0.0)))

    @property
    def yarn(self):
        """(s, L, alpha, beta) when the extension is on, else None."""
        if self.yarn_factor <= 1.0:
            return None
        return (self.yarn_factor, self.yarn_orig_len, self.yarn_alpha, self.yarn_beta)


def rope_frequencies(n, base=10000.0, yarn=None):
    """Rotation frequency of each of the n/2 pairs: base^(-2m/n) (the textbook RoPE frequencies).

    With yarn = (s, L, alpha, beta): the DeepSeek-V2 review page ("4. Pre-Training") extends the
    context of the decoupled key with YaRN and gives no formula, so the method is taken as
    published. A pair whose wavelength lambda = 2 pi / theta fits r = L / lambda times into the
    original context L is interpolated by 1/s if r < alpha, kept if r > beta, and blended linearly
    in r in between: theta' = (1 - gamma) theta / s + gamma theta."""
    m = np.arange(n // 2, dtype=np.float64)
    theta = np.power(float(base), -2.0 * m / n)
    if yarn is None or yarn[0] <= 1.0:
        return theta
    s, L, alpha, beta = (float(v) for v in yarn)
    wavelength = 2.0 * np.pi / theta
    turns = L / wavelength
    gamma = np.clip((turns - alpha) / (beta - alpha), 0.0, 1.0)
    return (1.0 - gamma) * theta / s + gamma * theta


def score_scale(dims):
    """Softmax scale of the scores: 1/sqrt(d_h + d_h^R) ([Scratch] section 4.4), times YaRN's
    attention temperature (0.1 ln s + 1)^2 when the extension is on (the published method)."""
    scale = 1.0 / np.sqrt(dims.d_h + dims.d_r)
    y = getattr(dims, "yarn", None)
    if y is not None:
        scale *= (0.1 * np.log(y[0]) + 1.0) ** 2
    return scale


def softmax(z, axis=-1):
    """Softmax with the maximum subtracted first (same value, no overflow)."""
    z = np.asarray(z, dtype=np.float64)
    m = np.max(z, axis=axis, keepdims=True)
    e = np.exp(z - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def rope(x, pos, base=10000.0, yarn=None):
    """Rotary embedding of the last axis of x (even length) at integer position `pos`.

    [Scratch] section 3.1 defines RoPE only as a position-dependent rotation whose query-key dot
    product depends on the position difference; the pair layout and frequencies are the
    textbook ones (see the module docstring), optionally YaRN-extended (rope_frequencies)."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    assert n % 2 == 0
    theta = rope_frequencies(n, base, yarn)
    ang = float(pos) * theta
    c, s = np.cos(ang), np.sin(ang)
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def head_slices(W, dims: OracleDims):
    """Per-head blocks of the weights, [Scratch] sections 2.2, 4.1 and 5.1-5.2.
    Returns (W_uq[i]: d_h x d_cq, W_qr[i]: d_r x d_cq, W_uk[i]: d_h x d_c, W_uv[i]: d_h x d_c,
    W_o[i]: d x d_h)."""
    n, dh, dr = dims.n_h, dims.d_h, dims.d_r
    return (W["W_uq"].reshape(n, dh, dims.d_cq),
            W["W_qr"].reshape(n, dr, dims.d_cq),
            W["W_uk"].reshape(n, dh, dims.d_c),
            W["W_uv"].reshape(n, dh, dims.d_c),
            W["W_o"].reshape(dims.d, n, dh).transpose(1, 0, 2))


def new_token(W, h, pos, dims: OracleDims, cdtype):
    """Query and KV pathways for the current token ([Scratch] section 6).

    Returns q^C [n_h, d_h], q^R [n_h, d_r] (rotated), the cache row [c^KV ; k^R] exactly as
    computed (float64), and the row as stored (payload, scale) and as read back (float64)."""
    cQ = W["W_dq"] @ h                                         # c^Q = W^DQ h
    qC = (W["W_uq"] @ cQ).reshape(dims.n_h, dims.d_h)          # q^C = W^UQ c^Q, split by head
    qR = rope((W["W_qr"] @ cQ).reshape(dims.n_h, dims.d_r), pos, dims.rope_base, dims.yarn)
    cKV = W["W_dkv"] @ h                                       # c^KV = W^DKV h   (cached)
    kR = rope(W["W_kr"] @ h, pos, dims.rope_base, dims.yarn)  # k^R = RoPE(W^KR h) (cached)
    row = np.concatenate([cKV, kR])                            # row layout: latent, then k^R
    payload, scale = store_rows(row[None, :], cdtype)
    read = load_rows(payload, cdtype, scale)[0]
    return qC, qR, row, (payload[0], None if scale is None else scale[0]), read


def decode_step_explicit(W, h, prefix, dims: OracleDims, cdtype, heads=None, want_u=True,
                         chunk=4096):
    """One decode step of one layer for one sequence, with explicit key/value reconstruction.

    W: dict of float64 weights ([out, in]); h: [d] float64; prefix: [T-1, d_c + d_r] float64
    (the stored rows of positions 0..T-2, as the attention reads them).
    heads: optional subset of heads for the diagnostics (u needs all heads).
    Returns dict(u [d], o [n_h, d_h], o_lat [H, d_c], lse [H], row_new, stored_new, alpha_max).
    """
    prefix = np.asarray(prefix, dtype=np.float64).reshape(-1, dims.d_c + dims.d_r)
    T = prefix.shape[0] + 1
    pos = T - 1
    qC, qR, row, stored, read = new_token(W, h, pos, dims, cdtype)
    rows = np.vstack([prefix, read[None, :]])                  # [T, d_c + d_r]
    C, KR = rows[:, : dims.d_c], rows[:, dims.d_c:]
    Wuq, Wqr, Wuk, Wuv, Wo = head_slices(W, dims)
    heads = list(range(dims.n_h)) if heads is None else list(heads)
    if want_u:
        assert len(heads) == dims.n_h
    scale = score_scale(dims)

    # pass 1: scores s[j, i] = [q^C_i ; q^R_i] . [k^C_{j,i} ; k^R_j] / sqrt(d_h + d_r)
    S = np.empty((T, len(heads)))
    for a in range(0, T, chunk):
        Cc = C[a: a + chunk]
        for n, i in enumerate(heads):
            kC = Cc @ Wuk[i].T                                 # k^C_{j,i} = W^UK_i c_j
            k = np.concatenate([kC, KR[a: a + chunk]], axis=1)  # k_{j,i} = [k^C_{j,i}; k^R_j]
            q = np.concatenate([qC[i], qR[i]])                  # q_i = [q^C_i; q^R_i]
            S[a: a + chunk, n] = (k @ q) * scale
    alpha = softmax(S, axis=0)                                 # over the context j
    m = S.max(axis=0)
    lse = m + np.log(np.exp(S - m).sum(axis=0))

    # pass 2: o_i = sum_j alpha_{j,i} v^C_{j,i}, v^C_{j,i} = W^UV_i c_j
    o = np.zeros((len(heads), dims.d_h))
    o_lat = np.zeros((len(heads), dims.d_c))
    for a in range(0, T, chunk):
        Cc = C[a: a + chunk]
        for n, i in enumerate(heads):
            vC = Cc @ Wuv[i].T
            o[n] += alpha[a: a + chunk, n] @ vC
            o_lat[n] += alpha[a: a + chunk, n] @ Cc            # diagnostic only
    out = dict(o=o, o_lat=o_lat, lse=lse, row_new=row, stored_new=stored, read_new=read,
               alpha_max=alpha.max(axis=0), score_std=float(S.std()) if T > 1 else 0.0, T=T)
    if want_u:
        out["u"] = W["W_o"] @ o.reshape(-1)                    # u = W^O [o_1; ...; o_nh]
    return out


def decode_step_absorbed(W, h, prefix, dims: OracleDims, cdtype):
    """Second formulation, used only to pin the first: the absorbed form of [Scratch] section 5.

    q~_i = (W^UK_i)^T q^C_i scores the latent directly; the attention-weighted latent is
    up-projected afterwards by W^UV_i and then W^O_i. Different arithmetic, same exact result."""
    prefix = np.asarray(prefix, dtype=np.float64).reshape(-1, dims.d_c + dims.d_r)
    T = prefix.shape[0] + 1
    qC, qR, row, stored, read = new_token(W, h, T - 1, dims, cdtype)
    rows = np.vstack([prefix, read[None, :]])
    C, KR = rows[:, : dims.d_c], rows[:, dims.d_c:]
    Wuq, Wqr, Wuk, Wuv, Wo = head_slices(W, dims)
    scale = score_scale(dims)
    u = np.zeros(dims.d)
    o_lat = np.zeros((dims.n_h, dims.d_c))
    lse = np.zeros(dims.n_h)
    for i in range(dims.n_h):
        q_abs = Wuk[i].T @ qC[i]                               # (W^UK_i)^T q^C_i, in R^{d_c}
        s = (C @ q_abs + KR @ qR[i]) * scale
        a = softmax(s)
        m = s.max()
        lse[i] = m + np.log(np.exp(s - m).sum())
        o_lat[i] = a @ C                                       # sum_j alpha_j c_j
        u += Wo[i] @ (Wuv[i] @ o_lat[i])                       # W^O_i W^UV_i (sum alpha c)
    return dict(u=u, o_lat=o_lat, lse=lse)


def absorbed_query(W, h, pos, dims: OracleDims):
    """Stage outputs of the query pathway with W^UK absorbed ([Scratch] sections 4.1 and 5.1):
    q~_i = (W^UK_i)^T q^C_i [n_h, d_c], the rotated q^R [n_h, d_r], and the current token's row
    [c^KV ; RoPE(W^KR h)] before storage rounding."""
    qC, qR, row, _, _ = new_token(W, h, pos, dims, "f32")
    _, _, Wuk, _, _ = head_slices(W, dims)
    q_lat = np.stack([Wuk[i].T @ qC[i] for i in range(dims.n_h)])
    return q_lat, qR, row


def output_projection(W, o_lat, dims: OracleDims):
    """u = W^O [W^UV_1 o_lat_1; ...; W^UV_nh o_lat_nh] ([Scratch] sections 5.2 and 6)."""
    _, _, _, Wuv, _ = head_slices(W, dims)
    o = np.stack([Wuv[i] @ o_lat[i] for i in range(dims.n_h)])
    return W["W_o"] @ o.reshape(-1)


def precombined_heads(W, dims: OracleDims, rnd=None):
    """Per-head pre-combined matrices: [Scratch] section 5.1, W~^Q_i = (W^UK_i)^T W^UQ_i (d_c x d_cq),
    and section 5.2, W~^O_i = W^O_i W^UV_i (d x d_c). rnd: optional rounding applied to each matrix
    (the variant stores them in the weight type). Returns [(W~^Q_i, W~^O_i) for i < n_h]."""
    Wuq, _, Wuk, Wuv, Wo = head_slices(W, dims)
    r = (lambda x: x) if rnd is None else rnd
    return [(r(Wuk[i].T @ Wuq[i]), r(Wo[i] @ Wuv[i])) for i in range(dims.n_h)]


def precombined_weights(W, dims: OracleDims, rnd=None):
    """The per-head matrices stacked as the library stores them: Wq_pre [n_h * d_c, d_cq] with row
    block i = W~^Q_i, Wo_pre [d, n_h * d_c] with column block i = W~^O_i."""
    pre = precombined_heads(W, dims, rnd)
    return np.concatenate([q for q, _ in pre], axis=0), np.concatenate([o for _, o in pre], axis=1)


def decode_step_precombined(W, pre, h, prefix, dims: OracleDims, cdtype):
    """One decode step in the pre-combined form, head by head: q~_i = W~^Q_i c^Q scores the
    latents, and u = sum_i W~^O_i o_lat_i. pre: precombined_heads(...) (possibly rounded). The
    rotary query and the appended row are as in new_token."""
    prefix = np.asarray(prefix, dtype=np.float64).reshape(-1, dims.d_c + dims.d_r)
    T = prefix.shape[0] + 1
    _, qR, _, _, read = new_token(W, h, T - 1, dims, cdtype)
    cQ = W["W_dq"] @ h
    rows = np.vstack([prefix, read[None, :]])
    C, KR = rows[:, : dims.d_c], rows[:, dims.d_c:]
    scale = score_scale(dims)
    u = np.zeros(dims.d)
    q_lat = np.zeros((dims.n_h, dims.d_c))
    o_lat = np.zeros((dims.n_h, dims.d_c))
    lse = np.zeros(dims.n_h)
    for i, (Wq_i, Wo_i) in enumerate(pre):
        q_lat[i] = Wq_i @ cQ                                    # q~_i = W~^Q_i c^Q
        s = (C @ q_lat[i] + KR @ qR[i]) * scale
        a = softmax(s)
        m = s.max()
        lse[i] = m + np.log(np.exp(s - m).sum())
        o_lat[i] = a @ C
        u += Wo_i @ o_lat[i]                                    # W~^O_i o_lat_i
    return dict(u=u, o_lat=o_lat, lse=lse, q_lat=q_lat)


def decode_batch(W, h, prefixes, dims: OracleDims, cdtype, heads=None, want_u=True):
    """decode_step_explicit over a batch; prefixes[b] are sequence b's stored rows."""
    return [decode_step_explicit(W, h[b], prefixes[b], dims, cdtype, heads=heads, want_u=want_u)
            for b in range(len(prefixes))]


def prefill_chunk(W, H, prefix, dims: OracleDims, cdtype, want_u=True):
    """Chunked prefill of one sequence: C new tokens H [C, d] after the stored rows `prefix`
    [p0, d_c + d_r]. By the definition of causal attention ([Scratch] section 6: token t attends to
    positions 0..t), token t of the chunk sits at position p0 + t and attends to the prefix and to
    the chunk's tokens 0..t; each token's own row is stored (rounded to the cache type) before the
    tokens after it read it. Written out as the decode steps of the chunk's tokens in order.
    Returns the list of per-token results of decode_step_explicit."""
    rows = np.asarray(prefix, dtype=np.float64).reshape(-1, dims.d_c + dims.d_r)
    outs = []
    for t in range(len(H)):
        r = decode_step_explicit(W, np.asarray(H[t], dtype=np.float64), rows, dims, cdtype, want_u=want_u)
        outs.append(r)
        rows = np.vstack([rows, r["read_new"][None, :]])
    return outs
