"""Reference oracle for absorbed Multi-head Latent Attention (MLA) decode and prefill.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the test suite, the package smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP library
and imports nothing from the product package.

It is a plain, slow, fp64 NumPy implementation of the *un-absorbed* MLA
equations as written in the "DeepSeek-V3" equation notes (ekkoxiao.github.io,
sections KeyValue, Query, 注意力计算, 潜在向量的作用, RoPE 数据流, YaRN 扩展).
For every head i it expands the cached latent rows into per-head keys and
values, k^C = W_i^UK c^KV and v^C = W_i^UV c^KV, and runs ordinary softmax
attention over them.  The absorbed quantities the GPU path produces are also
emitted, each from its own defining equation:

    q~_i = (W_i^UK)^T q_i^C                       (§潜在向量的作用, definition of q~)
    z_i  = sum_j a_{i,j} c_j^KV                   (§潜在向量的作用, value in latent space)
    lse_i = log sum_j exp(s_{i,j})

Notation and shapes (dimensions from "DeepSeek-V3 技术报告精读", oopvo.github.io,
§维度分解详解): d_c = 512 (kv_lora_rank), d_h = 128 (qk_nope_head_dim),
d_h^R = 64 (qk_rope_head_dim), d_v = 128 (v_head_dim).

    q_c   [H, 128]   content query of one decode token, per head
    q_r   [H, 64]    position query *before* rotation, per head
    c_kv  [L, 512]   cached latent rows of one sequence
    k_r   [L, 64]    shared position key *before* rotation, per token
    w_uk  [H, 128, 512]   head i's row block of the key up-projection
    w_uv  [H, 128, 512]   head i's row block of the value up-projection

Around the attention it also gives the projections the pages define: the
cache append c^KV = W^DKV h, k^R = RoPE(W^KR h) (§KeyValue), the query path
c^Q = W^DQ h, q_i^C = W_i^UQ c^Q, q_i^R = RoPE(W_i^QR c^Q) (§Query), the
output u = W^O [o_1; ...; o_H] (§注意力计算) and W^O with W^UV folded into it.

Readings of points the pages leave open (each is restated where it is used):
  * RoPE rotates interleaved pairs (2m, 2m+1) counter-clockwise by pos*theta_m,
    theta_m = base^(-2m/64).  The pages give the per-pair angle (§YaRN 扩展)
    and the frequency formula (page "企业官网建设流程全解析", discosf.com, §4.3) but
    not the pair layout.
  * A decode query sits at position L-1: it is the newest token, already in
    the cache, and the softmax sum runs over j = 1..t inclusive (§注意力计算).
  * Key j of a sequence is at position j (0-based).
  * The softmax scale is 1/sqrt(d_h + d_h^R) = 1/sqrt(192) (§注意力计算).
  * The fp8 latent cache uses OCP E4M3 (max 448; "DeepSeek-V3 技术报告精读",
    §FP8 混合精度训练) with one fp32 scale per token per 128 channels (the 1x128
    tile rule of "DeepSeek-V3 Technical Report", process-cxr.github.io,
    §Fine-grained quantization), scale = amax/448 computed in fp32, 1.0 for an
    all-zero tile; codes are round-to-nearest-even with saturation.
  * No normalisation sits between a down-projection and its up-projection:
    the equations of §KeyValue and §Query show none.  The model width d is
    not given by the pages; every function here takes it from its inputs.

Parity status: every function here is pinned by the CPU tests in
tests/test_oracle.py against things other than itself: closed forms and
identities, a textbook attention routine, brute force on tiny inputs, the
library fp8 cast, and hand-worked values inside the YaRN ramp.  The one
value that nothing outside the oracle can fix is the ramp's shape itself
(the pages only sketch it): the hand-worked values pin the reading taken,
not the pages' intent.
"""

from __future__ import annotations

import math

import numpy as np

D_C = 512  # kv_lora_rank
D_R = 64  # qk_rope_head_dim
D_H = 128  # qk_nope_head_dim
D_V = 128  # v_head_dim
ROW = D_C + D_R  # cached elements per token per layer (§KeyValue: d_c + d_h^R)
E4M3_MAX = 448.0
FP8_TILE = 128


def default_softmax_scale() -> float:
    """1/sqrt(d_h + d_h^R) from the score equation (§注意力计算)."""
    return 1.0 / math.sqrt(D_H + D_R)


# ----------------------------------------------------------------------------
# RoPE
# ----------------------------------------------------------------------------

def rope_frequencies(dim: int = D_R, base: float = 10000.0) -> np.ndarray:
    """theta_m = base^(-2m/dim), m = 0 .. dim/2-1.

    Frequency formula: "企业官网建设流程全解析" (discosf.com), §4.3, with base
    10000.  Used as one frequency per 2-D group as in §YaRN 扩展 of the
    "DeepSeek-V3" notes (phi_{m,j} = m * theta_j).
    """
    m = np.arange(dim // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * m / dim)


YARN_FACTOR = 40.0    # s       ("DeepSeek-V3 Technical Report", §Long Context Extension)
YARN_ALPHA = 1.0      # alpha
YARN_BETA = 32.0      # beta
YARN_ORIG_LEN = 4096  # context length before the extension (4K -> 32K -> 128K)


def yarn_frequencies(dim: int = D_R, base: float = 10000.0, factor: float = YARN_FACTOR,
                     alpha: float = YARN_ALPHA, beta: float = YARN_BETA, orig_len: int = YARN_ORIG_LEN) -> np.ndarray:
    """YaRN frequencies of the decoupled RoPE path ("DeepSeek-V3" notes, §YaRN 扩展):

        theta'_j = (1 - gamma_j) * theta_j / s + gamma_j * theta_j,

    gamma_j = 1 for the high-frequency groups (frequency kept), 0 for the
    low-frequency ones (divided by s), in between a smooth transition.  The
    pages fix s, alpha, beta ("DeepSeek-V3 Technical Report", §Long Context
    Extension) but only sketch the ramp.  Reading taken: gamma_j is linear in
    the number of full turns r_j = orig_len * theta_j / (2 pi) that group j
    makes over the pre-extension context (4K), 0 for r_j <= alpha and 1 for
    r_j >= beta.
    """
    theta = rope_frequencies(dim, base)
    r = orig_len * theta / (2.0 * math.pi)
    gamma = np.clip((r - alpha) / (beta - alpha), 0.0, 1.0)
    return (1.0 - gamma) * theta / factor + gamma * theta


def yarn_attention_factor(factor: float = YARN_FACTOR) -> float:
    """0.1 ln s + 1 ("DeepSeek-V3 Technical Report", §Long Context Extension).
    Reading taken: it multiplies the attention scores once, i.e. the softmax
    scale becomes (0.1 ln s + 1) / sqrt(192)."""
    return 0.1 * math.log(factor) + 1.0


def rope(x: np.ndarray, positions, base: float = 10000.0, theta=None) -> np.ndarray:
    """Rotate the last axis of x (length 64) at the given positions.

    Group m is the interleaved pair (x[2m], x[2m+1]); it is rotated
    counter-clockwise by the angle pos * theta_m (§YaRN 扩展: phi = m*theta_j):
        x'[2m]   = x[2m] cos(phi) - x[2m+1] sin(phi)
        x'[2m+1] = x[2m] sin(phi) + x[2m+1] cos(phi)
    `positions` broadcasts against x[..., 0].  theta: the per-group
    frequencies (default base^(-2m/64); yarn_frequencies() for YaRN).
    """
    x = np.asarray(x, dtype=np.float64)
    dim = x.shape[-1]
    theta = rope_frequencies(dim, base) if theta is None else np.asarray(theta, dtype=np.float64)
    pos = np.asarray(positions, dtype=np.float64)[..., None]
    phi = pos * theta  # [..., dim/2]
    c, s = np.cos(phi), np.sin(phi)
    xe, xo = x[..., 0::2], x[..., 1::2]
    out = np.empty(np.broadcast_shapes(x.shape, phi.shape[:-1] + (dim,)), dtype=np.float64)
    out[..., 0::2] = xe * c - xo * s
    out[..., 1::2] = xe * s + xo * c
    return out


# ----------------------------------------------------------------------------
# Expanded (un-absorbed) attention
# ----------------------------------------------------------------------------

def _attend_expanded(q_c, q_r_rot, c_kv, k_r_rot, w_uk, w_uv, scale):
    """Standard attention of H query heads over L expanded keys/values.

    k^C_{j,i} = W_i^UK c_j, v^C_{j,i} = W_i^UV c_j (§KeyValue);
    s_{j,i} = (q_i^C . k^C_{j,i} + q_i^R . k^R_j) * scale (§注意力计算);
    a = softmax over j with the row maximum subtracted; o_i = sum_j a v^C.
    Returns o [H,128], z [H,512], lse [H], probs [H,L].
    """
    H = q_c.shape[0]
    L = c_kv.shape[0]
    o = np.empty((H, D_V))
    z = np.empty((H, D_C))
    lse = np.empty(H)
    probs = np.empty((H, L))
    for i in range(H):
        k_c = c_kv @ w_uk[i].T  # [L,128]   expanded content keys
        v_c = c_kv @ w_uv[i].T  # [L,128]   expanded values
        s = (k_c @ q_c[i] + k_r_rot @ q_r_rot[i]) * scale  # [L]
        m = s.max()
        e = np.exp(s - m)
        den = e.sum()
        a = e / den
        probs[i] = a
        o[i] = a @ v_c
        z[i] = a @ c_kv  # latent-space aggregate (§潜在向量的作用)
        lse[i] = m + math.log(den)
    return o, z, lse, probs


def absorb_query(q_c, w_uk):
    """q~_i = (W_i^UK)^T q_i^C, the absorbed query (§潜在向量的作用)."""
    q_c = np.asarray(q_c, dtype=np.float64)
    w_uk = np.asarray(w_uk, dtype=np.float64)
    return np.einsum("hdc,...hd->...hc", w_uk, q_c)


def decode_sequence(q_c, q_r, c_kv, k_r, w_uk, w_uv, *, softmax_scale=None, rope_base=10000.0,
                    return_probs=False, rope_theta=None):
    """One decode token of one sequence attending to its L cached tokens.

    Keys sit at positions 0..L-1 and the query at L-1.  Inputs are cast to
    fp64.  Returns a dict with o [H,128],
    z [H,512], lse [H], q_tilde [H,512], q_abs [H,576] (q~ followed by the
    rotated q_r) and optionally probs [H,L].
    """
    q_c = np.asarray(q_c, dtype=np.float64)
    q_r = np.asarray(q_r, dtype=np.float64)
    c_kv = np.asarray(c_kv, dtype=np.float64)
    k_r = np.asarray(k_r, dtype=np.float64)
    w_uk = np.asarray(w_uk, dtype=np.float64)
    w_uv = np.asarray(w_uv, dtype=np.float64)
    L = c_kv.shape[0]
    if L < 1:
        raise ValueError("softmax over an empty set of cached tokens has no value")
    scale = default_softmax_scale() if softmax_scale is None else float(softmax_scale)
    p = L - 1
    k_r_rot = rope(k_r, np.arange(L), rope_base, rope_theta)
    q_r_rot = rope(q_r, p, rope_base, rope_theta)
    o, z, lse, probs = _attend_expanded(q_c, q_r_rot, c_kv, k_r_rot, w_uk, w_uv, scale)
    q_t = absorb_query(q_c, w_uk)
    out = {"o": o, "z": z, "lse": lse, "q_tilde": q_t,
           "q_abs": np.concatenate([q_t, q_r_rot], axis=-1)}
    if return_probs:
        out["probs"] = probs
    return out


def prefill_causal(q_c, q_r, c_kv, k_r, w_uk, w_uv, rows=None, *, softmax_scale=None,
                   rope_base=10000.0, rope_theta=None):
    """Causal prefill of one sequence of T tokens at positions 0..T-1.

    Query row t attends to keys j <= t (the softmax sum of §注意力计算 runs
    up to and including the current position).  `rows` selects which query
    rows to compute (default: all).  Returns o [R,H,128], z [R,H,512],
    lse [R,H], q_abs [R,H,576] and the rotated keys k_r_rot [T,64] (what the
    latent cache must hold for the position part).
    """
    q_c = np.asarray(q_c, dtype=np.float64)
    q_r = np.asarray(q_r, dtype=np.float64)
    c_kv = np.asarray(c_kv, dtype=np.float64)
    k_r = np.asarray(k_r, dtype=np.float64)
    w_uk = np.asarray(w_uk, dtype=np.float64)
    w_uv = np.asarray(w_uv, dtype=np.float64)
    T = c_kv.shape[0]
    rows = np.arange(T) if rows is None else np.asarray(rows)
    scale = default_softmax_scale() if softmax_scale is None else float(softmax_scale)
    k_r_rot = rope(k_r, np.arange(T), rope_base, rope_theta)
    res = {"o": [], "z": [], "lse": [], "q_abs": []}
    for t in rows:
        t = int(t)
        q_r_rot = rope(q_r[t], t, rope_base, rope_theta)
        o, z, lse, _ = _attend_expanded(q_c[t], q_r_rot, c_kv[: t + 1], k_r_rot[: t + 1], w_uk, w_uv, scale)
        res["o"].append(o)
        res["z"].append(z)
        res["lse"].append(lse)
        res["q_abs"].append(np.concatenate([absorb_query(q_c[t], w_uk), q_r_rot], axis=-1))
    out = {k: np.stack(v) for k, v in res.items()}
    out["k_r_rot"] = k_r_rot
    return out


# ----------------------------------------------------------------------------
# Absorbed form (independent second formula, used to pin the expanded one)
# ----------------------------------------------------------------------------

def decode_sequence_absorbed(q_c, q_r, c_kv, k_r, w_uk, w_uv, *, softmax_scale=None,
                             rope_base=10000.0, rope_theta=None):
    """The same decode through the absorbed equations of §潜在向量的作用:

    s_{j,i} = (q~_i . c_j + q_i^R . k^R_j) * scale,  z_i = sum_j a c_j,
    o_i = W_i^UV z_i.  Associativity makes this equal to the expanded form up
    to rounding; the CPU tests hold the two to 1e-12.
    """
    c_kv = np.asarray(c_kv, dtype=np.float64)
    L = c_kv.shape[0]
    scale = default_softmax_scale() if softmax_scale is None else float(softmax_scale)
    q_t = absorb_query(q_c, w_uk)  # [H,512]
    k_r_rot = rope(k_r, np.arange(L), rope_base, rope_theta)
    q_r_rot = rope(q_r, L - 1, rope_base, rope_theta)
    s = (q_t @ c_kv.T + q_r_rot @ k_r_rot.T) * scale  # [H,L]
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    a = e / e.sum(axis=1, keepdims=True)
    z = a @ c_kv
    o = np.einsum("hdc,hc->hd", np.asarray(w_uv, dtype=np.float64), z)
    lse = (m[:, 0] + np.log(e.sum(axis=1)))
    return {"o": o, "z": z, "lse": lse}


# ----------------------------------------------------------------------------
# fp8 (E4M3) latent cache quantiser
# ----------------------------------------------------------------------------

def _e4m3_code_from_float(v: float) -> int:
    """Encode one finite fp32 value |v| <= 448 as OCP E4M3 (bias 7, 3 mantissa
    bits, no infinities), rounding to nearest with ties to even.

    Written from the format definition: normal numbers are
    (1 + m/8) * 2^(e-7) for e in 1..15 (e=15, m=7 is NaN, so 448 = 1.75*2^8
    is the largest), subnormals are (m/8) * 2^-6.
    """
    sign = 0x80 if (v < 0 or (v == 0 and math.copysign(1.0, v) < 0)) else 0
    a = abs(v)
    if a == 0.0:
        return sign
    # quantum of the binade holding a (subnormal quantum 2^-9 below 2^-6)
    if a < 2.0 ** -6:
        quantum = 2.0 ** -9
    else:
        quantum = 2.0 ** (math.floor(math.log2(a)) - 3)
        # guard against log2 rounding at exact powers of two
        while quantum * 8 > a:
            quantum /= 2
        while quantum * 16 <= a:
            quantum *= 2
    n = a / quantum  # exact in fp64 (a has 24 significant bits)
    r = math.floor(n)
    frac = n - r
    if frac > 0.5 or (frac == 0.5 and (r % 2 == 1)):
        r += 1
    val = r * quantum
    if val > E4M3_MAX:
        val = E4M3_MAX
    if val < 2.0 ** -6:
        m = int(round(val / 2.0 ** -9))
        return sign | m  # exponent field 0
    e = math.floor(math.log2(val))
    while 2.0 ** e > val:
        e -= 1
    while 2.0 ** (e + 1) <= val:
        e += 1
    m = int(round((val / 2.0 ** e - 1.0) * 8))
    if m == 8:
        e += 1
        m = 0
    return sign | ((e + 7) << 3) | m


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Value of each E4M3 code (uint8) as fp64; NaN codes decode to NaN."""
    codes = np.asarray(codes, dtype=np.uint8)
    s = np.where(codes & 0x80, -1.0, 1.0)
    e = (codes >> 3) & 0xF
    m = (codes & 0x7).astype(np.float64)
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.power(2.0, e.astype(np.float64) - 7))
    val = np.where((e == 15) & ((codes & 7) == 7), np.nan, val)
    return s * val


def quantize_latent_e4m3(c_kv: np.ndarray):
    """Per token and per 128-channel tile: scale = amax/448 (1.0 if the tile is
    all zero), code = E4M3(RNE(clamp(c/scale, -448, 448))).

    All arithmetic that decides a code (amax, the scale and c/scale) is done
    in fp32, one correctly rounded operation at a time.
    Returns codes uint8 [L,512] and scales float32 [L,4].
    """
    c = np.asarray(c_kv, dtype=np.float32)
    L = c.shape[0]
    tiles = c.reshape(L, D_C // FP8_TILE, FP8_TILE)
    amax = np.abs(tiles).max(axis=2)  # exact
    scale = np.where(amax > 0, (amax / np.float32(E4M3_MAX)).astype(np.float32), np.float32(1.0)).astype(np.float32)
    x = (tiles / scale[:, :, None]).astype(np.float32)  # fp32 division
    x = np.clip(x, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    # one encoder call per distinct bit pattern (not per distinct value: +0
    # and -0 compare equal but have codes 0x00 and 0x80)
    flat = np.ascontiguousarray(x.reshape(-1)).view(np.uint32)
    uniq, inv = np.unique(flat, return_inverse=True)
    enc = np.array([_e4m3_code_from_float(float(u)) for u in uniq.view(np.float32)], dtype=np.uint8)
    codes = enc[inv].reshape(L, D_C)
    return codes, scale.astype(np.float32)


def dequantize_latent_e4m3(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """c~ = value(code) * scale of its (token, 128-channel) tile, in fp64."""
    vals = e4m3_decode(codes).reshape(codes.shape[0], D_C // FP8_TILE, FP8_TILE)
    return (vals * np.asarray(scales, dtype=np.float64)[:, :, None]).reshape(codes.shape[0], D_C)


# ----------------------------------------------------------------------------
# Projections before and after the attention
# ----------------------------------------------------------------------------
# Shapes are generic (the tests also run them at toy widths).  Head i's
# blocks of the stacked matrices are contiguous row (or column) ranges:
#   w_uq [H*d_h,  d_c'], rows i*d_h   .. (i+1)*d_h   - 1 are W_i^UQ
#   w_qr [H*d_hR, d_c'], rows i*d_hR  .. (i+1)*d_hR  - 1 are W_i^QR
#   w_o  [d, H*d_v],     columns i*d_v .. (i+1)*d_v - 1 meet o_i
# Readings: the equations of §KeyValue and §Query carry no normalisation
# between the down- and up-projections, so none is applied here.

def kv_projection(h, w_dkv, w_kr, positions, *, rope_base=10000.0, rope_theta=None):
    """What one token appends to the cache (§KeyValue):

        c_t^KV = W^DKV h_t,    k_t^R = RoPE_t(W^KR h_t).

    h [T, d] (row t is h_t), w_dkv [d_c, d], w_kr [d_hR, d], positions [T].
    Returns c_kv [T, d_c], k_r [T, d_hR] before rotation and k_r_rot after.
    """
    h = np.asarray(h, dtype=np.float64)
    c_kv = h @ np.asarray(w_dkv, dtype=np.float64).T
    k_r = h @ np.asarray(w_kr, dtype=np.float64).T
    k_r_rot = rope(k_r, np.asarray(positions), rope_base, rope_theta)
    return {"c_kv": c_kv, "k_r": k_r, "k_r_rot": k_r_rot}


def query_projection(h, w_dq, w_uq, w_qr, positions, heads, *, rope_base=10000.0, rope_theta=None):
    """The per-head queries of a token (§Query):

        c_t^Q = W^DQ h_t,  q_{t,i}^C = W_i^UQ c_t^Q,  q_{t,i}^R = RoPE_t(W_i^QR c_t^Q).

    h [T, d], w_dq [d_c', d], w_uq [H*d_h, d_c'], w_qr [H*d_hR, d_c'].
    Returns c_q [T, d_c'], q_c [T, H, d_h], q_r [T, H, d_hR] before rotation
    and q_r_rot after.
    """
    h = np.asarray(h, dtype=np.float64)
    w_uq = np.asarray(w_uq, dtype=np.float64)
    w_qr = np.asarray(w_qr, dtype=np.float64)
    T, H = h.shape[0], int(heads)
    dh, dhr = w_uq.shape[0] // H, w_qr.shape[0] // H
    c_q = h @ np.asarray(w_dq, dtype=np.float64).T
    q_c = np.empty((T, H, dh))
    q_r = np.empty((T, H, dhr))
    for i in range(H):
        q_c[:, i] = c_q @ w_uq[i * dh:(i + 1) * dh].T
        q_r[:, i] = c_q @ w_qr[i * dhr:(i + 1) * dhr].T
    pos = np.asarray(positions)[:, None]  # the same angle for every head of a token
    q_r_rot = rope(q_r, pos, rope_base, rope_theta)
    return {"c_q": c_q, "q_c": q_c, "q_r": q_r, "q_r_rot": q_r_rot}


def output_projection(o, w_o):
    """u_t = W^O [o_{t,1}; ...; o_{t,H}] (§注意力计算): the head outputs are
    concatenated in head order and projected back to the model width.

    o [T, H, d_v], w_o [d, H*d_v] -> u [T, d].
    """
    o = np.asarray(o, dtype=np.float64)
    T, H, dv = o.shape
    cat = o.reshape(T, H * dv)
    return cat @ np.asarray(w_o, dtype=np.float64).T


def fold_wuv_into_wo(w_uv, w_o):
    """The output matrix with the value up-projection absorbed into it
    ("DeepSeek-V3 技术报告精读", §一 MLA, KV 权重吸收; o_i = W_i^UV z_i from
    §潜在向量的作用):

        W' = W^O blockdiag(W_1^UV, ..., W_H^UV),   u = W' [z_1; ...; z_H].

    w_uv [H, d_v, d_c], w_o [d, H*d_v] -> W' [d, H*d_c]; column block i is
    (columns i*d_v.. of W^O) @ W_i^UV.
    """
    w_uv = np.asarray(w_uv, dtype=np.float64)
    w_o = np.asarray(w_o, dtype=np.float64)
    H, dv, dc = w_uv.shape
    out = np.zeros((w_o.shape[0], H * dc))
    for i in range(H):
        out[:, i * dc:(i + 1) * dc] = w_o[:, i * dv:(i + 1) * dv] @ w_uv[i]
    return out


def layer_decode_from_hidden(h_seq, w_dkv, w_kr, w_dq, w_uq, w_qr, w_uk, w_uv, w_o, *,
                             softmax_scale=None, rope_base=10000.0, rope_theta=None):
    """The attention layer's output for the newest token of one sequence,
    from the hidden states h_0 .. h_{L-1} of all its tokens (positions
    0..L-1): every token's (c^KV, k^R) from kv_projection, the newest token's
    queries from query_projection, the expanded attention of decode_sequence,
    and output_projection.  Returns a dict with u [d], o [H, d_v], z [H, d_c],
    and the pieces c_kv, k_r (before rotation), q_c, q_r (before rotation).
    """
    h_seq = np.asarray(h_seq, dtype=np.float64)
    L = h_seq.shape[0]
    H = np.asarray(w_uk).shape[0]
    kv = kv_projection(h_seq, w_dkv, w_kr, np.arange(L), rope_base=rope_base, rope_theta=rope_theta)
    q = query_projection(h_seq[L - 1:], w_dq, w_uq, w_qr, [L - 1], H, rope_base=rope_base,
                         rope_theta=rope_theta)
    att = decode_sequence(q["q_c"][0], q["q_r"][0], kv["c_kv"], kv["k_r"], w_uk, w_uv,
                          softmax_scale=softmax_scale, rope_base=rope_base, rope_theta=rope_theta)
    u = output_projection(att["o"][None], w_o)[0]
    return {"u": u, "o": att["o"], "z": att["z"], "c_kv": kv["c_kv"], "k_r": kv["k_r"],
            "q_c": q["q_c"][0], "q_r": q["q_r"][0]}
