"""Seeded synthetic MLA workloads and the paged latent-cache layout.

This module holds no attention arithmetic: it draws the random inputs of the
decode and prefill workloads, rounds them to the input dtype, and lays the
cached tokens out in a pool of 64-token pages.  Both the HIP path and the
CPU oracle consume what it produces.

Workloads (the shapes, sizes and value distributions of the DeepSeek-V3 MLA
layer: d_c = 512, rope dim 64, nope dim 128, v dim 128, from
"DeepSeek-V3 技术报告精读", §维度分解详解):

  tiny_f32        decode, fp32, B=1,  H=16,  L=64 (keys at positions 0..63)
  decode_h16      decode, bf16, B=16, H=16,  L ~ U[1024, 4096]
  decode_h128     decode, bf16, B=64, H=128, L ~ U[8192, 32768]
  prefill_h128    causal prefill, bf16, T=8192, H=128
  long_bf16       decode, bf16, B=8,  H=128, L = 131072, 32 splits
  long_fp8        as long_bf16 with an e4m3 latent cache

Distributions: c_KV, k_R, q_C, q_R ~ N(0,1); W_UK, W_UV ~ N(0, 1/512)
(variance 1/512).  Lengths U[a,b] are integers inclusive at both ends.
Every tensor has its own counter-based sub-stream keyed by
(seed, workload, tensor, sequence), so any one sequence can be regenerated
alone.  bf16 inputs are rounded to nearest-even from fp32 here, so the oracle
sees exactly the values the GPU receives.
"""

from __future__ import annotations

import dataclasses
import zlib
from typing import Optional

import numpy as np

PAGE = 64
D_C = 512
D_R = 64
D_H = 128
ROW = D_C + D_R


def _key(name: str) -> int:
    return zlib.crc32(name.encode()) & 0x7FFFFFFF


def stream(seed: int, workload: str, tensor: str, index: int = 0) -> np.random.Generator:
    """Independent PCG64 stream for one (seed, workload, tensor, index)."""
    ss = np.random.SeedSequence([int(seed), _key(workload), _key(tensor), int(index)])
    return np.random.Generator(np.random.PCG64(ss))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bfloat16 (ties to even); returns fp32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32)
    # keep NaNs NaN (none are generated; defensive)
    return np.where(np.isnan(x), x, out)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of bf16-representable fp32 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


@dataclasses.dataclass
class Workload:
    name: str
    kind: str  # "decode" or "prefill"
    dtype: str  # "f32", "bf16" or "fp8" (fp8: e4m3 latent, bf16 everything else)
    B: int
    H: int
    lens: np.ndarray  # int32 [B] cached tokens per sequence (prefill: [T])
    splits: int = 0  # 0 = let the library choose
    seed: int = 0

    @property
    def total_tokens(self) -> int:
        return int(self.lens.sum())

    @property
    def pages_per_seq(self) -> np.ndarray:
        return (self.lens + PAGE - 1) // PAGE

    @property
    def max_pages(self) -> int:
        return int(self.pages_per_seq.max())


def make_workload(name: str, seed: int = 0, B: Optional[int] = None, H: Optional[int] = None,
                  lens=None, dtype: Optional[str] = None, splits: Optional[int] = None) -> Workload:
    """One of the named workloads; any size argument overrides the default
    (used for scaled-down parity cases with the same structure)."""
    table = {
        "tiny_f32": ("decode", "f32", 1, 16, ("fixed", 64), 0),
        "decode_h16": ("decode", "bf16", 16, 16, ("uniform", 1024, 4096), 0),
        "decode_h128": ("decode", "bf16", 64, 128, ("uniform", 8192, 32768), 0),
        "prefill_h128": ("prefill", "bf16", 1, 128, ("fixed", 8192), 0),
        "long_bf16": ("decode", "bf16", 8, 128, ("fixed", 131072), 32),
        "long_fp8": ("decode", "fp8", 8, 128, ("fixed", 131072), 32),
    }
    kind, dt, b, h, ld, sp = table[name]
    b = b if B is None else B
    h = h if H is None else H
    dt = dt if dtype is None else dtype
    sp = sp if splits is None else splits
    if lens is not None:
        arr = np.asarray(lens, dtype=np.int32).reshape(-1)
        if arr.size == 1 and b > 1:
            arr = np.full(b, int(arr[0]), dtype=np.int32)
    elif ld[0] == "fixed":
        arr = np.full(b, ld[1], dtype=np.int32)
    else:
        arr = stream(seed, name, "lens").integers(ld[1], ld[2], size=b, endpoint=True).astype(np.int32)
    if kind == "prefill":
        b = 1
    return Workload(name=name, kind=kind, dtype=dt, B=b, H=h, lens=arr, splits=sp, seed=seed)


def _normal(gen: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = gen.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _cast(x: np.ndarray, dtype: str) -> np.ndarray:
    return x if dtype == "f32" else round_bf16(x)


def weights(wl: Workload):
    """W_UK, W_UV [H,128,512] ~ N(0, 1/512), rounded to the input dtype."""
    std = float(np.sqrt(1.0 / 512.0))
    w_uk = _cast(_normal(stream(wl.seed, wl.name, "W_UK"), (wl.H, D_H, D_C), std), wl.dtype)
    w_uv = _cast(_normal(stream(wl.seed, wl.name, "W_UV"), (wl.H, D_H, D_C), std), wl.dtype)
    return w_uk, w_uv


def queries(wl: Workload):
    """q_C [N,H,128] and raw (un-rotated) q_R [N,H,64] ~ N(0,1).

    N = B for decode (one new token per sequence), N = T for prefill."""
    n = wl.B if wl.kind == "decode" else int(wl.lens[0])
    q_c = _cast(_normal(stream(wl.seed, wl.name, "q_C"), (n, wl.H, D_H)), wl.dtype)
    q_r = _cast(_normal(stream(wl.seed, wl.name, "q_R"), (n, wl.H, D_R)), wl.dtype)
    return q_c, q_r


def multi_queries(wl: Workload, q_len: int):
    """q_C [B,q_len,H,128] and raw q_R [B,q_len,H,64] ~ N(0,1) for multi-token
    decode: the q_len newest tokens of every sequence are queries, token t of
    sequence b at position L_b - q_len + t."""
    q_c = _cast(_normal(stream(wl.seed, wl.name, "q_C_multi", q_len), (wl.B, q_len, wl.H, D_H)), wl.dtype)
    q_r = _cast(_normal(stream(wl.seed, wl.name, "q_R_multi", q_len), (wl.B, q_len, wl.H, D_R)), wl.dtype)
    return q_c, q_r


def sequence_latents(wl: Workload, b: int):
    """c_KV [L_b,512] and raw (un-rotated) k_R [L_b,64] of sequence b, ~ N(0,1).

    fp8 workloads draw bf16 values; the quantisation happens in the cache
    write (and, independently, in the oracle)."""
    L = int(wl.lens[b])
    c = _cast(_normal(stream(wl.seed, wl.name, "c_KV", b), (L, D_C)), wl.dtype)
    k = _cast(_normal(stream(wl.seed, wl.name, "k_R", b), (L, D_R)), wl.dtype)
    return c, k


@dataclasses.dataclass
class PagedLayout:
    """Where every cached token lives in the page pool.

    block_table[b, i] is the pool page holding tokens 64i..64i+63 of sequence
    b (-1 past the sequence's last page); slots[off_b + j] = page*64 + j%64 is
    the pool row of token j; offsets are the prefix sums of lens."""
    num_pages: int
    block_table: np.ndarray  # int32 [B, max_pages]
    slots: np.ndarray  # int32 [sum L]
    offsets: np.ndarray  # int64 [B+1]
    positions: np.ndarray  # int32 [sum L] position of each token within its sequence


def paged_layout(wl: Workload, spare_pages: int = 0, shuffle: bool = True) -> PagedLayout:
    """Seeded random permutation of pool pages over the sequences' pages."""
    pps = wl.pages_per_seq.astype(np.int64)
    need = int(pps.sum())
    num_pages = need + int(spare_pages)
    if shuffle:
        perm = stream(wl.seed, wl.name, "pages").permutation(num_pages)[:need].astype(np.int32)
    else:
        perm = np.arange(need, dtype=np.int32)
    maxp = int(pps.max())
    bt = np.full((wl.B, maxp), -1, dtype=np.int32)
    offsets = np.zeros(wl.B + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(wl.lens.astype(np.int64))
    slots = np.empty(int(offsets[-1]), dtype=np.int32)
    positions = np.empty(int(offsets[-1]), dtype=np.int32)
    p0 = 0
    for b in range(wl.B):
        n = int(pps[b])
        bt[b, :n] = perm[p0:p0 + n]
        p0 += n
        L = int(wl.lens[b])
        j = np.arange(L, dtype=np.int64)
        slots[offsets[b]:offsets[b + 1]] = (bt[b, j // PAGE].astype(np.int64) * PAGE + j % PAGE).astype(np.int32)
        positions[offsets[b]:offsets[b + 1]] = j.astype(np.int32)
    return PagedLayout(num_pages=num_pages, block_table=bt, slots=slots, offsets=offsets, positions=positions)


def all_latents(wl: Workload):
    """Concatenated c_KV [sum L,512] and raw k_R [sum L,64] over the batch."""
    cs, ks = [], []
    for b in range(wl.B):
        c, k = sequence_latents(wl, b)
        cs.append(c)
        ks.append(k)
    return np.concatenate(cs, axis=0), np.concatenate(ks, axis=0)


# ---------------------------------------------------------------------------
# Inputs of the projections around the attention
# ---------------------------------------------------------------------------
# The pages fix d_c' = 1536 (q_lora_rank, §维度分解详解) but not the model
# width d; D_MODEL is a synthetic choice (a multiple of 128, as the 128-wide
# block quantisation tiles of the FP8 scheme assume).
D_MODEL = 7168
D_CQ = 1536


def projection_weights(wl: Workload, d: int = D_MODEL, dcq: int = D_CQ):
    """bf16 weights of the projections, each ~ N(0, 1/fan_in) so that every
    projected vector has unit variance for unit-variance inputs:
    W^DKV [512, d], W^KR [64, d], W^DQ [dcq, d], W^UQ [H*128, dcq],
    W^QR [H*64, dcq], W^O [d, H*128]."""
    def w(tag, shape, fan_in):
        return round_bf16(_normal(stream(wl.seed, wl.name, tag, d), shape, float(np.sqrt(1.0 / fan_in))))
    return {
        "w_dkv": w("W_DKV", (D_C, d), d),
        "w_kr": w("W_KR", (D_R, d), d),
        "w_dq": w("W_DQ", (dcq, d), d),
        "w_uq": w("W_UQ", (wl.H * D_H, dcq), dcq),
        "w_qr": w("W_QR", (wl.H * D_R, dcq), dcq),
        "w_o": w("W_O", (d, wl.H * D_H), wl.H * D_H),
    }


def hidden_states(wl: Workload, b: int, d: int = D_MODEL, rows: Optional[int] = None) -> np.ndarray:
    """h [rows, d] ~ N(0, 1) in bf16: the hidden states of sequence b's
    tokens (rows defaults to its length)."""
    n = int(wl.lens[b]) if rows is None else int(rows)
    return round_bf16(_normal(stream(wl.seed, wl.name, "h", b * 1_000_003 + d), (n, d)))


def new_token_hidden(wl: Workload, d: int = D_MODEL) -> np.ndarray:
    """h [B, d] ~ N(0, 1) bf16: the hidden state of each sequence's new token."""
    return round_bf16(_normal(stream(wl.seed, wl.name, "h_new", d), (wl.B, d)))


def fp8_edge_rows(seed: int = 0) -> np.ndarray:
    """Latent rows [8, 512] (bf16 values, as fp32) that reach every branch of
    an E4M3 tile quantiser: all-zero tiles (with negative zeros mixed in),
    a single non-zero element, tiles whose amax is 448 (scale exactly 1) with
    values on the rounding ties of the subnormal grid (odd multiples of
    2^-10), of the normal grid and near the top of the range, tiny and huge
    amax, and magnitudes spread log-uniformly from amax down to 2^-24 amax
    (normal codes, subnormal codes and values that round to zero)."""
    g = stream(seed, "fp8_edges", "rows")
    r = np.zeros((8, D_C), dtype=np.float32)
    # row 0: four all-zero tiles; tiles 1 and 3 mix negative zeros in
    r[0, 128:256:2] = -0.0
    r[0, 384:512:3] = -0.0
    # row 1: tile 0 zero; tile 1 one non-zero element; tile 2 negative amax;
    # tile 3 log-uniform magnitudes below amax = 1
    r[1, 128 + 37] = -3.5
    r[1, 256:384] = g.standard_normal(128) * 0.25
    r[1, 256 + 5] = -7.0
    r[1, 384] = 1.0
    r[1, 385:512] = g.choice([-1.0, 1.0], 127) * np.exp2(g.uniform(-24.0, 0.0, 127))
    # row 2: amax 448 (scale 1): subnormal ties (2m+1) 2^-10, normal ties,
    # values near 448, signed zeros
    t = np.zeros(128, dtype=np.float32)
    t[0] = 448.0
    t[1:17] = np.concatenate([(2 * np.arange(8) + 1) * 2.0 ** -10, -(2 * np.arange(8) + 1) * 2.0 ** -10])
    t[17:25] = [1.0625, 1.1875, -1.3125, 2.125, 0.02734375, 0.0146484375, 30.0, -31.0]
    t[25:33] = [440.0, 432.0, -424.0, 400.0, 416.0, 447.0, 3.0 * 2.0 ** -10, 2.0 ** -10]
    t[33] = -0.0
    t[34:128] = g.standard_normal(94)
    r[2, :128] = t
    r[2, 128:256] = -t
    r[2, 256:384] = t * 2.0 ** -60     # tiny amax (scale 2^-60)
    r[2, 384:512] = t * 2.0 ** 100     # huge amax (scale 2^100)
    # rows 3..7: log-uniform magnitudes over 2^-24 .. 1 of a random amax
    for i in range(3, 8):
        amax = np.exp2(g.uniform(-20.0, 20.0, 4))
        mag = np.exp2(g.uniform(-24.0, 0.0, (4, 128)))
        mag[:, 0] = 1.0
        sgn = g.choice([-1.0, 1.0], (4, 128))
        r[i] = (sgn * mag * amax[:, None]).reshape(D_C)
    return round_bf16(r)
