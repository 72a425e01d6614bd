"""The GPU E4M3 encoders on the quantiser's edge cases, bit-exact against the
oracle: all-zero tiles (scale 1, signed zeros), a lone non-zero element,
amax 448 with values on the rounding ties of the subnormal and normal grids,
tiny and huge amax, and magnitudes down to 2^-24 of the tile's amax
(subnormal codes and values that round to zero).

Both encoders are covered: the cache write from given latents
(mla_cache_write) and the one that quantises summed projection partials
(mla_kv_append).  The tile rule is the 1x128 per-token scaling of the
"DeepSeek-V3 Technical Report" (§Fine-grained quantization) with the E4M3
maximum 448 ("DeepSeek-V3 技术报告精读", §FP8 混合精度训练).
"""

import sys

import numpy as np
import pytest
import torch

import mla_latent_kv_30_amd as mla
from mla_latent_kv_30_amd import workload as W
from oracle import mla_oracle as orc

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _slots(T, num_pages):
    # scattered slots over a pool of num_pages pages
    rng = np.random.default_rng(3)
    return np.sort(rng.choice(num_pages * 64, T, replace=False)).astype(np.int32)


def _read_fp8(cache, slots):
    codes = cache.ckv.cpu().numpy().reshape(-1, 512)[slots]
    scales = cache.scale.cpu().numpy().reshape(-1, 4)[slots]
    return codes, scales


def test_cache_write_fp8_edge_tiles_bit_exact():
    _note("case fp8 edge rows through mla_cache_write")
    c = W.fp8_edge_rows()
    T = c.shape[0]
    k = W.round_bf16(np.random.default_rng(4).standard_normal((T, 64)).astype(np.float32))
    cache = mla.PagedCache(2, "fp8", device=DEV, fill=float("nan"))
    slots = _slots(T, 2)
    pos = np.arange(T, dtype=np.int32) + 5
    mla.cache_write(cache, torch.from_numpy(c).to(DEV, torch.bfloat16), torch.from_numpy(k).to(DEV, torch.bfloat16),
                    torch.from_numpy(pos).to(DEV), torch.from_numpy(slots).to(DEV))
    torch.cuda.synchronize()
    codes, scales = _read_fp8(cache, slots)
    rc, rs = orc.quantize_latent_e4m3(c)
    np.testing.assert_array_equal(scales, rs)
    np.testing.assert_array_equal(codes, rc)
    assert (codes[0, 128:256:2] == 0x80).all()  # negative zeros keep their sign


def test_kv_append_fp8_edge_tiles_bit_exact():
    """h_t = e_t (one-hot, exact in bf16) makes c^KV_t = column t of W^DKV
    exactly, whatever the order of the partial sums, so the encoder sees the
    edge rows themselves (signed zeros aside: a sum of products is +0)."""
    _note("case fp8 edge rows through mla_kv_append")
    c = W.fp8_edge_rows()
    c = np.where(c == 0.0, np.float32(0.0), c)  # the product of a one-hot row gives +0
    T, d = c.shape[0], 64
    h = np.zeros((T, d), dtype=np.float32)
    h[np.arange(T), np.arange(T)] = 1.0
    w_dkv = np.zeros((512, d), dtype=np.float32)
    w_dkv[:, :T] = c.T
    w_kr = W.round_bf16(np.random.default_rng(5).standard_normal((64, d)).astype(np.float32) * 0.125)
    cache = mla.PagedCache(2, "fp8", device=DEV, fill=float("nan"))
    slots = _slots(T, 2)
    pos = np.arange(T, dtype=np.int32)
    td = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV, torch.bfloat16)
    mla.kv_append(cache, td(h), td(w_dkv), td(w_kr), torch.from_numpy(pos).to(DEV), torch.from_numpy(slots).to(DEV))
    torch.cuda.synchronize()
    codes, scales = _read_fp8(cache, slots)
    ref_c = orc.kv_projection(h, w_dkv, w_kr, pos)["c_kv"]
    rc, rs = orc.quantize_latent_e4m3(ref_c.astype(np.float32))
    np.testing.assert_array_equal(scales, rs)
    np.testing.assert_array_equal(codes, rc)
