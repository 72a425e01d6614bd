"""Host-side checks of the seeded workload generator and the paged layout."""

import numpy as np
import torch

from mla_latent_kv_30_amd import workload as W


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([0.0, -0.0, 1e-40, 3.0e38, 1.00390625, 1.01171875], dtype=np.float32)])
    ours = W.round_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(ours.view(np.uint32), ref.view(np.uint32))


def test_streams_are_deterministic_and_independent():
    a = W.stream(0, "decode_h16", "c_KV", 3).standard_normal(8)
    b = W.stream(0, "decode_h16", "c_KV", 3).standard_normal(8)
    c = W.stream(0, "decode_h16", "c_KV", 4).standard_normal(8)
    np.testing.assert_array_equal(a, b)
    assert not np.array_equal(a, c)


def test_named_workloads_shapes():
    wl = W.make_workload("decode_h16")
    assert wl.B == 16 and wl.H == 16 and wl.dtype == "bf16"
    assert ((wl.lens >= 1024) & (wl.lens <= 4096)).all()
    wl = W.make_workload("decode_h128")
    assert wl.B == 64 and wl.H == 128 and ((wl.lens >= 8192) & (wl.lens <= 32768)).all()
    wl = W.make_workload("tiny_f32")
    assert wl.B == 1 and wl.H == 16 and list(wl.lens) == [64] and wl.dtype == "f32"
    wl = W.make_workload("long_fp8")
    assert wl.B == 8 and (wl.lens == 131072).all() and wl.splits == 32 and wl.dtype == "fp8"
    wl = W.make_workload("prefill_h128")
    assert wl.kind == "prefill" and wl.B == 1 and wl.lens[0] == 8192


def test_inputs_are_bf16_representable_and_scaled():
    wl = W.make_workload("decode_h16", B=2, lens=[70, 130])
    w_uk, w_uv = W.weights(wl)
    assert w_uk.shape == (16, 128, 512)
    assert (W.round_bf16(w_uk) == w_uk).all()
    assert abs(w_uk.std() - 512 ** -0.5) < 0.01 * 512 ** -0.5 * 10
    c, k = W.sequence_latents(wl, 1)
    assert c.shape == (130, 512) and k.shape == (130, 64)
    assert abs(c.std() - 1.0) < 0.05
    c2, _ = W.sequence_latents(wl, 1)
    np.testing.assert_array_equal(c, c2)


def test_paged_layout_is_a_permutation():
    wl = W.make_workload("decode_h16", B=5, lens=[1, 64, 65, 200, 128])
    pl = W.paged_layout(wl, spare_pages=3)
    assert pl.num_pages == 1 + 1 + 2 + 4 + 2 + 3
    used = pl.block_table[pl.block_table >= 0]
    assert len(np.unique(used)) == used.size == 10
    assert len(np.unique(pl.slots)) == pl.slots.size == wl.total_tokens
    for b in range(wl.B):
        L = int(wl.lens[b])
        s = pl.slots[pl.offsets[b]:pl.offsets[b + 1]]
        j = np.arange(L)
        np.testing.assert_array_equal(s, pl.block_table[b, j // 64] * 64 + j % 64)
        np.testing.assert_array_equal(pl.positions[pl.offsets[b]:pl.offsets[b + 1]], j)
        assert (pl.block_table[b, (L + 63) // 64:] == -1).all()
