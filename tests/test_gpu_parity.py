"""GPU parity of the HIP path (through the C-ABI) against the fp64 CPU oracle.

Tolerances (stated for the three precisions of the path):
  fp32:       max |gpu - oracle| <= 1e-5 (absolute)
  bf16:       max |gpu - oracle| / max |oracle| <= 2e-2 over the whole tensor
  fp8 cache:  the same ratio <= 6e-2, against the oracle on the unquantised cache
The oracle always sees exactly the values the GPU received (bf16 inputs are
rounded before both sides get them).
"""

import math
import sys

import numpy as np
import pytest
import torch

import mla_latent_kv_30_amd as mla
from mla_latent_kv_30_amd import device_inputs as DI
from mla_latent_kv_30_amd import workload as W
from oracle import mla_oracle as orc

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _rel(gpu, ref):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.isfinite(gpu).all(), "non-finite GPU output"
    return float(np.abs(gpu - ref).max() / max(np.abs(ref).max(), 1e-30))


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _oracle_decode(dd, seqs=None, heads=None):
    h = dd.host
    off = h["offsets"]
    seqs = range(dd.wl.B) if seqs is None else seqs
    out = {"o": [], "z": [], "lse": [], "q_abs": []}
    for b in seqs:
        qc, qr, wk, wv = h["q_c"][b], h["q_r"][b], h["w_uk"], h["w_uv"]
        if heads is not None:
            qc, qr, wk, wv = qc[heads], qr[heads], wk[heads], wv[heads]
        r = orc.decode_sequence(qc, qr, h["c_kv"][off[b]:off[b + 1]], h["k_r"][off[b]:off[b + 1]], wk, wv)
        for k in out:
            out[k].append(r[k])
    return {k: np.stack(v) for k, v in out.items()}


def _run_decode(dd, num_splits=0, out_dtype=torch.float32):
    q_abs = mla.absorb_q(dd.q_c, dd.q_r, dd.pos, dd.w_uk)
    z, lse = mla.decode(q_abs, dd.cache, dd.block_table, dd.seq_lens, num_splits=num_splits)
    o = mla.upproj_v(z, dd.w_uv, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return {"q_abs": q_abs.float().cpu().numpy(), "z": z.cpu().numpy(), "lse": lse.cpu().numpy(),
            "o": o.float().cpu().numpy()}


# --------------------------------------------------------------------------- fp32

def test_tiny_f32_full_path():
    wl = W.make_workload("tiny_f32")
    _note(f"case tiny_f32 B={wl.B} H={wl.H} lens={list(wl.lens)}")
    dd = DI.decode_inputs(wl, DEV, poison=True, spare_pages=2)
    ref = _oracle_decode(dd)
    for S in (0, 1, 2, 3):
        got = _run_decode(dd, num_splits=S)
        for k in ("q_abs", "z", "lse", "o"):
            err = np.abs(got[k] - ref[k]).max()
            assert err <= 1e-5, (S, k, err)


def test_f32_ragged_lengths_and_splits():
    wl = W.make_workload("tiny_f32", B=4, lens=[1, 63, 130, 300])
    _note(f"case f32 ragged lens={list(wl.lens)}")
    dd = DI.decode_inputs(wl, DEV, poison=True, spare_pages=3)
    ref = _oracle_decode(dd)
    for S in (0, 1, 5):
        got = _run_decode(dd, num_splits=S)
        for k in ("z", "lse", "o"):
            err = np.abs(got[k] - ref[k]).max()
            assert err <= 1e-5, (S, k, err)


# --------------------------------------------------------------------------- bf16 decode

@pytest.mark.parametrize("H,lens", [
    (16, [1, 17, 64, 65, 130, 1000]),
    (32, [40, 300, 129]),
    (64, [64, 257]),
    (128, [33, 700]),
    (24, [90, 5]),
    (100, [200]),
])
def test_bf16_decode_matches_oracle(H, lens):
    wl = W.make_workload("decode_h16", B=len(lens), H=H, lens=lens)
    _note(f"case bf16 decode H={H} lens={lens}")
    dd = DI.decode_inputs(wl, DEV, poison=True, spare_pages=3)
    ref = _oracle_decode(dd)
    for S in (0, 1, 3):
        got = _run_decode(dd, num_splits=S)
        assert _rel(got["o"], ref["o"]) <= 2e-2, ("o", S)
        assert _rel(got["z"], ref["z"]) <= 2e-2, ("z", S)
        assert np.abs(got["lse"] - ref["lse"]).max() <= 2e-2, ("lse", S)
        assert _rel(got["q_abs"], ref["q_abs"]) <= 1e-2


def test_bf16_split_count_invariance_and_determinism():
    wl = W.make_workload("decode_h16", B=3, H=16, lens=[3000, 1234, 77])
    _note(f"case bf16 split invariance lens={list(wl.lens)}")
    dd = DI.decode_inputs(wl, DEV)
    q_abs = mla.absorb_q(dd.q_c, dd.q_r, dd.pos, dd.w_uk)
    outs = {}
    for S in (0, 1, 2, 7, 32):
        z, lse = mla.decode(q_abs, dd.cache, dd.block_table, dd.seq_lens, num_splits=S)
        outs[S] = (z.clone(), lse.clone())
    torch.cuda.synchronize()
    base = outs[1][0].cpu().numpy()
    for S, (z, lse) in outs.items():
        assert _rel(z.cpu().numpy(), base) <= 1e-2, S
    # same call twice: bit-identical (fixed reduction order, whichever unit merges)
    z2, _ = mla.decode(q_abs, dd.cache, dd.block_table, dd.seq_lens, num_splits=0)
    torch.cuda.synchronize()
    assert torch.equal(z2, outs[0][0])


def test_bf16_page_permutation_invariance():
    """Physical page placement must not matter (same values, different pool order)."""
    wl = W.make_workload("decode_h16", B=2, H=16, lens=[500, 129])
    _note("case bf16 page permutation")
    dd = DI.decode_inputs(wl, DEV, spare_pages=5)
    q_abs = mla.absorb_q(dd.q_c, dd.q_r, dd.pos, dd.w_uk)
    z1, _ = mla.decode(q_abs, dd.cache, dd.block_table, dd.seq_lens)
    # move every page to a new pool slot and rewrite the table
    n = dd.cache.num_pages
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(3)).to(DEV)
    moved = mla.PagedCache(n, torch.bfloat16, DEV, fill=float("nan"))
    moved.rows[perm] = dd.cache.rows
    bt2 = perm[dd.block_table.long()].to(torch.int32)
    z2, _ = mla.decode(q_abs, moved, bt2, dd.seq_lens)
    torch.cuda.synchronize()
    assert torch.equal(z1, z2)


def test_bf16_decode_equals_partial_plus_merge_and_reuses_workspace():
    """mla_decode is mla_decode_partial followed by mla_decode_merge (bit for
    bit), and a workspace can be reused by the next call."""
    lens = [4096, 1, 2500, 33, 700, 64, 65, 1900]
    wl = W.make_workload("decode_h16", B=len(lens), H=16, lens=lens)
    _note(f"case decode == partial + merge lens={lens}")
    dd = DI.decode_inputs(wl, DEV)
    q_abs = mla.absorb_q(dd.q_c, dd.q_r, dd.pos, dd.w_uk)
    B, H = wl.B, wl.H
    for S in (0, 5):
        ws = mla.decode_workspace(B, H, S, DEV)
        z1, l1 = mla.decode(q_abs, dd.cache, dd.block_table, dd.seq_lens, num_splits=S, workspace=ws)
        z1, l1 = z1.clone(), l1.clone()
        z2, l2 = mla.decode(q_abs, dd.cache, dd.block_table, dd.seq_lens, num_splits=S, workspace=ws)
        zt = torch.empty_like(z1)
        lt = torch.empty_like(l1)
        ws2 = mla.decode_partial(q_abs, dd.cache, dd.block_table, dd.seq_lens, None, zt, lt, num_splits=S)
        mla.decode_merge(dd.seq_lens, H, ws2, zt, lt, num_splits=S)
        torch.cuda.synchronize()
        assert torch.equal(z1, z2) and torch.equal(l1, l2), S
        assert torch.equal(z1, zt) and torch.equal(l1, lt), S


def test_bf16_many_short_sequences_share_units():
    """More sequences than compute units: each unit walks several sequences,
    streaming pages across their boundaries, and ranges start mid-page."""
    rng = np.random.default_rng(7)
    lens = [int(x) for x in rng.integers(1, 160, size=700)]
    wl = W.make_workload("decode_h16", B=len(lens), H=16, lens=lens)
    _note(f"case many short sequences B={wl.B} total={sum(lens)}")
    dd = DI.decode_inputs(wl, DEV, poison=True, spare_pages=2)
    got = _run_decode(dd, num_splits=0)
    seqs = list(range(0, wl.B, 7)) + [wl.B - 1]
    ref = _oracle_decode(dd, seqs=seqs)
    assert _rel(got["o"][seqs], ref["o"]) <= 2e-2
    assert _rel(got["z"][seqs], ref["z"]) <= 2e-2
    assert np.abs(got["lse"][seqs] - ref["lse"]).max() <= 2e-2


@pytest.mark.parametrize("B", [1, 63, 64, 65, 300])
def test_bf16_balanced_split_on_both_sides_of_the_one_wave_prefix(B):
    """The balanced split's prefix over the sequences is scanned by one wave
    for up to 64 sequences and by the whole workgroup beyond that, and the
    first sequence of a unit is found by a ballot or by a binary search
    accordingly: both sides of that boundary, every sequence up to B = 65 and
    a sample at B = 300."""
    rng = np.random.default_rng(100 + B)
    lens = [int(x) for x in rng.integers(1, 700, size=B)]
    wl = W.make_workload("decode_h16", B=B, H=16, lens=lens)
    _note(f"case balanced split B={B} total={sum(lens)}")
    dd = DI.decode_inputs(wl, DEV, poison=True, spare_pages=2)
    got = _run_decode(dd, num_splits=0)
    seqs = list(range(B)) if B <= 65 else list(range(0, B, 11)) + [B - 1]
    ref = _oracle_decode(dd, seqs=seqs)
    assert _rel(got["o"][seqs], ref["o"]) <= 2e-2
    assert _rel(got["z"][seqs], ref["z"]) <= 2e-2
    assert np.abs(got["lse"][seqs] - ref["lse"]).max() <= 2e-2


# --------------------------------------------------------------------------- fp8 cache decode

def _oracle_decode_dequantised(dd, seqs=None):
    """The oracle on the cache contents the fp8 path actually holds (codes x scale)."""
    h = dd.host
    codes, scales = orc.quantize_latent_e4m3(h["c_kv"])
    deq = orc.dequantize_latent_e4m3(codes, scales)
    off = h["offsets"]
    seqs = range(dd.wl.B) if seqs is None else seqs
    out = {"o": [], "z": []}
    for b in seqs:
        r = orc.decode_sequence(h["q_c"][b], h["q_r"][b], deq[off[b]:off[b + 1]], h["k_r"][off[b]:off[b + 1]],
                                h["w_uk"], h["w_uv"])
        out["o"].append(r["o"])
        out["z"].append(r["z"])
    return {k: np.stack(v) for k, v in out.items()}


@pytest.mark.parametrize("H,lens", [
    (16, [1, 64, 65, 300, 1000]),
    (128, [33, 700]),
    (40, [129, 2]),
])
def test_fp8_decode_matches_oracle(H, lens):
    wl = W.make_workload("long_fp8", B=len(lens), H=H, lens=lens)
    _note(f"case fp8 decode H={H} lens={lens}")
    dd = DI.decode_inputs(wl, DEV, poison=True, spare_pages=2)
    ref = _oracle_decode(dd)                  # unquantised cache: the stated bound
    deq = _oracle_decode_dequantised(dd)      # what the cache holds: kernel rounding only
    for S in (0, 1, 3):
        got = _run_decode(dd, num_splits=S)
        assert _rel(got["o"], ref["o"]) <= 6e-2, ("o", S)
        assert _rel(got["z"], ref["z"]) <= 6e-2, ("z", S)
        assert _rel(got["o"], deq["o"]) <= 2e-2, ("o vs dequantised", S)
        assert _rel(got["z"], deq["z"]) <= 2e-2, ("z vs dequantised", S)


# --------------------------------------------------------------------------- pieces

def test_cache_write_rows_match_oracle_rope():
    wl = W.make_workload("decode_h16", B=2, H=16, lens=[70, 131])
    dd = DI.decode_inputs(wl, DEV, poison=True, spare_pages=1)
    torch.cuda.synchronize()
    rows = dd.cache.rows.float().cpu().numpy().reshape(-1, 576)
    slots = dd.layout.slots
    c, k = dd.host["c_kv"], dd.host["k_r"]
    np.testing.assert_array_equal(rows[slots, :512], c)
    kr_ref = orc.rope(k, dd.layout.positions)
    assert np.abs(rows[slots, 512:] - kr_ref).max() <= 2 ** -8 * np.abs(kr_ref).max()
    # untouched slots keep their poison
    unused = np.setdiff1d(np.arange(rows.shape[0]), slots)
    assert np.isnan(rows[unused]).all()


def test_fp8_cache_write_bit_exact():
    wl = W.make_workload("long_fp8", B=2, H=16, lens=[100, 64])
    _note("case fp8 cache write")
    dd = DI.decode_inputs(wl, DEV, spare_pages=1)
    torch.cuda.synchronize()
    slots = dd.layout.slots
    codes = dd.cache.ckv.cpu().numpy().reshape(-1, 512)[slots]
    scales = dd.cache.scale.cpu().numpy().reshape(-1, 4)[slots]
    rc, rs = orc.quantize_latent_e4m3(dd.host["c_kv"])
    np.testing.assert_array_equal(scales, rs)
    np.testing.assert_array_equal(codes, rc)
    kr = dd.cache.kr.float().cpu().numpy().reshape(-1, 64)[slots]
    kr_ref = orc.rope(dd.host["k_r"], dd.layout.positions)
    assert np.abs(kr - kr_ref).max() <= 2 ** -8 * np.abs(kr_ref).max()


def test_upproj_bf16_and_f32():
    g = torch.Generator().manual_seed(5)
    for H, N in [(16, 3), (128, 300), (7, 1)]:
        z = torch.randn(N, H, 512, generator=g)
        w = (torch.randn(H, 128, 512, generator=g) / math.sqrt(512)).to(torch.bfloat16)
        ref = np.einsum("hdc,nhc->nhd", w.double().numpy(), z.double().numpy())
        o = mla.upproj_v(z.to(DEV), w.to(DEV), out_dtype=torch.float32)
        ob = mla.upproj_v(z.to(DEV), w.to(DEV), out_dtype=torch.bfloat16)
        of = mla.upproj_v(z.to(DEV), w.float().to(DEV), out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert _rel(o.cpu().numpy(), ref) <= 1e-2
        assert _rel(ob.float().cpu().numpy(), ref) <= 2e-2
        assert np.abs(of.cpu().numpy() - ref).max() <= 1e-5


@pytest.mark.parametrize("N,H", [(1, 24), (16, 24), (31, 24), (32, 24), (33, 24), (64, 24), (100, 24), (128, 24),
                                 (129, 24), (300, 24), (300, 5), (129, 3), (40, 1), (300, 128), (1000, 64)])
def test_absorb_and_upproj_row_counts(N, H):
    """mla_absorb_q and mla_upproj_v (bf16) at row counts on both sides of
    the few-rows kernels' limit (32 rows) and of the tiled kernels' row
    blocks, against the oracle's absorption and RoPE and an fp64 product.
    Rows and heads are ragged against the tiles; with H = 5, 3 and 1 the
    absorb's jobs are not a whole number of its groups of eight, so some of
    its workgroups have no job; with H = 128 and 64 each absorb workgroup
    walks several row blocks (3 and 4), the last one ragged."""
    _note(f"case absorb/upproj N={N} H={H}")
    g = torch.Generator().manual_seed(100 + N + 1000 * H)
    q_c = torch.randn(N, H, 128, generator=g).to(torch.bfloat16)
    q_r = torch.randn(N, H, 64, generator=g).to(torch.bfloat16)
    pos = torch.randint(0, 40000, (N,), generator=g, dtype=torch.int32)
    w_uk = (torch.randn(H, 128, 512, generator=g) / math.sqrt(512)).to(torch.bfloat16)
    q_abs = mla.absorb_q(q_c.to(DEV), q_r.to(DEV), pos.to(DEV), w_uk.to(DEV))
    z = torch.randn(N, H, 512, generator=g)
    w_uv = (torch.randn(H, 128, 512, generator=g) / math.sqrt(512)).to(torch.bfloat16)
    o = mla.upproj_v(z.to(DEV), w_uv.to(DEV), out_dtype=torch.float32)
    torch.cuda.synchronize()
    qa = q_abs.float().cpu().numpy()
    ref_c = orc.absorb_query(q_c.double().numpy(), w_uk.double().numpy())
    ref_r = orc.rope(q_r.double().numpy(), pos.numpy()[:, None])
    assert _rel(qa[..., :512], ref_c) <= 1e-2
    assert _rel(qa[..., 512:], ref_r) <= 1e-2
    ref_o = np.einsum("hdc,nhc->nhd", w_uv.double().numpy(), z.double().numpy())
    assert _rel(o.cpu().numpy(), ref_o) <= 1e-2


@pytest.mark.parametrize("H,lens,S", [
    (16, [1, 17, 64, 65, 130, 1000, 2500], 0),   # balanced split: pieces merged, some sequences whole
    (16, [300, 1000], 3),                        # uniform split
    (128, [33, 700, 5], 0),
    (16, [50, 900], 1),                          # no partials at all: z straight from the decode pass
])
def test_merge_upproj_matches_oracle_and_separate_calls(H, lens, S):
    wl = W.make_workload("decode_h16", B=len(lens), H=H, lens=lens)
    _note(f"case merge+upproj H={H} lens={lens} S={S}")
    dd = DI.decode_inputs(wl, DEV, poison=True, spare_pages=2)
    ref = _oracle_decode(dd)
    B = wl.B
    q_abs = mla.absorb_q(dd.q_c, dd.q_r, dd.pos, dd.w_uk)
    ws = mla.decode_workspace(B, H, S, DEV)
    # separate calls
    z1 = torch.empty((B, H, 512), device=DEV)
    l1 = torch.empty((B, H), device=DEV)
    mla.decode_partial(q_abs, dd.cache, dd.block_table, dd.seq_lens, ws, z1, l1, num_splits=S)
    mla.decode_merge(dd.seq_lens, H, ws, z1, l1, num_splits=S)
    o1 = mla.upproj_v(z1, dd.w_uv)
    # fused, into buffers holding garbage
    z2 = torch.full((B, H, 512), float("nan"), device=DEV)
    l2 = torch.full((B, H), float("nan"), device=DEV)
    mla.decode_partial(q_abs, dd.cache, dd.block_table, dd.seq_lens, ws, z2, l2, num_splits=S)
    o2 = mla.decode_merge_upproj(dd.seq_lens, H, ws, z2, dd.w_uv, lse=l2, num_splits=S)
    o2b = mla.decode_merge_upproj(dd.seq_lens, H, ws, z2, dd.w_uv, lse=l2, num_splits=S, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    # same merge, pieces folded in batches of 16 instead of 32: equal up to rounding order
    assert _rel(z2.cpu().numpy(), z1.cpu().numpy()) <= 1e-6
    assert (l2 - l1).abs().max().item() <= 1e-5
    o2n, o1n = o2.cpu().numpy(), o1.cpu().numpy()
    assert _rel(o2n, ref["o"]) <= 2e-2
    assert _rel(o2b.float().cpu().numpy(), ref["o"]) <= 2e-2
    if H <= 64:
        # the fused product keeps z in fp32; the matrix-core one rounds it to bf16
        assert _rel(o2n, o1n) <= 1e-2
        zz = z2.double().cpu().numpy()
        o_exact = np.einsum("hdc,bhc->bhd", dd.host["w_uv"], zz)
        assert np.abs(o2n - o_exact).max() <= 1e-4 * max(1.0, np.abs(o_exact).max())
    else:
        # more than 64 heads: mla_decode_merge_upproj is the two separate calls
        np.testing.assert_array_equal(o2n, o1n)


def test_merge_upproj_many_sequences_and_f32_weights_take_the_two_launch_path():
    wl = W.make_workload("decode_h16", B=40, H=16, lens=[int(x) for x in np.random.default_rng(3).integers(1, 400, 40)])
    _note(f"case merge+upproj B={wl.B}")
    dd = DI.decode_inputs(wl, DEV)
    ref = _oracle_decode(dd, seqs=[0, 13, 39])
    q_abs = mla.absorb_q(dd.q_c, dd.q_r, dd.pos, dd.w_uk)
    ws = mla.decode_workspace(wl.B, wl.H, 0, DEV)
    z = torch.empty((wl.B, wl.H, 512), device=DEV)
    mla.decode_partial(q_abs, dd.cache, dd.block_table, dd.seq_lens, ws, z, None)
    o = mla.decode_merge_upproj(dd.seq_lens, wl.H, ws, z, dd.w_uv)
    torch.cuda.synchronize()
    assert _rel(o.cpu().numpy()[[0, 13, 39]], ref["o"]) <= 2e-2
    # fp32 weights on a small batch: merge then the fp32 up-projection
    wl2 = W.make_workload("tiny_f32", B=2, lens=[64, 200])
    dd2 = DI.decode_inputs(wl2, DEV)
    ref2 = _oracle_decode(dd2)
    q2 = mla.absorb_q(dd2.q_c, dd2.q_r, dd2.pos, dd2.w_uk)
    ws2 = mla.decode_workspace(2, wl2.H, 0, DEV)
    z2 = torch.empty((2, wl2.H, 512), device=DEV)
    mla.decode_partial(q2, dd2.cache, dd2.block_table, dd2.seq_lens, ws2, z2, None)
    o2 = mla.decode_merge_upproj(dd2.seq_lens, wl2.H, ws2, z2, dd2.w_uv)
    torch.cuda.synchronize()
    assert np.abs(o2.cpu().numpy() - ref2["o"]).max() <= 1e-5


@pytest.mark.parametrize("H,lens", [(16, [3000, 1, 700, 64, 1500]), (128, [900, 33, 2048])])
def test_step_graph_replays_match_eager(H, lens):
    """The decode step captured as a HIP graph, as bench.py times it: every
    replay, with eager work and synchronisations between replays, equals the
    eager result bit for bit.  (The step records no memset: the workspace
    needs no clearing.)"""
    wl = W.make_workload("decode_h16", B=len(lens), H=H, lens=lens)
    _note(f"case graph replay H={H} lens={lens}")
    dd = DI.decode_inputs(wl, DEV)
    B = wl.B
    q_abs = torch.empty((B, H, 576), dtype=torch.bfloat16, device=DEV)
    z = torch.empty((B, H, 512), device=DEV)
    lse = torch.empty((B, H), device=DEV)
    o = torch.empty((B, H, 128), device=DEV)
    ws = mla.decode_workspace(B, H, 0, DEV)

    def step():
        mla.absorb_q(dd.q_c, dd.q_r, dd.pos, dd.w_uk, out=q_abs)
        mla.decode_partial(q_abs, dd.cache, dd.block_table, dd.seq_lens, ws, z, lse)
        mla.decode_merge_upproj(dd.seq_lens, H, ws, z, dd.w_uv, lse=lse, out=o)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (q_abs, z, lse, o)]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        for t in (q_abs, z, lse, o):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((q_abs, z, lse, o), ref):
            assert torch.equal(got, want), rep
        step()  # eager work between replays
        torch.cuda.synchronize()


def test_multi_step_graph_over_replicas_matches_eager():
    """Several decode steps in one HIP graph, each over its own replica of the
    inputs (its own cache, queries and weights), as bench.py captures them:
    after every replay each replica's outputs equal its eager step bit for bit,
    with the graphs' replays alternating and eager work in between."""
    lens = [3000, 1, 700, 64, 1500]
    H, R, G = 16, 3, 3
    _note(f"case multi-step graph H={H} replicas={R} lens={lens}")
    reps = []
    for r in range(R):
        wl = W.make_workload("decode_h16", seed=r, B=len(lens), H=H, lens=lens)
        dd = DI.decode_inputs(wl, DEV, keep_host=False)
        B = wl.B
        outs = (torch.empty((B, H, 576), dtype=torch.bfloat16, device=DEV), torch.empty((B, H, 512), device=DEV),
                torch.empty((B, H), device=DEV), torch.empty((B, H, 128), device=DEV))
        reps.append((dd, outs, mla.decode_workspace(B, H, 0, DEV)))

    def step(r):
        dd, (q_abs, z, lse, o), ws = reps[r]
        mla.absorb_q(dd.q_c, dd.q_r, dd.pos, dd.w_uk, out=q_abs)
        mla.decode_partial(q_abs, dd.cache, dd.block_table, dd.seq_lens, ws, z, lse)
        mla.decode_merge_upproj(dd.seq_lens, H, ws, z, dd.w_uv, lse=lse, out=o)

    for r in range(R):
        step(r)
    torch.cuda.synchronize()
    ref = [[t.clone() for t in reps[r][1]] for r in range(R)]
    assert not torch.equal(ref[0][3], ref[1][3])  # the replicas differ
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graphs = []
    with torch.cuda.stream(side):
        for j in range(2):  # two graphs that start at different replicas
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                for i in range(G):
                    step((j + i) % R)
            graphs.append(g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        for r in range(R):
            for t in reps[r][1]:
                t.fill_(float("nan"))
        torch.cuda.synchronize()
        graphs[rep % 2].replay()
        torch.cuda.synchronize()
        for r in range(R):
            for got, want in zip(reps[r][1], ref[r]):
                assert torch.equal(got, want), (rep, r)
        step(rep % R)  # eager work between replays
        torch.cuda.synchronize()


# --------------------------------------------------------------------------- multi-token decode

def _oracle_multi(dd, q_c, q_r, q_len, seqs=None):
    """Query token t of sequence b is the newest token of the prefix of length
    L_b - q_len + t + 1: the oracle's one-token decode on that prefix."""
    h = dd.host
    off = h["offsets"]
    seqs = range(dd.wl.B) if seqs is None else seqs
    out = {"o": [], "z": [], "lse": []}
    for b in seqs:
        L = int(dd.wl.lens[b])
        per = {"o": [], "z": [], "lse": []}
        for t in range(q_len):
            n = L - q_len + t + 1
            r = orc.decode_sequence(q_c[b, t], q_r[b, t], h["c_kv"][off[b]:off[b] + n], h["k_r"][off[b]:off[b] + n],
                                    h["w_uk"], h["w_uv"])
            for k in per:
                per[k].append(r[k])
        for k in out:
            out[k].append(np.stack(per[k]))
    return {k: np.stack(v) for k, v in out.items()}


@pytest.mark.parametrize("name,H,q_len,lens,tol", [
    ("decode_h16", 16, 2, [2, 5, 64, 65, 300, 1000], 2e-2),
    ("decode_h16", 32, 4, [4, 97, 700], 2e-2),
    ("decode_h16", 40, 3, [3, 129], 2e-2),
    ("tiny_f32", 16, 3, [3, 65, 200], None),
    ("long_fp8", 16, 2, [2, 65, 333], 6e-2),
])
def test_multi_token_decode_matches_oracle(name, H, q_len, lens, tol):
    wl = W.make_workload(name, B=len(lens), H=H, lens=lens)
    _note(f"case multi-token {name} H={H} q_len={q_len} lens={lens}")
    dd = DI.decode_inputs(wl, DEV, poison=True, spare_pages=2)
    q_c, q_r, pos, hq_c, hq_r = DI.multi_query_inputs(dd, q_len)
    ref = _oracle_multi(dd, hq_c, hq_r, q_len)
    B = wl.B
    q_abs = mla.absorb_q(q_c, q_r, pos, dd.w_uk).view(B, q_len, H, 576)
    for S in (0, 1, 3):
        z, lse = mla.decode_multi(q_abs, dd.cache, dd.block_table, dd.seq_lens, num_splits=S)
        o = mla.upproj_v(z.view(B * q_len, H, 512), dd.w_uv).view(B, q_len, H, 128)
        torch.cuda.synchronize()
        zn, ln, on = z.cpu().numpy(), lse.cpu().numpy(), o.cpu().numpy()
        if tol is None:  # fp32 path: absolute 1e-5
            assert np.abs(zn - ref["z"]).max() <= 1e-5, S
            assert np.abs(on - ref["o"]).max() <= 1e-5, S
            assert np.abs(ln - ref["lse"]).max() <= 1e-5, S
        else:
            assert _rel(on, ref["o"]) <= tol, ("o", S)
            assert _rel(zn, ref["z"]) <= tol, ("z", S)
            assert np.abs(ln - ref["lse"]).max() <= tol, ("lse", S)


@pytest.mark.parametrize("name,H,q_len,lens,o_dtype", [
    ("decode_h16", 16, 2, [1500, 9, 700, 64], torch.float32),     # fused merge + W^UV (B <= 32)
    ("decode_h16", 32, 4, [3000, 200], torch.bfloat16),
    ("tiny_f32", 16, 3, [300, 64, 5], torch.float32),             # fp32 weights: merge, then upproj_v
    ("long_fp8", 64, 2, [2048, 131], torch.float32),
])
def test_multi_token_decode_upproj_matches_oracle(name, H, q_len, lens, o_dtype):
    """mla_decode_multi_upproj: the up-projected outputs of every query token
    (head h' of the merge takes W^UV row block h' % H), for the automatic and
    explicit splits."""
    wl = W.make_workload(name, B=len(lens), H=H, lens=lens)
    _note(f"case multi-token upproj {name} H={H} q_len={q_len} lens={lens}")
    dd = DI.decode_inputs(wl, DEV, poison=True, spare_pages=2)
    q_c, q_r, pos, hq_c, hq_r = DI.multi_query_inputs(dd, q_len)
    ref = _oracle_multi(dd, hq_c, hq_r, q_len)
    B = wl.B
    q_abs = mla.absorb_q(q_c, q_r, pos, dd.w_uk).view(B, q_len, H, 576)
    tol = {"decode_h16": 2e-2, "long_fp8": 6e-2}.get(name)
    for S in (0, 1, 3):
        lse = torch.empty((B, q_len, H), device=DEV)
        o, z, lse = mla.decode_multi_upproj(q_abs, dd.cache, dd.block_table, dd.seq_lens, dd.w_uv, num_splits=S,
                                            lse=lse, out_dtype=o_dtype)
        torch.cuda.synchronize()
        on, zn, ln = o.float().cpu().numpy(), z.cpu().numpy(), lse.cpu().numpy()
        if tol is None:  # fp32 path
            assert np.abs(on - ref["o"]).max() <= 1e-5, S
            assert np.abs(zn - ref["z"]).max() <= 1e-5, S
        else:
            assert _rel(on, ref["o"]) <= tol, ("o", S)
            assert _rel(zn, ref["z"]) <= tol, ("z", S)
            assert np.abs(ln - ref["lse"]).max() <= tol, ("lse", S)


def test_multi_token_decode_with_one_token_equals_decode():
    wl = W.make_workload("decode_h16", B=3, H=16, lens=[3000, 77, 1])
    _note("case multi-token q_len=1")
    dd = DI.decode_inputs(wl, DEV)
    q_abs = mla.absorb_q(dd.q_c, dd.q_r, dd.pos, dd.w_uk)
    z1, l1 = mla.decode(q_abs, dd.cache, dd.block_table, dd.seq_lens)
    z2, l2 = mla.decode_multi(q_abs.view(3, 1, 16, 576), dd.cache, dd.block_table, dd.seq_lens)
    torch.cuda.synchronize()
    assert torch.equal(z1, z2.view(3, 16, 512)) and torch.equal(l1, l2.view(3, 16))


# --------------------------------------------------------------------------- YaRN

@pytest.mark.parametrize("name,lens,tol", [
    ("decode_h16", [70, 1000, 5000], 2e-2),
    ("tiny_f32", [64, 300], None),
])
def test_yarn_decode_matches_oracle(name, lens, tol):
    """k^R written and q^R rotated with YaRN frequencies (s = 40, alpha = 1,
    beta = 32, 4K original context), softmax scale times 0.1 ln s + 1."""
    wl = W.make_workload(name, B=len(lens), H=16, lens=lens)
    _note(f"case YaRN decode {name} lens={lens}")
    rope = mla.yarn_rope()
    dd = DI.decode_inputs(wl, DEV, poison=True, spare_pages=1, rope=rope)
    scale = mla.default_softmax_scale() * mla.yarn_attention_factor(40.0)
    q_abs = mla.absorb_q(dd.q_c, dd.q_r, dd.pos, dd.w_uk, rope=rope)
    z, lse = mla.decode(q_abs, dd.cache, dd.block_table, dd.seq_lens, softmax_scale=scale)
    o = mla.upproj_v(z, dd.w_uv)
    torch.cuda.synchronize()
    h = dd.host
    off = h["offsets"]
    theta = orc.yarn_frequencies()
    oscale = orc.default_softmax_scale() * orc.yarn_attention_factor(40.0)
    for b in range(wl.B):
        r = orc.decode_sequence(h["q_c"][b], h["q_r"][b], h["c_kv"][off[b]:off[b + 1]], h["k_r"][off[b]:off[b + 1]],
                                h["w_uk"], h["w_uv"], softmax_scale=oscale, rope_theta=theta)
        if tol is None:
            assert np.abs(o[b].cpu().numpy() - r["o"]).max() <= 1e-5, b
            assert np.abs(q_abs[b].cpu().numpy() - r["q_abs"]).max() <= 1e-5, b
        else:
            assert _rel(o[b].cpu().numpy(), r["o"]) <= tol, b
            assert _rel(z[b].cpu().numpy(), r["z"]) <= tol, b
            assert np.abs(lse[b].cpu().numpy() - r["lse"]).max() <= tol, b
            assert _rel(q_abs[b].float().cpu().numpy(), r["q_abs"]) <= 1e-2, b
    # the rotated keys in the cache are the oracle's YaRN rotation
    rows = dd.cache.rows.float().cpu().numpy().reshape(-1, 576)[dd.layout.slots]
    kr_ref = orc.rope(h["k_r"], dd.layout.positions, theta=theta)
    assert np.abs(rows[:, 512:] - kr_ref).max() <= (2 ** -8 if tol else 1e-6) * np.abs(kr_ref).max()


def test_yarn_prefill_matches_oracle():
    T, H = 150, 16
    wl = W.make_workload("prefill_h128", H=H, lens=[T])
    _note("case YaRN prefill")
    dt = torch.bfloat16
    w_uk, w_uv = W.weights(wl)
    q_c, q_r = W.queries(wl)
    c, k = W.sequence_latents(wl, 0)
    npg = (T + 63) // 64
    cache = mla.PagedCache(npg, dt, DEV, fill=float("nan"))
    bt = torch.arange(npg, dtype=torch.int32, device=DEV)
    td = lambda x: torch.from_numpy(x).to(DEV, dt)
    rope = mla.yarn_rope()
    scale = mla.default_softmax_scale() * mla.yarn_attention_factor(40.0)
    q_abs = mla.absorb_q(td(q_c), td(q_r), torch.arange(T, dtype=torch.int32, device=DEV), td(w_uk), rope=rope)
    z, lse = mla.prefill_causal(q_abs, td(c), td(k), cache, bt, softmax_scale=scale, rope=rope)
    torch.cuda.synchronize()
    ref = orc.prefill_causal(q_c, q_r, c, k, w_uk, w_uv, softmax_scale=orc.default_softmax_scale() *
                             orc.yarn_attention_factor(40.0), rope_theta=orc.yarn_frequencies())
    assert _rel(z.cpu().numpy(), ref["z"]) <= 2e-2
    assert np.abs(lse.cpu().numpy() - ref["lse"]).max() <= 2e-2


def test_yarn_with_factor_one_is_plain_rope():
    wl = W.make_workload("decode_h16", B=2, H=16, lens=[300, 65])
    dd = DI.decode_inputs(wl, DEV)
    plain = mla.absorb_q(dd.q_c, dd.q_r, dd.pos, dd.w_uk)
    one = mla.absorb_q(dd.q_c, dd.q_r, dd.pos, dd.w_uk, rope=mla.MlaRope(10000.0, 1.0, 1.0, 32.0, 4096))
    torch.cuda.synchronize()
    assert torch.equal(plain, one)


# --------------------------------------------------------------------------- prefill

@pytest.mark.parametrize("H,T", [(16, 200), (128, 130)])
def test_bf16_prefill_matches_oracle(H, T):
    wl = W.make_workload("prefill_h128", H=H, lens=[T])
    _note(f"case bf16 prefill H={H} T={T}")
    dt = torch.bfloat16
    w_uk, w_uv = W.weights(wl)
    q_c, q_r = W.queries(wl)
    c, k = W.sequence_latents(wl, 0)
    npg = (T + 63) // 64
    cache = mla.PagedCache(npg + 2, dt, DEV, fill=float("nan"))
    bt = torch.tensor(np.random.default_rng(1).permutation(npg + 2)[:npg], dtype=torch.int32, device=DEV)
    pos = torch.arange(T, dtype=torch.int32, device=DEV)
    td = lambda x: torch.from_numpy(x).to(DEV, dt)
    q_abs = mla.absorb_q(td(q_c), td(q_r), pos, td(w_uk))
    z, lse = mla.prefill_causal(q_abs, td(c), td(k), cache, bt)
    o = mla.upproj_v(z, td(w_uv))
    torch.cuda.synchronize()
    rows = [0, 1, 63, 64, 65, T // 2, T - 1]
    ref = orc.prefill_causal(q_c, q_r, c, k, w_uk, w_uv, rows=rows)
    assert _rel(o.cpu().numpy()[rows], ref["o"]) <= 2e-2
    assert _rel(z.cpu().numpy()[rows], ref["z"]) <= 2e-2
    assert np.abs(lse.cpu().numpy()[rows] - ref["lse"]).max() <= 2e-2
    # the cache now holds exactly what a cache write produces
    pool = cache.rows.float().cpu().numpy().reshape(-1, 576)
    j = np.arange(T)
    slot = bt.cpu().numpy()[j // 64] * 64 + j % 64
    np.testing.assert_array_equal(pool[slot, :512], c)
    assert np.abs(pool[slot, 512:] - ref["k_r_rot"]).max() <= 2 ** -8 * np.abs(ref["k_r_rot"]).max()


@pytest.mark.parametrize("H", [16, 128])
def test_prefill_row_equals_decode_at_length_t_plus_1(H):
    wl = W.make_workload("prefill_h128", H=H, lens=[150])
    dt = torch.bfloat16
    w_uk, _ = W.weights(wl)
    q_c, q_r = W.queries(wl)
    c, k = W.sequence_latents(wl, 0)
    T = 150
    cache = mla.PagedCache(3, dt, DEV)
    bt = torch.tensor([2, 0, 1], dtype=torch.int32, device=DEV)
    td = lambda x: torch.from_numpy(x).to(DEV, dt)
    q_abs = mla.absorb_q(td(q_c), td(q_r), torch.arange(T, dtype=torch.int32, device=DEV), td(w_uk))
    zp, _ = mla.prefill_causal(q_abs, td(c), td(k), cache, bt)
    rows = [0, 63, 64, 149]
    lens = torch.tensor([t + 1 for t in rows], dtype=torch.int32, device=DEV)
    zd, _ = mla.decode(q_abs[rows].contiguous(), cache, bt.repeat(len(rows), 1), lens, num_splits=1)
    torch.cuda.synchronize()
    assert _rel(zd.cpu().numpy(), zp[rows].cpu().numpy()) <= 1e-3


@pytest.mark.parametrize("H", [16, 128])
def test_fp8_prefill_matches_oracle(H):
    """fp8 cache in prefill mode: the eight-wave kernel (16 heads) and the
    four-wave kernel (128 heads, staged expansion without the non-temporal
    hint)."""
    T = 150
    wl = W.make_workload("prefill_h128", H=H, lens=[T])
    _note(f"case fp8 prefill H={H} T={T}")
    dt = torch.bfloat16
    w_uk, w_uv = W.weights(wl)
    q_c, q_r = W.queries(wl)
    c, k = W.sequence_latents(wl, 0)
    npg = (T + 63) // 64
    cache = mla.PagedCache(npg + 1, "fp8", DEV, fill=float("nan"))
    bt = torch.tensor([3, 0, 2], dtype=torch.int32, device=DEV)
    td = lambda x: torch.from_numpy(x).to(DEV, dt)
    q_abs = mla.absorb_q(td(q_c), td(q_r), torch.arange(T, dtype=torch.int32, device=DEV), td(w_uk))
    z, lse = mla.prefill_causal(q_abs, td(c), td(k), cache, bt)
    o = mla.upproj_v(z, td(w_uv))
    torch.cuda.synchronize()
    rows = [0, 31, 32, 63, 64, 100, T - 1]
    ref = orc.prefill_causal(q_c, q_r, c, k, w_uk, w_uv, rows=rows)
    assert _rel(o.cpu().numpy()[rows], ref["o"]) <= 6e-2
    assert _rel(z.cpu().numpy()[rows], ref["z"]) <= 6e-2
    # the pool holds the quantised tokens
    codes = cache.ckv.cpu().numpy().reshape(-1, 512)
    j = np.arange(T)
    slot = bt.cpu().numpy()[j // 64] * 64 + j % 64
    rc, _ = orc.quantize_latent_e4m3(c)
    np.testing.assert_array_equal(codes[slot], rc)


# --------------------------------------------------------------------------- debug mode

def test_debug_mode_rejects_bad_lengths_and_pages_before_launch():
    """With mla_set_debug(1) the decode entry points check the device-side
    lengths and block table on the host and return MLA_ERR_INVALID_ARG
    (nothing launched) for a length of 0, a length past the block table, a
    page outside the pool, or fewer tokens than query tokens."""
    wl = W.make_workload("decode_h16", B=3, H=16, lens=[100, 65, 1])
    _note("case debug mode")
    dd = DI.decode_inputs(wl, DEV)
    q_abs = mla.absorb_q(dd.q_c, dd.q_r, dd.pos, dd.w_uk)
    mla.set_debug(True)
    try:
        z, lse = mla.decode(q_abs, dd.cache, dd.block_table, dd.seq_lens)   # valid inputs still run
        torch.cuda.synchronize()
        assert torch.isfinite(z).all()
        maxp = dd.block_table.shape[1]
        for b, L in ((1, 0), (0, 64 * maxp + 1)):
            bad = dd.seq_lens.clone()
            bad[b] = L
            with pytest.raises(mla.MLAError) as e:
                mla.decode(q_abs, dd.cache, dd.block_table, bad)
            assert e.value.status == mla.MLA_ERR_INVALID_ARG
        bt = dd.block_table.clone()
        bt[0, 0] = dd.cache.num_pages
        with pytest.raises(mla.MLAError):
            mla.decode(q_abs, dd.cache, bt, dd.seq_lens)
        q2 = torch.zeros((3, 2, 16, 576), dtype=torch.bfloat16, device=DEV)
        with pytest.raises(mla.MLAError):   # sequence 2 holds 1 token, 2 query tokens
            mla.decode_multi(q2, dd.cache, dd.block_table, dd.seq_lens)
    finally:
        mla.set_debug(False)
