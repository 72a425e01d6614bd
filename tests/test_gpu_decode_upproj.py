"""mla_decode_upproj: decode, merge and the W^UV up-projection of one new
token per sequence.  For up to 64 heads, a bf16 or fp8 cache and a bf16
weight on few sequences the whole step is one launch: the decode kernel
publishes every piece through a per-sequence counter in the workspace and
runs the (sequence, head) merge jobs itself.

Its results must equal, bit for bit, those of the two-launch form
(mla_decode_partial then mla_decode_merge_upproj) on the same inputs: both
merge the pieces in slot order with the same batches and the same
arithmetic.  Against the oracle the bar is the decode tolerance (2e-2 of the
output's largest magnitude for bf16, on the dequantised cache for fp8).
The counters must be zero again after every call, also under graph replay,
where no memset is recorded."""

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


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _rel(gpu, ref):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.isfinite(gpu).all(), "non-finite GPU output"
    return float(np.abs(gpu - ref).max() / max(np.abs(ref).max(), 1e-30))


def _inputs(B, H, lens, dtype="bf16", seed=0, keep_host=False):
    wl = W.make_workload("decode_h16", seed=seed, B=B, H=H, lens=lens, dtype=dtype)
    dd = DI.decode_inputs(wl, DEV, poison=True, spare_pages=2, keep_host=keep_host)
    q_abs = mla.absorb_q(dd.q_c, dd.q_r, dd.pos, dd.w_uk)
    return wl, dd, q_abs


def _two_launch(dd, q_abs, H, S, out_dtype):
    B = q_abs.shape[0]
    ws = mla.decode_workspace(B, H, S, DEV)
    z = torch.full((B, H, 512), float("nan"), device=DEV)
    lse = torch.full((B, H), float("nan"), device=DEV)
    mla.decode_partial(q_abs, dd.cache, dd.block_table, dd.seq_lens, ws, z, lse, num_splits=S)
    o = mla.decode_merge_upproj(dd.seq_lens, H, ws, z, dd.w_uv, lse=lse, num_splits=S, out_dtype=out_dtype)
    return o, z, lse


def _one_call(dd, q_abs, H, S, out_dtype, ws):
    B = q_abs.shape[0]
    z = torch.full((B, H, 512), float("nan"), device=DEV)
    lse = torch.full((B, H), float("nan"), device=DEV)
    o = torch.full((B, H, 128), float("nan"), device=DEV, dtype=out_dtype)
    mla.decode_upproj(q_abs, dd.cache, dd.block_table, dd.seq_lens, dd.w_uv, num_splits=S, workspace=ws, z=z,
                      lse=lse, out=o, out_dtype=out_dtype)
    return o, z, lse


def _counters(ws, B, H, S):
    base = mla.decode_workspace_size(B, H, S)
    return ws[base:base + 256 * B].view(torch.int32)


CASES = [
    # (B, H, lens, splits, cache dtype)
    (16, 16, "h16", 0, "bf16"),                  # the 16-head decode workload's shape, shorter
    (7, 16, [1, 17, 64, 65, 130, 1000, 2500], 0, "bf16"),  # whole and split sequences side by side
    (1, 16, [5000], 0, "bf16"),                  # one sequence over every unit
    (32, 64, "mixed", 0, "bf16"),                # four head groups, the largest batch of the one-launch form
    (20, 32, "mixed", 0, "bf16"),
    (8, 16, [300, 1000, 64, 2000, 1, 129, 4000, 700], 4, "bf16"),  # uniform split
    (5, 16, [1, 100, 1500, 3000, 64], 0, "fp8"),
    (3, 24, [2000, 33, 900], 0, "bf16"),         # heads past H in the last group
]


def _lens(spec, B, seed):
    rng = np.random.default_rng(seed)
    if spec == "h16":
        return [int(x) for x in rng.integers(1024, 4097, B)]
    if spec == "mixed":
        return [int(x) for x in rng.integers(1, 3000, B)]
    return list(spec)


@pytest.mark.parametrize("B,H,lens,S,dtype", CASES)
def test_one_launch_equals_two_launch_bitwise(B, H, lens, S, dtype):
    lens = _lens(lens, B, B * 31 + H)
    _note(f"case decode_upproj B={B} H={H} S={S} {dtype} lens[:8]={lens[:8]}")
    wl, dd, q_abs = _inputs(B, H, lens, dtype)
    ws = mla.decode_upproj_workspace(B, H, S, DEV)
    for out_dtype in (torch.float32, torch.bfloat16):
        o2, z2, l2 = _two_launch(dd, q_abs, H, S, out_dtype)
        o1, z1, l1 = _one_call(dd, q_abs, H, S, out_dtype, ws)
        torch.cuda.synchronize()
        assert torch.equal(z1, z2)
        assert torch.equal(l1, l2)
        assert torch.equal(o1, o2)
        assert int(_counters(ws, B, H, S).abs().sum().item()) == 0


@pytest.mark.parametrize("B,H,lens,dtype,tol", [
    (6, 16, [1, 64, 700, 1500, 3000, 65], "bf16", 2e-2),
    (4, 64, [2000, 1, 130, 900], "bf16", 2e-2),
    (4, 16, [1, 900, 2500, 64], "fp8", 2e-2),
])
def test_one_launch_matches_oracle(B, H, lens, dtype, tol):
    _note(f"case decode_upproj oracle B={B} H={H} {dtype} lens={lens}")
    wl, dd, q_abs = _inputs(B, H, lens, dtype, seed=5, keep_host=True)
    o, z, lse = mla.decode_upproj(q_abs, dd.cache, dd.block_table, dd.seq_lens, dd.w_uv,
                                  lse=torch.empty((B, H), device=DEV))
    torch.cuda.synchronize()
    h = dd.host
    off = h["offsets"]
    ckv_all = h["c_kv"]
    if dtype == "fp8":  # the cache as it is stored: codes times scales
        ckv_all = orc.dequantize_latent_e4m3(*orc.quantize_latent_e4m3(ckv_all))
    for b in range(B):
        r = orc.decode_sequence(h["q_c"][b], h["q_r"][b], ckv_all[off[b]:off[b + 1]], h["k_r"][off[b]:off[b + 1]],
                                h["w_uk"], h["w_uv"])
        assert _rel(o[b].cpu().numpy(), r["o"]) <= tol, b
        assert _rel(z[b].cpu().numpy(), r["z"]) <= tol, b
        assert np.abs(lse[b].cpu().numpy() - r["lse"]).max() <= 2e-2 * max(1.0, np.abs(r["lse"]).max()), b


def test_counters_reset_across_calls_of_different_sizes():
    """Calls in a row on one workspace (sized for the largest): a large batch,
    a smaller one, then the first again; each equals its two-launch result and
    leaves the counters zero."""
    ws = mla.decode_upproj_workspace(24, 64, 0, DEV)
    runs = [(24, 64, 1), (3, 16, 2), (24, 64, 1)]
    for k, (B, H, seed) in enumerate(runs):
        lens = _lens("mixed", B, seed)
        _note(f"case decode_upproj sequence call {k} B={B} H={H}")
        wl, dd, q_abs = _inputs(B, H, lens, seed=seed)
        o2, z2, l2 = _two_launch(dd, q_abs, H, 0, torch.float32)
        o1, z1, l1 = _one_call(dd, q_abs, H, 0, torch.float32, ws)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(z1, z2) and torch.equal(l1, l2), k
        base = mla.decode_workspace_size(B, H, 0)
        assert int(ws[base:base + 256 * B].view(torch.int32).abs().sum().item()) == 0, k


def test_alternating_inputs_of_one_shape_read_fresh_pieces():
    """Two input sets with the same lengths (so the same pieces land in the
    same workspace slots) in alternation: a merge that read a piece left by
    the previous call, or a piece not yet complete, would show as a mismatch
    with the two-launch result of the current inputs."""
    B, H = 16, 16
    lens = _lens("h16", B, 4)
    _note(f"case decode_upproj alternating inputs B={B} H={H}")
    sets = [_inputs(B, H, lens, seed=s) for s in (21, 22)]
    refs = [_two_launch(dd, q_abs, H, 0, torch.float32) for _, dd, q_abs in sets]
    torch.cuda.synchronize()
    assert not torch.equal(refs[0][0], refs[1][0])
    ws = mla.decode_upproj_workspace(B, H, 0, DEV)
    for k in range(8):
        _, dd, q_abs = sets[k % 2]
        o1, z1, l1 = _one_call(dd, q_abs, H, 0, torch.float32, ws)
        torch.cuda.synchronize()
        o2, z2, l2 = refs[k % 2]
        assert torch.equal(o1, o2) and torch.equal(z1, z2) and torch.equal(l1, l2), k


def test_graph_replays_match_eager():
    """The step (absorb, then the one-launch decode) captured as a HIP graph:
    every replay, with eager calls in between, equals the eager result bit for
    bit, and the counters are zero after each."""
    B, H = 9, 16
    lens = [3000, 1, 700, 64, 1500, 2048, 33, 4000, 999]
    _note(f"case decode_upproj graph B={B} H={H}")
    wl, dd, _ = _inputs(B, H, lens, seed=3)
    q_abs = torch.empty((B, H, 576), dtype=torch.bfloat16, device=DEV)
    z = torch.empty((B, H, 512), device=DEV)
    lse = torch.empty((B, H), device=DEV)
    o = torch.empty((B, H, 128), device=DEV)
    ws = mla.decode_upproj_workspace(B, H, 0, DEV)

    def step():
        mla.absorb_q(dd.q_c, dd.q_r, dd.pos, dd.w_uk, out=q_abs)
        mla.decode_upproj(q_abs, dd.cache, dd.block_table, dd.seq_lens, dd.w_uv, workspace=ws, z=z, lse=lse, out=o)

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
    cnt = _counters(ws, B, H, 0)
    for rep in range(4):
        for t in (q_abs, z, lse, o):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((q_abs, z, lse, o), ref):
            assert torch.equal(got, want), rep
        assert int(cnt.abs().sum().item()) == 0, rep
        step()
        torch.cuda.synchronize()


def test_outside_the_one_launch_form_equals_two_launch():
    """128 heads (the four-wave kernel), fp32 weights and 40 sequences take
    the two-launch path inside mla_decode_upproj."""
    for B, H, wdt in ((3, 128, torch.bfloat16), (4, 16, torch.float32), (40, 16, torch.bfloat16)):
        lens = _lens("mixed", B, 77 + B)
        _note(f"case decode_upproj two-launch form B={B} H={H} w={wdt}")
        wl, dd, q_abs = _inputs(B, H, lens, seed=B)
        w = dd.w_uv.to(wdt).contiguous()
        ws = mla.decode_workspace(B, H, 0, DEV)
        z2 = torch.empty((B, H, 512), device=DEV)
        l2 = torch.empty((B, H), device=DEV)
        mla.decode_partial(q_abs, dd.cache, dd.block_table, dd.seq_lens, ws, z2, l2)
        o2 = mla.decode_merge_upproj(dd.seq_lens, H, ws, z2, w, lse=l2)
        o1, z1, l1 = mla.decode_upproj(q_abs, dd.cache, dd.block_table, dd.seq_lens, w,
                                       lse=torch.empty((B, H), device=DEV))
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(z1, z2) and torch.equal(l1, l2)


def test_workspace_too_small_is_refused():
    B, H = 4, 16
    wl, dd, q_abs = _inputs(B, H, [100, 200, 300, 400])
    small = torch.zeros(mla.decode_workspace_size(B, H, 0), dtype=torch.uint8, device=DEV)
    with pytest.raises(mla.MLAError) as e:
        mla.decode_upproj(q_abs, dd.cache, dd.block_table, dd.seq_lens, dd.w_uv, workspace=small)
    assert e.value.status == mla.MLA_ERR_WORKSPACE
