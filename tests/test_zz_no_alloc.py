"""mla_decode_noalloc, the decode entry point that takes no workspace (its
split partials live in a device array inside the library), called through
the C interface against mla_decode on the same inputs.  Both run the same
kernels with the same launch shapes, so z and lse must agree bit for bit
(stricter than the 2e-2 bf16 / 6e-2 fp8 bar of the decode parity tests).

Each case makes two calls in a row, the second with a smaller input: the
array then still holds the first call's partials, which the second must
neither need cleared nor be disturbed by.  A call whose partials exceed the
array is refused with MLA_ERR_WORKSPACE."""

import sys

import pytest
import torch

import mla_latent_kv_30_amd as mla
from mla_latent_kv_30_amd import device_inputs as DI
from mla_latent_kv_30_amd import workload as W

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _case(B, H, lens, dtype, seed):
    wl = W.make_workload("decode_h16", seed=seed, B=B, H=H, lens=lens, dtype=dtype)
    dd = DI.decode_inputs(wl, DEV, poison=True, spare_pages=2, keep_host=False)
    q_abs = mla.absorb_q(dd.q_c, dd.q_r, dd.pos, dd.w_uk)
    return dd, q_abs


def _nan_like(t):
    return torch.full_like(t, float("nan"))


@pytest.mark.parametrize("dtype,big,small", [
    # automatic split: 128 heads (the four-wave kernel) then 16 heads
    ("bf16", (12, 128, 2000, 9000, 0), (5, 16, 1, 3000, 0)),
    # fixed split, fp8 cache; the second call has fewer heads and splits
    ("fp8", (8, 128, 4000, 20000, 8), (3, 32, 100, 5000, 3)),
    # the largest automatic-split call the array holds at 128 heads: B = 64
    ("bf16", (64, 128, 64, 2000, 0), (2, 128, 33, 700, 0)),
])
def test_noalloc_matches_decode_on_two_calls(dtype, big, small):
    gen = torch.Generator().manual_seed(11)
    cases = []
    for k, (B, H, lo, hi, S) in enumerate((big, small)):
        lens = torch.randint(lo, hi + 1, (B,), generator=gen).tolist()
        _note(f"case noalloc {dtype} B={B} H={H} lens in [{lo}, {hi}] splits={S}")
        assert mla.decode_workspace_size(B, H, S) <= mla.NOALLOC_SCRATCH_BYTES
        dd, q_abs = _case(B, H, lens, dtype, seed=k)
        z_ref, lse_ref = mla.decode(q_abs, dd.cache, dd.block_table, dd.seq_lens, num_splits=S)
        cases.append((dd, q_abs, S, z_ref, lse_ref))
    torch.cuda.synchronize()
    outs = [(_nan_like(c[3]), _nan_like(c[4])) for c in cases]
    for (dd, q_abs, S, _, _), (z, lse) in zip(cases, outs):  # two calls in a row, nothing in between
        mla.decode_noalloc(q_abs, dd.cache, dd.block_table, dd.seq_lens, z, lse, num_splits=S)
    torch.cuda.synchronize()
    for (dd, q_abs, S, z_ref, lse_ref), (z, lse) in zip(cases, outs):
        assert torch.equal(z, z_ref), ("z", S)
        assert torch.equal(lse, lse_ref), ("lse", S)
    # and once more on the first input after the second: the leftovers of a
    # smaller call do not disturb a larger one
    dd, q_abs, S, z_ref, lse_ref = cases[0]
    z, lse = _nan_like(z_ref), _nan_like(lse_ref)
    mla.decode_noalloc(q_abs, dd.cache, dd.block_table, dd.seq_lens, z, lse, num_splits=S)
    torch.cuda.synchronize()
    assert torch.equal(z, z_ref) and torch.equal(lse, lse_ref)


def test_noalloc_refuses_partials_beyond_its_array():
    B, H, S = 64, 128, 64
    assert mla.decode_workspace_size(B, H, S) > mla.NOALLOC_SCRATCH_BYTES
    _note(f"case noalloc oversized B={B} H={H} splits={S}")
    dd, q_abs = _case(B, H, [64] * B, "bf16", seed=3)
    z = torch.zeros((B, H, mla.D_C), dtype=torch.float32, device=DEV)
    with pytest.raises(mla.MLAError) as e:
        mla.decode_noalloc(q_abs, dd.cache, dd.block_table, dd.seq_lens, z, None, num_splits=S)
    assert e.value.status == mla.MLA_ERR_WORKSPACE
    # nothing was launched: z is untouched
    torch.cuda.synchronize()
    assert not z.any()
