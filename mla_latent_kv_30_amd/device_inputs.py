"""Move a seeded workload onto the GPU and fill its paged latent cache.

Host arrays come from workload.py; this module only copies them to device
memory and calls the library's cache-write entry point.  No attention
arithmetic happens here.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

from . import _lib
from . import workload as W


@dataclasses.dataclass
class DeviceDecode:
    wl: W.Workload
    layout: W.PagedLayout
    cache: _lib.PagedCache
    q_c: torch.Tensor
    q_r: torch.Tensor
    pos: torch.Tensor          # [B] query positions (L_b - 1)
    w_uk: torch.Tensor
    w_uv: torch.Tensor
    block_table: torch.Tensor  # [B, max_pages] int32 (-1 past the end)
    seq_lens: torch.Tensor     # [B] int32
    host: dict                 # the host copies (float32 numpy) the oracle uses


def _t(x: np.ndarray, dtype, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(device=device, dtype=dtype)


def decode_inputs(wl: W.Workload, device="cuda", spare_pages: int = 0, poison: bool = False,
                  keep_host: bool = True, latents: Optional[tuple] = None, rope=None) -> DeviceDecode:
    """All inputs of a decode workload on `device`, cache filled through
    mla_cache_write (so k_R is rotated by the library at its position)."""
    dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    layout = W.paged_layout(wl, spare_pages=spare_pages)
    cache = _lib.PagedCache(layout.num_pages, "fp8" if wl.dtype == "fp8" else dt, device=device,
                            fill=float("nan") if poison else None)
    w_uk, w_uv = W.weights(wl)
    q_c, q_r = W.queries(wl)
    c_all, k_all = W.all_latents(wl) if latents is None else latents
    pos_tok = _t(layout.positions, torch.int32, device)
    slots = _t(layout.slots, torch.int32, device)
    # write in chunks to bound the temporary device copies
    step = 1 << 18
    for s0 in range(0, c_all.shape[0], step):
        s1 = min(s0 + step, c_all.shape[0])
        _lib.cache_write(cache, _t(c_all[s0:s1], dt, device), _t(k_all[s0:s1], dt, device), pos_tok[s0:s1],
                         slots[s0:s1], rope=rope)
    host = {}
    if keep_host:
        host = dict(q_c=q_c, q_r=q_r, w_uk=w_uk, w_uv=w_uv, c_kv=c_all, k_r=k_all, offsets=layout.offsets)
    return DeviceDecode(
        wl=wl, layout=layout, cache=cache, q_c=_t(q_c, dt, device), q_r=_t(q_r, dt, device),
        pos=_t(wl.lens - 1, torch.int32, device), w_uk=_t(w_uk, dt, device), w_uv=_t(w_uv, dt, device),
        block_table=_t(np.where(layout.block_table < 0, 0, layout.block_table), torch.int32, device),
        seq_lens=_t(wl.lens, torch.int32, device), host=host)


def multi_query_inputs(dd: DeviceDecode, q_len: int):
    """Multi-token queries of a decode workload on the device of `dd`:
    q_c [B*q_len,H,128], q_r [B*q_len,H,64] (token-major within a sequence)
    and their positions L_b - q_len + t, plus the host copies."""
    wl = dd.wl
    dt = dd.q_c.dtype
    dev = dd.q_c.device
    q_c, q_r = W.multi_queries(wl, q_len)
    pos = (np.asarray(wl.lens)[:, None] - q_len + np.arange(q_len)[None, :]).reshape(-1)
    return (_t(q_c.reshape(-1, wl.H, q_c.shape[-1]), dt, dev), _t(q_r.reshape(-1, wl.H, q_r.shape[-1]), dt, dev),
            _t(pos, torch.int32, dev), q_c, q_r)
