"""ctypes binding of libmla (include/mla.h): argument marshalling only.

Every entry point takes torch tensors that already live on the GPU, checks
their dtype, shape and contiguity, and passes raw device pointers plus the
current HIP stream to the C library.  Nothing here computes any part of the
attention; if libmla.so is missing the calls raise.
"""

from __future__ import annotations

import ctypes
import math
import os
import re
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmla.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
HEADER = os.path.join(INCLUDE, "mla.h")

MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_WORKSPACE, MLA_ERR_HIP = range(5)
MLA_F32, MLA_BF16, MLA_FP8_E4M3 = 0, 1, 2
D_C, D_R, D_NOPE, D_V, ROW, PAGE = 512, 64, 128, 128, 576, 64

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_f32 = ctypes.c_float


class MlaCache(ctypes.Structure):
    _fields_ = [("dtype", _i32), ("num_pages", _i32), ("page_size", _i32), ("reserved", _i32),
                ("rows", _vp), ("ckv_fp8", _vp), ("ckv_scale", _vp), ("kr", _vp)]


class MlaRope(ctypes.Structure):
    """mla_rope: rotary frequencies of the decoupled RoPE path (plain or YaRN)."""
    _fields_ = [("base", _f32), ("yarn_factor", _f32), ("yarn_alpha", _f32), ("yarn_beta", _f32),
                ("orig_len", _i32)]


def yarn_rope(factor: float = 40.0, alpha: float = 1.0, beta: float = 32.0, orig_len: int = 4096,
              base: float = 10000.0) -> MlaRope:
    """YaRN frequencies with the long-context configuration (s = 40, alpha = 1, beta = 32, 4K original)."""
    return MlaRope(base, factor, alpha, beta, orig_len)


def yarn_attention_factor(factor: float = 40.0) -> float:
    """0.1 ln s + 1: multiply the softmax scale by it when the keys use YaRN (mla_yarn_attention_factor)."""
    return float(lib().mla_yarn_attention_factor(float(factor)))


class MLAError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)}")


_LIB = None


def lib() -> ctypes.CDLL:
    """Load libmla.so (built in-tree by mla_latent_kv_30_amd.build)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m mla_latent_kv_30_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    L.mla_status_string.restype = ctypes.c_char_p
    L.mla_status_string.argtypes = [_i32]
    L.mla_absorb_q.restype = _i32
    L.mla_absorb_q.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _f32, _vp]
    L.mla_cache_write.restype = _i32
    L.mla_cache_write.argtypes = [_vp, _vp, _vp, _vp, _i32, _i32, ctypes.POINTER(MlaCache), _f32, _vp]
    L.mla_decode_workspace_size.restype = ctypes.c_size_t
    L.mla_decode_workspace_size.argtypes = [_i32, _i32, _i32]
    L.mla_decode.restype = _i32
    L.mla_decode.argtypes = [_vp, ctypes.POINTER(MlaCache), _vp, _vp, _i32, _i32, _i32, _f32, _i32, _vp,
                             ctypes.c_size_t, _vp, _vp, _vp]
    L.mla_decode_partial.restype = _i32
    L.mla_decode_partial.argtypes = list(L.mla_decode.argtypes)
    L.mla_decode_merge.restype = _i32
    L.mla_decode_merge.argtypes = [_vp, _i32, _i32, _i32, _vp, ctypes.c_size_t, _vp, _vp, _vp]
    L.mla_absorb_q_rope.restype = _i32
    L.mla_absorb_q_rope.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, ctypes.POINTER(MlaRope), _vp]
    L.mla_cache_write_rope.restype = _i32
    L.mla_cache_write_rope.argtypes = [_vp, _vp, _vp, _vp, _i32, _i32, ctypes.POINTER(MlaCache),
                                       ctypes.POINTER(MlaRope), _vp]
    L.mla_prefill_causal_rope.restype = _i32
    L.mla_prefill_causal_rope.argtypes = [_vp, _vp, _vp, _i32, ctypes.POINTER(MlaCache), _vp, _i32, _i32, _f32,
                                          ctypes.POINTER(MlaRope), _vp, _vp, _vp]
    L.mla_yarn_attention_factor.restype = ctypes.c_double
    L.mla_yarn_attention_factor.argtypes = [ctypes.c_double]
    L.mla_decode_multi.restype = _i32
    L.mla_decode_multi.argtypes = [_vp, ctypes.POINTER(MlaCache), _vp, _vp, _i32, _i32, _i32, _i32, _f32, _i32, _vp,
                                   ctypes.c_size_t, _vp, _vp, _vp]
    L.mla_decode_noalloc.restype = _i32
    L.mla_decode_noalloc.argtypes = [_vp, ctypes.POINTER(MlaCache), _vp, _vp, _i32, _i32, _i32, _f32, _i32, _vp, _vp,
                                     _vp]
    L.mla_validate_decode_inputs.restype = _i32
    L.mla_validate_decode_inputs.argtypes = [_vp, _vp, _i32, _i32, _i32, _i32]
    L.mla_set_debug.restype = None
    L.mla_set_debug.argtypes = [_i32]
    L.mla_decode_multi_upproj.restype = _i32
    L.mla_decode_multi_upproj.argtypes = [_vp, ctypes.POINTER(MlaCache), _vp, _vp, _i32, _i32, _i32, _i32, _f32,
                                          _i32, _vp, ctypes.c_size_t, _vp, _vp, _vp, _i32, _vp, _i32, _vp]
    L.mla_decode_upproj.restype = _i32
    L.mla_decode_upproj.argtypes = [_vp, ctypes.POINTER(MlaCache), _vp, _vp, _i32, _i32, _i32, _f32, _i32, _vp,
                                    ctypes.c_size_t, _vp, _vp, _vp, _i32, _vp, _i32, _vp]
    L.mla_decode_upproj_workspace_size.restype = ctypes.c_size_t
    L.mla_decode_upproj_workspace_size.argtypes = [_i32, _i32, _i32]
    L.mla_decode_upproj_launches.restype = _i32
    L.mla_decode_upproj_launches.argtypes = [_i32, _i32, _i32, _i32, _i32]
    L.mla_decode_merge_upproj.restype = _i32
    L.mla_decode_merge_upproj.argtypes = [_vp, _i32, _i32, _i32, _vp, ctypes.c_size_t, _vp, _vp, _vp, _i32, _vp,
                                          _i32, _vp]
    L.mla_prefill_causal.restype = _i32
    L.mla_prefill_causal.argtypes = [_vp, _vp, _vp, _i32, ctypes.POINTER(MlaCache), _vp, _i32, _i32, _f32, _f32,
                                     _vp, _vp, _vp]
    L.mla_upproj_v.restype = _i32
    L.mla_upproj_v.argtypes = [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp]
    _sz = ctypes.c_size_t
    L.mla_linear_workspace_size.restype = _sz
    L.mla_linear_workspace_size.argtypes = [_i32, _i32, _i32]
    L.mla_linear.restype = _i32
    L.mla_linear.argtypes = [_vp, _vp, _i32, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _vp, _sz, _vp]
    L.mla_kv_append_workspace_size.restype = _sz
    L.mla_kv_append_workspace_size.argtypes = [_i32, _i32, _i32]
    L.mla_kv_append.restype = _i32
    L.mla_kv_append.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _i32, ctypes.POINTER(MlaCache),
                                ctypes.POINTER(MlaRope), _vp, _sz, _vp]
    L.mla_q_project_workspace_size.restype = _sz
    L.mla_q_project_workspace_size.argtypes = [_i32, _i32, _i32, _i32]
    L.mla_q_project.restype = _i32
    L.mla_q_project.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _sz, _vp]
    L.mla_qkv_project_workspace_size.restype = _sz
    L.mla_qkv_project_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32]
    L.mla_qkv_project.restype = _i32
    L.mla_qkv_project.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                  ctypes.POINTER(MlaCache), ctypes.POINTER(MlaRope), _vp, _vp, _i32, _vp, _sz, _vp]
    L.mla_output_proj.restype = _i32
    L.mla_output_proj.argtypes = [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _sz, _vp]
    L.mla_fold_wuv_wo.restype = _i32
    L.mla_fold_wuv_wo.argtypes = [_vp, _vp, _vp, _i32, _i32, _vp]
    # mla_ceilings.h
    _dp = ctypes.POINTER(ctypes.c_double)
    L.mla_ceiling_sink_floats.restype = _i32
    L.mla_ceiling_sink_floats.argtypes = []
    L.mla_ceiling_hbm_read.restype = _i32
    L.mla_ceiling_hbm_read.argtypes = [_vp, _sz, _vp, _dp, _vp]
    L.mla_ceiling_mfma_bf16.restype = _i32
    L.mla_ceiling_mfma_bf16.argtypes = [_i32, _i32, _vp, _dp, _vp]
    L.mla_ceiling_lds_read.restype = _i32
    L.mla_ceiling_lds_read.argtypes = [_i32, _i32, _vp, _dp, _vp]
    _LIB = L
    return L


def declared_symbols() -> list:
    """Names of the functions the headers under include/ declare."""
    names = set()
    for f in sorted(os.listdir(INCLUDE)):
        if f.endswith(".h"):
            txt = open(os.path.join(INCLUDE, f)).read()
            names |= set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(mla_\w+)\s*\(", txt, flags=re.M))
    return sorted(names)


def status_string(status: int) -> str:
    return lib().mla_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status != MLA_OK:
        raise MLAError(status, what)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _dt_code(dtype) -> int:
    if dtype == torch.float32:
        return MLA_F32
    if dtype == torch.bfloat16:
        return MLA_BF16
    raise TypeError(f"unsupported dtype {dtype}")


def default_softmax_scale() -> float:
    return 1.0 / math.sqrt(D_NOPE + D_R)


class PagedCache:
    """A pool of 64-token pages holding each cached token's (c_KV, rotated k_R).

    dtype torch.float32 / torch.bfloat16: rows [num_pages, 64, 576].
    dtype "fp8": ckv [num_pages, 64, 512] uint8 (E4M3 codes),
    scale [num_pages, 64, 4] float32, kr [num_pages, 64, 64] bfloat16.
    `fill` initialises the storage (e.g. float('nan') to poison unused slots).
    """

    def __init__(self, num_pages: int, dtype, device="cuda", fill: Optional[float] = None):
        self.num_pages = int(num_pages)
        self.device = torch.device(device)
        self.rows = self.ckv = self.scale = self.kr = None
        if dtype == "fp8":
            self.code = MLA_FP8_E4M3
            self.ckv = torch.empty((num_pages, PAGE, D_C), dtype=torch.uint8, device=device)
            self.scale = torch.empty((num_pages, PAGE, 4), dtype=torch.float32, device=device)
            self.kr = torch.empty((num_pages, PAGE, D_R), dtype=torch.bfloat16, device=device)
            if fill is not None:
                self.ckv.fill_(0x7F if math.isnan(fill) else 0)  # 0x7F is an E4M3 NaN
                self.scale.fill_(fill)
                self.kr.fill_(fill)
        else:
            self.code = _dt_code(dtype)
            self.rows = torch.empty((num_pages, PAGE, ROW), dtype=dtype, device=device)
            if fill is not None:
                self.rows.fill_(fill)

    @property
    def is_fp8(self) -> bool:
        return self.code == MLA_FP8_E4M3

    @property
    def input_dtype(self):
        return torch.float32 if self.code == MLA_F32 else torch.bfloat16

    def descriptor(self) -> MlaCache:
        return MlaCache(self.code, self.num_pages, PAGE, 0, _ptr(self.rows), _ptr(self.ckv), _ptr(self.scale),
                        _ptr(self.kr))

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.rows, self.ckv, self.scale, self.kr) if t is not None)


def absorb_q(q_c: torch.Tensor, q_r: torch.Tensor, pos: torch.Tensor, w_uk: torch.Tensor,
             out: Optional[torch.Tensor] = None, rope_base: float = 10000.0,
             rope: Optional[MlaRope] = None) -> torch.Tensor:
    """q_abs[N,H,576] = [W_UK^T q_C | RoPE_pos(q_R)] (mla_absorb_q; mla_absorb_q_rope if `rope` is given)."""
    N, H = q_c.shape[0], q_c.shape[1]
    dt = q_c.dtype
    _need(q_c, "q_c", dt, (N, H, D_NOPE))
    _need(q_r, "q_r", dt, (N, H, D_R))
    _need(pos, "pos", torch.int32, (N,))
    _need(w_uk, "w_uk", dt, (H, D_NOPE, D_C))
    if out is None:
        out = torch.empty((N, H, ROW), dtype=dt, device=q_c.device)
    _need(out, "out", dt, (N, H, ROW))
    if rope is not None:
        _check(lib().mla_absorb_q_rope(_ptr(q_c), _ptr(q_r), _ptr(pos), _ptr(w_uk), _ptr(out), N, H, _dt_code(dt),
                                       ctypes.byref(rope), _stream(q_c.device)), "mla_absorb_q_rope")
        return out
    _check(lib().mla_absorb_q(_ptr(q_c), _ptr(q_r), _ptr(pos), _ptr(w_uk), _ptr(out), N, H, _dt_code(dt),
                              float(rope_base), _stream(q_c.device)), "mla_absorb_q")
    return out


def cache_write(cache: PagedCache, c_kv: torch.Tensor, k_r: torch.Tensor, pos: torch.Tensor, slot: torch.Tensor,
                rope_base: float = 10000.0, rope: Optional[MlaRope] = None) -> None:
    """Store T tokens' (c_KV, RoPE_pos(k_R)) at pool rows `slot` (mla_cache_write)."""
    T = c_kv.shape[0]
    dt = cache.input_dtype
    _need(c_kv, "c_kv", dt, (T, D_C))
    _need(k_r, "k_r", dt, (T, D_R))
    _need(pos, "pos", torch.int32, (T,))
    _need(slot, "slot", torch.int32, (T,))
    desc = cache.descriptor()
    if rope is not None:
        _check(lib().mla_cache_write_rope(_ptr(c_kv), _ptr(k_r), _ptr(pos), _ptr(slot), T, _dt_code(dt),
                                          ctypes.byref(desc), ctypes.byref(rope), _stream(c_kv.device)),
               "mla_cache_write_rope")
        return
    _check(lib().mla_cache_write(_ptr(c_kv), _ptr(k_r), _ptr(pos), _ptr(slot), T, _dt_code(dt), ctypes.byref(desc),
                                 float(rope_base), _stream(c_kv.device)), "mla_cache_write")


def decode_workspace_size(B: int, H: int, num_splits: int = 0) -> int:
    return int(lib().mla_decode_workspace_size(int(B), int(H), int(num_splits)))


def decode_workspace(B: int, H: int, num_splits: int = 0, device="cuda") -> Optional[torch.Tensor]:
    """A workspace for mla_decode / mla_decode_partial (None when none is needed)."""
    need = decode_workspace_size(B, H, num_splits)
    return torch.empty(need, dtype=torch.uint8, device=device) if need > 0 else None


def _decode_call(fn_name, q_abs, cache, block_table, seq_lens, softmax_scale, num_splits, workspace, z, lse,
                 want_lse):
    B, H = q_abs.shape[0], q_abs.shape[1]
    _need(q_abs, "q_abs", cache.input_dtype, (B, H, ROW))
    _need(block_table, "block_table", torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_pages]")
    _need(seq_lens, "seq_lens", torch.int32, (B,))
    dev = q_abs.device
    if z is None:
        z = torch.empty((B, H, D_C), dtype=torch.float32, device=dev)
    _need(z, "z", torch.float32, (B, H, D_C))
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, H))
    if workspace is None:
        workspace = decode_workspace(B, H, num_splits, dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    scale = default_softmax_scale() if softmax_scale is None else float(softmax_scale)
    desc = cache.descriptor()
    fn = getattr(lib(), fn_name)
    _check(fn(_ptr(q_abs), ctypes.byref(desc), _ptr(block_table), _ptr(seq_lens), B, H, block_table.shape[1], scale,
              int(num_splits), _ptr(workspace), ws_bytes, _ptr(z), _ptr(lse), _stream(dev)), fn_name)
    return z, lse, workspace


def decode(q_abs: torch.Tensor, cache: PagedCache, block_table: torch.Tensor, seq_lens: torch.Tensor,
           softmax_scale: Optional[float] = None, num_splits: int = 0, workspace: Optional[torch.Tensor] = None,
           z: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None, want_lse: bool = True):
    """z[B,H,512], lse[B,H] of one new token per sequence (mla_decode)."""
    z, lse, _ = _decode_call("mla_decode", q_abs, cache, block_table, seq_lens, softmax_scale, num_splits,
                             workspace, z, lse, want_lse)
    return z, lse


def decode_partial(q_abs: torch.Tensor, cache: PagedCache, block_table: torch.Tensor, seq_lens: torch.Tensor,
                   workspace: Optional[torch.Tensor], z: torch.Tensor, lse: Optional[torch.Tensor] = None,
                   softmax_scale: Optional[float] = None, num_splits: int = 0):
    """The split pass of mla_decode (mla_decode_partial); returns the workspace."""
    _, _, ws = _decode_call("mla_decode_partial", q_abs, cache, block_table, seq_lens, softmax_scale, num_splits,
                            workspace, z, lse, lse is not None)
    return ws


def decode_merge(seq_lens: torch.Tensor, H: int, workspace: Optional[torch.Tensor], z: torch.Tensor,
                 lse: Optional[torch.Tensor] = None, num_splits: int = 0) -> None:
    """The merge pass of mla_decode (mla_decode_merge)."""
    B = seq_lens.shape[0]
    _need(seq_lens, "seq_lens", torch.int32, (B,))
    _need(z, "z", torch.float32, (B, H, D_C))
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().mla_decode_merge(_ptr(seq_lens), B, int(H), int(num_splits), _ptr(workspace), ws_bytes, _ptr(z),
                                  _ptr(lse), _stream(z.device)), "mla_decode_merge")


NOALLOC_SCRATCH_BYTES = 96 << 20  # MLA_DECODE_NOALLOC_SCRATCH_BYTES


def decode_noalloc(q_abs: torch.Tensor, cache: PagedCache, block_table: torch.Tensor, seq_lens: torch.Tensor,
                   z: torch.Tensor, lse: Optional[torch.Tensor] = None, softmax_scale: Optional[float] = None,
                   num_splits: int = 0) -> None:
    """mla_decode_noalloc: decode() into caller-provided z (and lse) with the split partials in the
    library's own device array; nothing is allocated on either side of the call."""
    B, H = q_abs.shape[0], q_abs.shape[1]
    _need(q_abs, "q_abs", cache.input_dtype, (B, H, ROW))
    _need(block_table, "block_table", torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_pages]")
    _need(seq_lens, "seq_lens", torch.int32, (B,))
    _need(z, "z", torch.float32, (B, H, D_C))
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, H))
    scale = default_softmax_scale() if softmax_scale is None else float(softmax_scale)
    desc = cache.descriptor()
    _check(lib().mla_decode_noalloc(_ptr(q_abs), ctypes.byref(desc), _ptr(block_table), _ptr(seq_lens), B, H,
                                    block_table.shape[1], scale, int(num_splits), _ptr(z), _ptr(lse),
                                    _stream(q_abs.device)), "mla_decode_noalloc")


def decode_multi(q_abs: torch.Tensor, cache: PagedCache, block_table: torch.Tensor, seq_lens: torch.Tensor,
                 softmax_scale: Optional[float] = None, num_splits: int = 0, workspace: Optional[torch.Tensor] = None,
                 z: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None, want_lse: bool = True):
    """z[B,q_len,H,512], lse[B,q_len,H] of q_len new tokens per sequence (mla_decode_multi)."""
    B, q_len, H = q_abs.shape[0], q_abs.shape[1], q_abs.shape[2]
    _need(q_abs, "q_abs", cache.input_dtype, (B, q_len, H, ROW))
    _need(block_table, "block_table", torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_pages]")
    _need(seq_lens, "seq_lens", torch.int32, (B,))
    dev = q_abs.device
    if z is None:
        z = torch.empty((B, q_len, H, D_C), dtype=torch.float32, device=dev)
    _need(z, "z", torch.float32, (B, q_len, H, D_C))
    if lse is None and want_lse:
        lse = torch.empty((B, q_len, H), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, q_len, H))
    if workspace is None:
        workspace = decode_workspace(B, q_len * H, num_splits, dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    scale = default_softmax_scale() if softmax_scale is None else float(softmax_scale)
    desc = cache.descriptor()
    _check(lib().mla_decode_multi(_ptr(q_abs), ctypes.byref(desc), _ptr(block_table), _ptr(seq_lens), B, q_len, H,
                                  block_table.shape[1], scale, int(num_splits), _ptr(workspace), ws_bytes, _ptr(z),
                                  _ptr(lse), _stream(dev)), "mla_decode_multi")
    return z, lse


def decode_multi_upproj(q_abs: torch.Tensor, cache: PagedCache, block_table: torch.Tensor, seq_lens: torch.Tensor,
                        w_uv: torch.Tensor, softmax_scale: Optional[float] = None, num_splits: int = 0,
                        workspace: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
                        lse: Optional[torch.Tensor] = None, out_dtype=torch.float32,
                        out: Optional[torch.Tensor] = None):
    """(o[B,q_len,H,128], z, lse) of q_len new tokens per sequence (mla_decode_multi_upproj)."""
    B, q_len, H = q_abs.shape[0], q_abs.shape[1], q_abs.shape[2]
    _need(q_abs, "q_abs", cache.input_dtype, (B, q_len, H, ROW))
    _need(block_table, "block_table", torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_pages]")
    _need(seq_lens, "seq_lens", torch.int32, (B,))
    _need(w_uv, "w_uv", None, (H, D_V, D_C))
    dev = q_abs.device
    if z is None:
        z = torch.empty((B, q_len, H, D_C), dtype=torch.float32, device=dev)
    _need(z, "z", torch.float32, (B, q_len, H, D_C))
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, q_len, H))
    if out is None:
        out = torch.empty((B, q_len, H, D_V), dtype=out_dtype, device=dev)
    _need(out, "out", out_dtype, (B, q_len, H, D_V))
    if workspace is None:
        workspace = decode_workspace(B, q_len * H, num_splits, dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    scale = default_softmax_scale() if softmax_scale is None else float(softmax_scale)
    desc = cache.descriptor()
    _check(lib().mla_decode_multi_upproj(_ptr(q_abs), ctypes.byref(desc), _ptr(block_table), _ptr(seq_lens), B,
                                         q_len, H, block_table.shape[1], scale, int(num_splits), _ptr(workspace),
                                         ws_bytes, _ptr(z), _ptr(lse), _ptr(w_uv), _dt_code(w_uv.dtype), _ptr(out),
                                         _dt_code(out_dtype), _stream(dev)), "mla_decode_multi_upproj")
    return out, z, lse


def decode_merge_upproj(seq_lens: torch.Tensor, H: int, workspace: Optional[torch.Tensor], z: torch.Tensor,
                        w_uv: torch.Tensor, lse: Optional[torch.Tensor] = None, num_splits: int = 0,
                        out_dtype=torch.float32, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The merge pass followed by the value up-projection (mla_decode_merge_upproj); returns o[B,H,128]."""
    B = seq_lens.shape[0]
    _need(seq_lens, "seq_lens", torch.int32, (B,))
    _need(z, "z", torch.float32, (B, H, D_C))
    _need(w_uv, "w_uv", None, (H, D_V, D_C))
    if out is None:
        out = torch.empty((B, H, D_V), dtype=out_dtype, device=z.device)
    _need(out, "out", out_dtype, (B, H, D_V))
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().mla_decode_merge_upproj(_ptr(seq_lens), B, int(H), int(num_splits), _ptr(workspace), ws_bytes,
                                         _ptr(z), _ptr(lse), _ptr(w_uv), _dt_code(w_uv.dtype), _ptr(out),
                                         _dt_code(out_dtype), _stream(z.device)), "mla_decode_merge_upproj")
    return out


def decode_upproj_workspace(B: int, H: int, num_splits: int = 0, device="cuda") -> torch.Tensor:
    """A workspace for mla_decode_upproj: zeroed, as its counters must be before the first call."""
    need = int(lib().mla_decode_upproj_workspace_size(int(B), int(H), int(num_splits)))
    return torch.zeros(need, dtype=torch.uint8, device=device)


def decode_upproj_launches(B: int, H: int, num_splits: int, cache_dtype: int, w_dtype=torch.bfloat16) -> int:
    """Launches mla_decode_upproj makes on the current device (1: the one-launch form)."""
    return int(lib().mla_decode_upproj_launches(int(B), int(H), int(num_splits), int(cache_dtype),
                                                _dt_code(w_dtype)))


def decode_upproj(q_abs: torch.Tensor, cache: PagedCache, block_table: torch.Tensor, seq_lens: torch.Tensor,
                  w_uv: torch.Tensor, softmax_scale: Optional[float] = None, num_splits: int = 0,
                  workspace: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
                  lse: Optional[torch.Tensor] = None, out_dtype=torch.float32, out: Optional[torch.Tensor] = None):
    """(o[B,H,128], z, lse) of one new token per sequence (mla_decode_upproj: decode, merge and W^UV,
    in one launch where the library can)."""
    B, H = q_abs.shape[0], q_abs.shape[1]
    _need(q_abs, "q_abs", cache.input_dtype, (B, H, ROW))
    _need(block_table, "block_table", torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_pages]")
    _need(seq_lens, "seq_lens", torch.int32, (B,))
    _need(w_uv, "w_uv", None, (H, D_V, D_C))
    dev = q_abs.device
    if z is None:
        z = torch.empty((B, H, D_C), dtype=torch.float32, device=dev)
    _need(z, "z", torch.float32, (B, H, D_C))
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, H))
    if out is None:
        out = torch.empty((B, H, D_V), dtype=out_dtype, device=dev)
    _need(out, "out", out_dtype, (B, H, D_V))
    if workspace is None:
        workspace = decode_upproj_workspace(B, H, num_splits, dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    scale = default_softmax_scale() if softmax_scale is None else float(softmax_scale)
    desc = cache.descriptor()
    _check(lib().mla_decode_upproj(_ptr(q_abs), ctypes.byref(desc), _ptr(block_table), _ptr(seq_lens), B, H,
                                   block_table.shape[1], scale, int(num_splits), _ptr(workspace), ws_bytes, _ptr(z),
                                   _ptr(lse), _ptr(w_uv), _dt_code(w_uv.dtype), _ptr(out), _dt_code(out_dtype),
                                   _stream(dev)), "mla_decode_upproj")
    return out, z, lse


def prefill_causal(q_abs: torch.Tensor, c_kv: torch.Tensor, k_r: torch.Tensor, cache: PagedCache,
                   block_table_row: torch.Tensor, pos0: int = 0, softmax_scale: Optional[float] = None,
                   rope_base: float = 10000.0, z: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                   want_lse: bool = True, rope: Optional[MlaRope] = None):
    """Append T tokens at positions pos0.. and attend causally (mla_prefill_causal)."""
    T, H = q_abs.shape[0], q_abs.shape[1]
    dt = cache.input_dtype
    _need(q_abs, "q_abs", dt, (T, H, ROW))
    _need(c_kv, "c_kv", dt, (T, D_C))
    _need(k_r, "k_r", dt, (T, D_R))
    _need(block_table_row, "block_table_row", torch.int32)
    if block_table_row.numel() < (pos0 + T + PAGE - 1) // PAGE:
        raise ValueError("block_table_row too short for pos0 + T tokens")
    dev = q_abs.device
    if z is None:
        z = torch.empty((T, H, D_C), dtype=torch.float32, device=dev)
    _need(z, "z", torch.float32, (T, H, D_C))
    if lse is None and want_lse:
        lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    scale = default_softmax_scale() if softmax_scale is None else float(softmax_scale)
    desc = cache.descriptor()
    if rope is not None:
        _check(lib().mla_prefill_causal_rope(_ptr(q_abs), _ptr(c_kv), _ptr(k_r), int(pos0), ctypes.byref(desc),
                                             _ptr(block_table_row), T, H, scale, ctypes.byref(rope), _ptr(z),
                                             _ptr(lse), _stream(dev)), "mla_prefill_causal_rope")
        return z, lse
    _check(lib().mla_prefill_causal(_ptr(q_abs), _ptr(c_kv), _ptr(k_r), int(pos0), ctypes.byref(desc),
                                    _ptr(block_table_row), T, H, scale, float(rope_base), _ptr(z), _ptr(lse),
                                    _stream(dev)), "mla_prefill_causal")
    return z, lse


def upproj_v(z: torch.Tensor, w_uv: torch.Tensor, out_dtype=torch.float32,
             out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """o[N,H,128] = W_UV z per head (mla_upproj_v)."""
    N, H = z.shape[0], z.shape[1]
    _need(z, "z", torch.float32, (N, H, D_C))
    _need(w_uv, "w_uv", None, (H, D_V, D_C))
    if out is None:
        out = torch.empty((N, H, D_V), dtype=out_dtype, device=z.device)
    _need(out, "out", out_dtype, (N, H, D_V))
    _check(lib().mla_upproj_v(_ptr(z), _ptr(w_uv), _ptr(out), N, H, _dt_code(w_uv.dtype), _dt_code(out_dtype),
                              _stream(z.device)), "mla_upproj_v")
    return out


# ---------------------------------------------------------------------------
# Projections around the attention
# ---------------------------------------------------------------------------

def _workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    return torch.empty(int(nbytes), dtype=torch.uint8, device=device) if nbytes > 0 else None


def _ws_args(ws: Optional[torch.Tensor]):
    return (_ptr(ws), 0 if ws is None else ws.numel())


def linear_workspace_size(N: int, M: int, K: int) -> int:
    return int(lib().mla_linear_workspace_size(int(N), int(M), int(K)))


def linear(x: torch.Tensor, w0: torch.Tensor, w1: Optional[torch.Tensor] = None, out_dtype=torch.bfloat16,
           workspace: Optional[torch.Tensor] = None):
    """Y = X W^T with W = [w0; w1] (mla_linear).  Returns y0 [N, M0], or
    (y0, y1) when w1 is given."""
    N, K = x.shape
    M0 = w0.shape[0]
    M1 = 0 if w1 is None else w1.shape[0]
    _need(x, "x", torch.bfloat16, (N, K))
    _need(w0, "w0", torch.bfloat16, (M0, K))
    if w1 is not None:
        _need(w1, "w1", torch.bfloat16, (M1, K))
    y0 = torch.empty((N, M0), dtype=out_dtype, device=x.device)
    y1 = torch.empty((N, M1), dtype=out_dtype, device=x.device) if M1 else None
    if workspace is None:
        workspace = _workspace(linear_workspace_size(N, M0 + M1, K), x.device)
    _check(lib().mla_linear(_ptr(x), _ptr(w0), M0, _ptr(w1), M1, _ptr(y0), _ptr(y1), N, K, _dt_code(out_dtype),
                            *_ws_args(workspace), _stream(x.device)), "mla_linear")
    return y0 if w1 is None else (y0, y1)


def kv_append_workspace_size(T: int, d: int, cache_dtype: int) -> int:
    return int(lib().mla_kv_append_workspace_size(int(T), int(d), int(cache_dtype)))


def kv_append(cache: PagedCache, h: torch.Tensor, w_dkv: torch.Tensor, w_kr: torch.Tensor, pos: torch.Tensor,
              slot: torch.Tensor, rope: Optional[MlaRope] = None, workspace: Optional[torch.Tensor] = None) -> None:
    """c^KV = W^DKV h and RoPE_pos(W^KR h) of T tokens into the cache (mla_kv_append)."""
    T, d = h.shape
    _need(h, "h", torch.bfloat16, (T, d))
    _need(w_dkv, "w_dkv", torch.bfloat16, (D_C, d))
    _need(w_kr, "w_kr", torch.bfloat16, (D_R, d))
    _need(pos, "pos", torch.int32, (T,))
    _need(slot, "slot", torch.int32, (T,))
    desc = cache.descriptor()
    if workspace is None:
        workspace = _workspace(kv_append_workspace_size(T, d, desc.dtype), h.device)
    _check(lib().mla_kv_append(_ptr(h), _ptr(w_dkv), _ptr(w_kr), _ptr(pos), _ptr(slot), T, d, ctypes.byref(desc),
                               None if rope is None else ctypes.byref(rope), *_ws_args(workspace),
                               _stream(h.device)), "mla_kv_append")


def q_project_workspace_size(T: int, d: int, dcq: int, H: int) -> int:
    return int(lib().mla_q_project_workspace_size(int(T), int(d), int(dcq), int(H)))


def q_project(h: torch.Tensor, w_dq: torch.Tensor, w_uq: torch.Tensor, w_qr: torch.Tensor, H: int,
              out_dtype=torch.bfloat16, workspace: Optional[torch.Tensor] = None,
              q_c: Optional[torch.Tensor] = None, q_r: Optional[torch.Tensor] = None):
    """(q_c [T,H,128], q_r [T,H,64] before rotation) from hidden states (mla_q_project)."""
    T, d = h.shape
    dcq = w_dq.shape[0]
    _need(h, "h", torch.bfloat16, (T, d))
    _need(w_dq, "w_dq", torch.bfloat16, (dcq, d))
    _need(w_uq, "w_uq", torch.bfloat16, (H * D_NOPE, dcq))
    _need(w_qr, "w_qr", torch.bfloat16, (H * D_R, dcq))
    if q_c is None:
        q_c = torch.empty((T, H, D_NOPE), dtype=out_dtype, device=h.device)
    if q_r is None:
        q_r = torch.empty((T, H, D_R), dtype=out_dtype, device=h.device)
    _need(q_c, "q_c", out_dtype, (T, H, D_NOPE))
    _need(q_r, "q_r", out_dtype, (T, H, D_R))
    if workspace is None:
        workspace = _workspace(q_project_workspace_size(T, d, dcq, H), h.device)
    _check(lib().mla_q_project(_ptr(h), _ptr(w_dq), _ptr(w_uq), _ptr(w_qr), _ptr(q_c), _ptr(q_r), T, d, dcq, H,
                               _dt_code(out_dtype), *_ws_args(workspace), _stream(h.device)), "mla_q_project")
    return q_c, q_r


def qkv_project_workspace_size(T: int, d: int, dcq: int, H: int, cache_dtype: int) -> int:
    return int(lib().mla_qkv_project_workspace_size(int(T), int(d), int(dcq), int(H), int(cache_dtype)))


def qkv_project(cache: PagedCache, h: torch.Tensor, w_dq: torch.Tensor, w_dkv: torch.Tensor, w_kr: torch.Tensor,
                w_uq: torch.Tensor, w_qr: torch.Tensor, pos: torch.Tensor, slot: torch.Tensor, H: int,
                out_dtype=torch.bfloat16, rope: Optional[MlaRope] = None, workspace: Optional[torch.Tensor] = None,
                q_c: Optional[torch.Tensor] = None, q_r: Optional[torch.Tensor] = None):
    """Cache append and query path of T tokens from h in one call
    (mla_qkv_project); returns (q_c [T,H,128], q_r [T,H,64] before rotation)."""
    T, d = h.shape
    dcq = w_dq.shape[0]
    _need(h, "h", torch.bfloat16, (T, d))
    _need(w_dq, "w_dq", torch.bfloat16, (dcq, d))
    _need(w_dkv, "w_dkv", torch.bfloat16, (D_C, d))
    _need(w_kr, "w_kr", torch.bfloat16, (D_R, d))
    _need(w_uq, "w_uq", torch.bfloat16, (H * D_NOPE, dcq))
    _need(w_qr, "w_qr", torch.bfloat16, (H * D_R, dcq))
    _need(pos, "pos", torch.int32, (T,))
    _need(slot, "slot", torch.int32, (T,))
    if q_c is None:
        q_c = torch.empty((T, H, D_NOPE), dtype=out_dtype, device=h.device)
    if q_r is None:
        q_r = torch.empty((T, H, D_R), dtype=out_dtype, device=h.device)
    _need(q_c, "q_c", out_dtype, (T, H, D_NOPE))
    _need(q_r, "q_r", out_dtype, (T, H, D_R))
    desc = cache.descriptor()
    if workspace is None:
        workspace = _workspace(qkv_project_workspace_size(T, d, dcq, H, desc.dtype), h.device)
    _check(lib().mla_qkv_project(_ptr(h), _ptr(w_dq), _ptr(w_dkv), _ptr(w_kr), _ptr(w_uq), _ptr(w_qr), _ptr(pos),
                                 _ptr(slot), T, d, dcq, H, ctypes.byref(desc),
                                 None if rope is None else ctypes.byref(rope), _ptr(q_c), _ptr(q_r),
                                 _dt_code(out_dtype), *_ws_args(workspace), _stream(h.device)), "mla_qkv_project")
    return q_c, q_r


def output_proj(x: torch.Tensor, w: torch.Tensor, out_dtype=torch.float32,
                workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """u = W x per token (mla_output_proj): x = o [N,H,128] with W^O, or the
    bf16 latent z [N,H,512] with the folded matrix."""
    N = x.shape[0]
    K = x[0].numel()
    d = w.shape[0]
    _need(x, "x", torch.bfloat16)
    _need(w, "w", torch.bfloat16, (d, K))
    if out is None:
        out = torch.empty((N, d), dtype=out_dtype, device=x.device)
    _need(out, "out", out_dtype, (N, d))
    if workspace is None:
        workspace = _workspace(linear_workspace_size(N, d, K), x.device)
    _check(lib().mla_output_proj(_ptr(x), _ptr(w), _ptr(out), N, K, d, _dt_code(out_dtype), *_ws_args(workspace),
                                 _stream(x.device)), "mla_output_proj")
    return out


def fold_wuv_wo(w_uv: torch.Tensor, w_o: torch.Tensor) -> torch.Tensor:
    """W^O blockdiag(W^UV) [d, H*512] bf16 (mla_fold_wuv_wo)."""
    H = w_uv.shape[0]
    d = w_o.shape[0]
    _need(w_uv, "w_uv", torch.bfloat16, (H, D_V, D_C))
    _need(w_o, "w_o", torch.bfloat16, (d, H * D_V))
    out = torch.empty((d, H * D_C), dtype=torch.bfloat16, device=w_o.device)
    _check(lib().mla_fold_wuv_wo(_ptr(w_uv), _ptr(w_o), _ptr(out), H, d, _stream(w_o.device)), "mla_fold_wuv_wo")
    return out


def set_debug(on: bool) -> None:
    """Debug mode of the decode entry points (mla_set_debug): lengths and
    block table are checked on the host before every launch."""
    lib().mla_set_debug(1 if on else 0)


def validate_decode_inputs(seq_lens, block_table, num_pages: int, q_len: int = 1) -> int:
    """mla_validate_decode_inputs on host arrays (numpy or CPU tensors);
    returns the status code."""
    import numpy as _np
    lens = _np.ascontiguousarray(_np.asarray(seq_lens, dtype=_np.int32))
    bt = None if block_table is None else _np.ascontiguousarray(_np.asarray(block_table, dtype=_np.int32))
    B = lens.shape[0]
    max_pages = 1 if bt is None else bt.shape[1]
    return int(lib().mla_validate_decode_inputs(lens.ctypes.data_as(_vp), None if bt is None else bt.ctypes.data_as(_vp),
                                                B, max_pages if bt is not None else max(1, int(lens.max() + 63) // 64),
                                                int(num_pages), int(q_len)))


# ---------------------------------------------------------------------------
# Measured ceilings (include/mla_ceilings.h)
# ---------------------------------------------------------------------------
CEILING_MFMA_32X32X16, CEILING_MFMA_16X16X32 = 0, 1
CEILING_LDS_B128, CEILING_LDS_TR_B64 = 0, 1


def ceiling_sink(device) -> torch.Tensor:
    return torch.empty(int(lib().mla_ceiling_sink_floats()), dtype=torch.float32, device=device)


def ceiling_hbm_read(buf: torch.Tensor, sink: torch.Tensor) -> float:
    """Launch the streaming read of `buf`; returns the bytes it reads."""
    work = ctypes.c_double(0.0)
    _check(lib().mla_ceiling_hbm_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), ctypes.byref(work),
                                      _stream(buf.device)), "mla_ceiling_hbm_read")
    return work.value


def ceiling_mfma_bf16(shape: int, iters: int, sink: torch.Tensor) -> float:
    """Launch the bf16 matrix-core loop; returns the FLOPs it issues."""
    work = ctypes.c_double(0.0)
    _check(lib().mla_ceiling_mfma_bf16(int(shape), int(iters), _ptr(sink), ctypes.byref(work), _stream(sink.device)),
           "mla_ceiling_mfma_bf16")
    return work.value


def ceiling_lds_read(kind: int, iters: int, sink: torch.Tensor) -> float:
    """Launch the LDS read loop; returns the bytes it reads from LDS."""
    work = ctypes.c_double(0.0)
    _check(lib().mla_ceiling_lds_read(int(kind), int(iters), _ptr(sink), ctypes.byref(work), _stream(sink.device)),
           "mla_ceiling_lds_read")
    return work.value
