"""Causal prefill attention for MI355X (gfx950): FP8 (e4m3, per-block scales) and BF16.

A thin binding over the C ABI of libzyfa.so (include/zyfa.h). Each function checks
that its tensors are contiguous device tensors of the right dtype and shape, then
passes their device pointers and the current HIP stream to the library; all
arithmetic runs in the library's HIP kernels. PyTorch provides device memory and
streams only. There is no fallback: if libzyfa.so is missing, calls raise.

Functions mirror the C entry points:

* ``quantize_fp8(x, scale_block, hadamard)`` -> (codes uint8, scales float32)
* ``attn_fwd_fp8(q, k, v, q_scale, k_scale, v_scale, scale_block, softmax_scale)``
  -> (o bfloat16, lse float32 or None)
* ``attn_fwd_bf16(q, k, v, softmax_scale)`` -> (o bfloat16, lse float32 or None)
* ``attn_fwd_fp8_range(..., q_offset, k_begin, k_end)`` / ``attn_fwd_bf16_range``: a chunk
  of query rows (row i at sequence position q_offset + i) against the key window
  [k_begin, k_end) -> (o, lse or None)
* ``attn_merge(o_parts, lse_parts)`` -> (o bfloat16, lse float32 or None): combine partial
  results over disjoint key sets
* ``attn_fwd_fp8_varlen(q, k, v, q_scale, k_scale, v_scale, scale_block, cu_seqlens, max_seqlen)``
  / ``attn_fwd_bf16_varlen``: a batch of sequences of different lengths packed as
  [H, T, D] -> (o [Hq, T, Dv], lse or None)
* ``attn_fwd_fp8_paged(q, k_cache, v_cache, q_scale, k_cache_scale, v_cache_scale, scale_block,
  cu_seqlens, kv_lens, block_table, max_seqlen)`` / ``attn_fwd_bf16_paged``: chunks of new
  tokens (packed as in the varlen calls) against their sequences' keys in a paged cache
  [pages, Hkv, page_size, D] -> (o [Hq, T, Dv], lse or None)
* ``attn_decode_fp8_paged(q, k_cache, v_cache, q_scale, k_cache_scale, v_cache_scale, scale_block,
  kv_lens, block_table, max_kv_len)`` / ``attn_decode_bf16_paged``: one new token per sequence
  (q [B, Hq, Dqk]) against its paged cache, keys split over workgroups and merged
  -> (o [B, Hq, Dv], lse or None)
"""

import math

import torch

from . import _lib
from ._lib import ZyfaError, load

__all__ = ["quantize_fp8", "attn_fwd_fp8", "attn_fwd_bf16", "attn_fwd_fp8_range", "attn_fwd_bf16_range", "attn_merge",
           "attn_fwd_fp8_varlen", "attn_fwd_bf16_varlen", "attn_fwd_fp8_paged", "attn_fwd_bf16_paged",
           "attn_decode_fp8_paged", "attn_decode_fp8_paged_noalloc", "attn_decode_bf16_paged", "decode_split_keys", "ZyfaError",
           "NOALLOC_SCRATCH_BYTES", "load", "abi_version"]


def abi_version() -> int:
    return load().zyfa_abi_version()


def _stream(*tensors):
    """The current stream of the one device that holds all of a call's tensors (None
    entries skipped): the library enqueues its kernels on that stream, and the
    allocation-free decode finds that device's scratch array through it."""
    devices = {t.device for t in tensors if t is not None}
    if len(devices) != 1:
        raise ValueError(f"a call's tensors must all be on one device, got {sorted(str(d) for d in devices)}")
    return torch.cuda.current_stream(devices.pop()).cuda_stream


def _dev(t: torch.Tensor, name: str, dtype, ndim: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got {t.dim()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def quantize_fp8(x: torch.Tensor, scale_block: int = 128, hadamard: bool = False, codes=None, scales=None):
    """Quantize x [B, H, S, D] (float32 or bfloat16, on the GPU) to e4m3 codes with one
    float32 scale per (b, h, block of scale_block tokens). Returns (codes, scales)."""
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("x must be float32 or bfloat16")
    px = _dev(x, "x", x.dtype, 4)
    B, H, S, D = x.shape
    nb = (S + scale_block - 1) // scale_block if scale_block > 0 else 0
    if codes is None:
        codes = torch.empty((B, H, S, D), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((B, H, max(nb, 1)), dtype=torch.float32, device=x.device)
    pc = _dev(codes, "codes", torch.uint8, 4)
    ps = _dev(scales, "scales", torch.float32, 3)
    if tuple(codes.shape) != (B, H, S, D) or tuple(scales.shape) != (B, H, nb):
        raise ValueError("codes / scales have the wrong shape")
    stream = _stream(x, codes, scales)
    lib = load()
    st = lib.zyfa_quantize_fp8(px, int(x.dtype == torch.bfloat16), pc, ps, B, H, S, D, scale_block,
                               int(bool(hadamard)), stream)
    _lib.check(st, "zyfa_quantize_fp8")
    return codes, scales


def _attn_shapes(q, k, v):
    B, Hq, S, Dqk = q.shape
    Bk, Hkv, Sk, Dk = k.shape
    if (Bk, Sk, Dk) != (B, S, Dqk) or v.shape[0] != B or v.shape[1] != Hkv or v.shape[2] != S:
        raise ValueError(f"inconsistent shapes q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    return B, Hq, Hkv, S, Dqk, v.shape[3]


def _outputs(q, B, Hq, S, Dv, o, lse, return_lse):
    if o is None:
        o = torch.empty((B, Hq, S, Dv), dtype=torch.bfloat16, device=q.device)
    po = _dev(o, "o", torch.bfloat16, 4)
    if tuple(o.shape) != (B, Hq, S, Dv):
        raise ValueError("o has the wrong shape")
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    plse = None
    if lse is not None:
        plse = _dev(lse, "lse", torch.float32, 3)
        if tuple(lse.shape) != (B, Hq, S):
            raise ValueError("lse has the wrong shape")
    return o, po, lse, plse


def attn_fwd_fp8(q, k, v, q_scale, k_scale, v_scale, scale_block: int, softmax_scale=None, o=None, lse=None,
                 return_lse: bool = False, lean: bool = False):
    """Causal attention on e4m3 codes (uint8 tensors [B, H, S, D]) with float32 block
    scales [B, H, ceil(S / scale_block)]. Returns (o bfloat16 [B, Hq, S, Dv], lse or None).
    lean=True calls zyfa_attn_fwd_fp8_lean (linear probability codes, the faster opt-in
    mode) instead of zyfa_attn_fwd_fp8."""
    pq = _dev(q, "q", torch.uint8, 4)
    pk = _dev(k, "k", torch.uint8, 4)
    pv = _dev(v, "v", torch.uint8, 4)
    B, Hq, Hkv, S, Dqk, Dv = _attn_shapes(q, k, v)
    nb = (S + scale_block - 1) // scale_block if scale_block > 0 else 0
    psq = _dev(q_scale, "q_scale", torch.float32, 3)
    psk = _dev(k_scale, "k_scale", torch.float32, 3)
    psv = _dev(v_scale, "v_scale", torch.float32, 3)
    if tuple(q_scale.shape) != (B, Hq, nb) or tuple(k_scale.shape) != (B, Hkv, nb) or tuple(v_scale.shape) != (B, Hkv, nb):
        raise ValueError("scale tensors have the wrong shape")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(Dqk)
    o, po, lse, plse = _outputs(q, B, Hq, S, Dv, o, lse, return_lse)
    name = "zyfa_attn_fwd_fp8_lean" if lean else "zyfa_attn_fwd_fp8"
    stream = _stream(q, k, v, q_scale, k_scale, v_scale, o, lse)
    st = getattr(load(), name)(pq, pk, pv, psq, psk, psv, scale_block, po, plse, B, Hq, Hkv, S, Dqk, Dv,
                               float(softmax_scale), stream)
    _lib.check(st, name)
    return o, lse


def attn_fwd_bf16(q, k, v, softmax_scale=None, o=None, lse=None, return_lse: bool = False):
    """Causal attention on bfloat16 tensors [B, H, S, D]. Returns (o bfloat16, lse or None)."""
    pq = _dev(q, "q", torch.bfloat16, 4)
    pk = _dev(k, "k", torch.bfloat16, 4)
    pv = _dev(v, "v", torch.bfloat16, 4)
    B, Hq, Hkv, S, Dqk, Dv = _attn_shapes(q, k, v)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(Dqk)
    o, po, lse, plse = _outputs(q, B, Hq, S, Dv, o, lse, return_lse)
    stream = _stream(q, k, v, o, lse)
    st = load().zyfa_attn_fwd_bf16(pq, pk, pv, po, plse, B, Hq, Hkv, S, Dqk, Dv, float(softmax_scale), stream)
    _lib.check(st, "zyfa_attn_fwd_bf16")
    return o, lse


def _range_shapes(q, k, v):
    B, Hq, Sq, Dqk = q.shape
    Bk, Hkv, Skv, Dk = k.shape
    if (Bk, Dk) != (B, Dqk) or tuple(v.shape[:3]) != (B, Hkv, Skv):
        raise ValueError(f"inconsistent shapes q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    return B, Hq, Hkv, Sq, Skv, Dqk, v.shape[3]


def attn_fwd_fp8_range(q, k, v, q_scale, k_scale, v_scale, scale_block: int, q_offset: int = 0, k_begin: int = 0,
                       k_end=None, softmax_scale=None, o=None, lse=None, return_lse: bool = False,
                       lean: bool = False):
    """Causal attention of the query rows q [B, Hq, Sq, Dqk] (row i at sequence position
    q_offset + i) against the keys [k_begin, k_end) of k, v [B, Hkv, Skv, D] (e4m3 codes,
    uint8), with float32 block scales q_scale [B, Hq, ceil(Sq / blk)] and k_scale, v_scale
    [B, Hkv, ceil(Skv / blk)]. k_end defaults to Skv. Rows that see no key get O = 0 and
    LSE = -inf. Returns (o bfloat16 [B, Hq, Sq, Dv], lse or None)."""
    pq = _dev(q, "q", torch.uint8, 4)
    pk = _dev(k, "k", torch.uint8, 4)
    pv = _dev(v, "v", torch.uint8, 4)
    B, Hq, Hkv, Sq, Skv, Dqk, Dv = _range_shapes(q, k, v)
    nbq = (Sq + scale_block - 1) // scale_block if scale_block > 0 else 0
    nbk = (Skv + scale_block - 1) // scale_block if scale_block > 0 else 0
    psq = _dev(q_scale, "q_scale", torch.float32, 3)
    psk = _dev(k_scale, "k_scale", torch.float32, 3)
    psv = _dev(v_scale, "v_scale", torch.float32, 3)
    if (tuple(q_scale.shape) != (B, Hq, nbq) or tuple(k_scale.shape) != (B, Hkv, nbk)
            or tuple(v_scale.shape) != (B, Hkv, nbk)):
        raise ValueError("scale tensors have the wrong shape")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(Dqk)
    if k_end is None:
        k_end = Skv
    o, po, lse, plse = _outputs(q, B, Hq, Sq, Dv, o, lse, return_lse)
    stream = _stream(q, k, v, q_scale, k_scale, v_scale, o, lse)
    st = load().zyfa_attn_fwd_fp8_range(pq, pk, pv, psq, psk, psv, scale_block, po, plse, B, Hq, Hkv, Sq, Skv,
                                        int(q_offset), int(k_begin), int(k_end), Dqk, Dv, float(softmax_scale),
                                        int(bool(lean)), stream)
    _lib.check(st, "zyfa_attn_fwd_fp8_range")
    return o, lse


def attn_fwd_bf16_range(q, k, v, q_offset: int = 0, k_begin: int = 0, k_end=None, softmax_scale=None, o=None,
                        lse=None, return_lse: bool = False):
    """attn_fwd_fp8_range on bfloat16 tensors. Returns (o bfloat16 [B, Hq, Sq, Dv], lse or None)."""
    pq = _dev(q, "q", torch.bfloat16, 4)
    pk = _dev(k, "k", torch.bfloat16, 4)
    pv = _dev(v, "v", torch.bfloat16, 4)
    B, Hq, Hkv, Sq, Skv, Dqk, Dv = _range_shapes(q, k, v)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(Dqk)
    if k_end is None:
        k_end = Skv
    o, po, lse, plse = _outputs(q, B, Hq, Sq, Dv, o, lse, return_lse)
    stream = _stream(q, k, v, o, lse)
    st = load().zyfa_attn_fwd_bf16_range(pq, pk, pv, po, plse, B, Hq, Hkv, Sq, Skv, int(q_offset), int(k_begin),
                                         int(k_end), Dqk, Dv, float(softmax_scale), stream)
    _lib.check(st, "zyfa_attn_fwd_bf16_range")
    return o, lse


def attn_merge(o_parts, lse_parts, o=None, lse=None, return_lse: bool = False):
    """Combine partial results over disjoint key sets: o_parts [P, ..., Dv] bfloat16 and
    lse_parts [P, ...] float32 (natural log; -inf where a part saw no key of the row).
    Returns (o bfloat16 [..., Dv], lse float32 [...] or None)."""
    if o_parts.dim() < 2 or tuple(lse_parts.shape) != tuple(o_parts.shape[:-1]):
        raise ValueError(f"inconsistent shapes o_parts {tuple(o_parts.shape)} lse_parts {tuple(lse_parts.shape)}")
    po_p = _dev(o_parts, "o_parts", torch.bfloat16, o_parts.dim())
    pl_p = _dev(lse_parts, "lse_parts", torch.float32, lse_parts.dim())
    P, Dv = o_parts.shape[0], o_parts.shape[-1]
    rows = lse_parts.numel() // P
    out_shape = tuple(o_parts.shape[1:])
    if o is None:
        o = torch.empty(out_shape, dtype=torch.bfloat16, device=o_parts.device)
    po = _dev(o, "o", torch.bfloat16, len(out_shape))
    if tuple(o.shape) != out_shape:
        raise ValueError("o has the wrong shape")
    if lse is None and return_lse:
        lse = torch.empty(out_shape[:-1], dtype=torch.float32, device=o_parts.device)
    plse = None
    if lse is not None:
        plse = _dev(lse, "lse", torch.float32, len(out_shape) - 1)
        if tuple(lse.shape) != out_shape[:-1]:
            raise ValueError("lse has the wrong shape")
    stream = _stream(o_parts, lse_parts, o, lse)
    st = load().zyfa_attn_merge(po_p, pl_p, P, po, plse, rows, Dv, stream)
    _lib.check(st, "zyfa_attn_merge")
    return o, lse


def _varlen_common(q, k, v, cu_seqlens, max_seqlen, o, lse, return_lse):
    Hq, T, Dqk = q.shape
    Hkv, Tk, Dk = k.shape
    if (Tk, Dk) != (T, Dqk) or tuple(v.shape[:2]) != (Hkv, T):
        raise ValueError(f"inconsistent shapes q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    pcu = _dev(cu_seqlens, "cu_seqlens", torch.int32, 1)
    n_seqs = cu_seqlens.shape[0] - 1
    Dv = v.shape[2]
    if o is None:
        o = torch.zeros((Hq, T, Dv), dtype=torch.bfloat16, device=q.device)
    po = _dev(o, "o", torch.bfloat16, 3)
    if tuple(o.shape) != (Hq, T, Dv):
        raise ValueError("o has the wrong shape")
    if lse is None and return_lse:
        lse = torch.full((Hq, T), float("-inf"), dtype=torch.float32, device=q.device)
    plse = None
    if lse is not None:
        plse = _dev(lse, "lse", torch.float32, 2)
        if tuple(lse.shape) != (Hq, T):
            raise ValueError("lse has the wrong shape")
    return Hq, Hkv, T, Dqk, Dv, n_seqs, pcu, o, po, lse, plse


def attn_fwd_fp8_varlen(q, k, v, q_scale, k_scale, v_scale, scale_block: int, cu_seqlens, max_seqlen: int,
                        softmax_scale=None, o=None, lse=None, return_lse: bool = False, lean: bool = False):
    """Causal attention over a packed batch: q [Hq, T, Dqk], k [Hkv, T, Dqk], v [Hkv, T, Dv]
    (e4m3 codes, uint8), scales [H, ceil(T / scale_block)] (as quantize_fp8 writes them for
    the tensors viewed as [1, H, T, D]); sequence i is tokens cu_seqlens[i] ..
    cu_seqlens[i+1] - 1 (int32 device tensor; starts multiples of 64). Tokens outside every
    sequence are left as they are in o / lse (zeros and -inf when this call allocates them).
    Returns (o bfloat16 [Hq, T, Dv], lse or None)."""
    pq = _dev(q, "q", torch.uint8, 3)
    pk = _dev(k, "k", torch.uint8, 3)
    pv = _dev(v, "v", torch.uint8, 3)
    Hq, Hkv, T, Dqk, Dv, n_seqs, pcu, o, po, lse, plse = _varlen_common(q, k, v, cu_seqlens, max_seqlen, o, lse,
                                                                        return_lse)
    nb = (T + scale_block - 1) // scale_block if scale_block > 0 else 0
    psq = _dev(q_scale, "q_scale", torch.float32, 2)
    psk = _dev(k_scale, "k_scale", torch.float32, 2)
    psv = _dev(v_scale, "v_scale", torch.float32, 2)
    if tuple(q_scale.shape) != (Hq, nb) or tuple(k_scale.shape) != (Hkv, nb) or tuple(v_scale.shape) != (Hkv, nb):
        raise ValueError("scale tensors have the wrong shape")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(Dqk)
    stream = _stream(q, k, v, q_scale, k_scale, v_scale, cu_seqlens, o, lse)
    st = load().zyfa_attn_fwd_fp8_varlen(pq, pk, pv, psq, psk, psv, scale_block, po, plse, pcu, n_seqs,
                                         int(max_seqlen), Hq, Hkv, T, Dqk, Dv, float(softmax_scale), int(bool(lean)),
                                         stream)
    _lib.check(st, "zyfa_attn_fwd_fp8_varlen")
    return o, lse


def attn_fwd_bf16_varlen(q, k, v, cu_seqlens, max_seqlen: int, softmax_scale=None, o=None, lse=None,
                         return_lse: bool = False):
    """attn_fwd_fp8_varlen on bfloat16 tensors. Returns (o bfloat16 [Hq, T, Dv], lse or None)."""
    pq = _dev(q, "q", torch.bfloat16, 3)
    pk = _dev(k, "k", torch.bfloat16, 3)
    pv = _dev(v, "v", torch.bfloat16, 3)
    Hq, Hkv, T, Dqk, Dv, n_seqs, pcu, o, po, lse, plse = _varlen_common(q, k, v, cu_seqlens, max_seqlen, o, lse,
                                                                        return_lse)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(Dqk)
    stream = _stream(q, k, v, cu_seqlens, o, lse)
    st = load().zyfa_attn_fwd_bf16_varlen(pq, pk, pv, po, plse, pcu, n_seqs, int(max_seqlen), Hq, Hkv, T, Dqk, Dv,
                                          float(softmax_scale), stream)
    _lib.check(st, "zyfa_attn_fwd_bf16_varlen")
    return o, lse


def _paged_common(q, k_cache, v_cache, cu_seqlens, kv_lens, block_table, max_seqlen, o, lse, return_lse):
    Hq, T, Dqk = q.shape
    num_pages, Hkv, page_size, Dk = k_cache.shape
    if Dk != Dqk or tuple(v_cache.shape[:3]) != (num_pages, Hkv, page_size):
        raise ValueError(f"inconsistent shapes q {tuple(q.shape)} k_cache {tuple(k_cache.shape)} "
                         f"v_cache {tuple(v_cache.shape)}")
    pcu = _dev(cu_seqlens, "cu_seqlens", torch.int32, 1)
    n_seqs = cu_seqlens.shape[0] - 1
    pkl = _dev(kv_lens, "kv_lens", torch.int32, 1)
    pbt = _dev(block_table, "block_table", torch.int32, 2)
    if kv_lens.shape[0] != n_seqs or block_table.shape[0] != n_seqs:
        raise ValueError("kv_lens and block_table need one entry / row per sequence")
    max_pages = block_table.shape[1]
    Dv = v_cache.shape[3]
    if o is None:
        o = torch.zeros((Hq, T, Dv), dtype=torch.bfloat16, device=q.device)
    po = _dev(o, "o", torch.bfloat16, 3)
    if tuple(o.shape) != (Hq, T, Dv):
        raise ValueError("o has the wrong shape")
    if lse is None and return_lse:
        lse = torch.full((Hq, T), float("-inf"), dtype=torch.float32, device=q.device)
    plse = None
    if lse is not None:
        plse = _dev(lse, "lse", torch.float32, 2)
        if tuple(lse.shape) != (Hq, T):
            raise ValueError("lse has the wrong shape")
    return (Hq, Hkv, T, Dqk, Dv, n_seqs, num_pages, page_size, max_pages, pcu, pkl, pbt, o, po, lse, plse)


def attn_fwd_fp8_paged(q, k_cache, v_cache, q_scale, k_cache_scale, v_cache_scale, scale_block: int, cu_seqlens,
                       kv_lens, block_table, max_seqlen: int, softmax_scale=None, o=None, lse=None,
                       return_lse: bool = False, lean: bool = False):
    """Prefill of chunks of new tokens against a paged key/value cache. q [Hq, T, Dqk] (e4m3
    codes) packs the chunks as in attn_fwd_fp8_varlen (cu_seqlens, int32, starts multiples of
    64); k_cache / v_cache [num_pages, Hkv, page_size, D] (e4m3 codes), their scales
    [num_pages, Hkv, page_size / scale_block] (quantize_fp8 of the cache as
    [num_pages, Hkv, page_size, D]); block_table int32 [n_seqs, max_pages] lists each
    sequence's pages; kv_lens int32 [n_seqs] its token count, of which its chunk is the
    last. Row r of chunk i sits at position kv_lens[i] - L_i + r. Rows outside every chunk
    are left as they are. Returns (o bfloat16 [Hq, T, Dv], lse or None)."""
    pq = _dev(q, "q", torch.uint8, 3)
    pk = _dev(k_cache, "k_cache", torch.uint8, 4)
    pv = _dev(v_cache, "v_cache", torch.uint8, 4)
    (Hq, Hkv, T, Dqk, Dv, n_seqs, num_pages, page_size, max_pages, pcu, pkl, pbt, o, po, lse,
     plse) = _paged_common(q, k_cache, v_cache, cu_seqlens, kv_lens, block_table, max_seqlen, o, lse, return_lse)
    nbq = (T + scale_block - 1) // scale_block if scale_block > 0 else 0
    nbp = page_size // scale_block if scale_block > 0 else 0
    psq = _dev(q_scale, "q_scale", torch.float32, 2)
    psk = _dev(k_cache_scale, "k_cache_scale", torch.float32, 3)
    psv = _dev(v_cache_scale, "v_cache_scale", torch.float32, 3)
    if (tuple(q_scale.shape) != (Hq, nbq) or tuple(k_cache_scale.shape) != (num_pages, Hkv, nbp)
            or tuple(v_cache_scale.shape) != (num_pages, Hkv, nbp)):
        raise ValueError("scale tensors have the wrong shape")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(Dqk)
    stream = _stream(q, k_cache, v_cache, q_scale, k_cache_scale, v_cache_scale, cu_seqlens, kv_lens, block_table, o,
                     lse)
    st = load().zyfa_attn_fwd_fp8_paged(pq, pk, pv, psq, psk, psv, scale_block, po, plse, pcu, pkl, pbt, n_seqs,
                                        int(max_seqlen), max_pages, num_pages, page_size, Hq, Hkv, T, Dqk, Dv,
                                        float(softmax_scale), int(bool(lean)), stream)
    _lib.check(st, "zyfa_attn_fwd_fp8_paged")
    return o, lse


def attn_fwd_bf16_paged(q, k_cache, v_cache, cu_seqlens, kv_lens, block_table, max_seqlen: int, softmax_scale=None,
                        o=None, lse=None, return_lse: bool = False):
    """attn_fwd_fp8_paged on bfloat16 tensors. Returns (o bfloat16 [Hq, T, Dv], lse or None)."""
    pq = _dev(q, "q", torch.bfloat16, 3)
    pk = _dev(k_cache, "k_cache", torch.bfloat16, 4)
    pv = _dev(v_cache, "v_cache", torch.bfloat16, 4)
    (Hq, Hkv, T, Dqk, Dv, n_seqs, num_pages, page_size, max_pages, pcu, pkl, pbt, o, po, lse,
     plse) = _paged_common(q, k_cache, v_cache, cu_seqlens, kv_lens, block_table, max_seqlen, o, lse, return_lse)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(Dqk)
    stream = _stream(q, k_cache, v_cache, cu_seqlens, kv_lens, block_table, o, lse)
    st = load().zyfa_attn_fwd_bf16_paged(pq, pk, pv, po, plse, pcu, pkl, pbt, n_seqs, int(max_seqlen), max_pages,
                                         num_pages, page_size, Hq, Hkv, T, Dqk, Dv, float(softmax_scale), stream)
    _lib.check(st, "zyfa_attn_fwd_bf16_paged")
    return o, lse


def decode_split_keys(B: int, Hkv: int, max_kv_len: int, target_workgroups: int = 1024) -> int:
    """Keys per split for the decode calls: enough splits that B * Hkv * splits reaches
    about target_workgroups, at least 256 keys each, a multiple of 64. The default, 1024,
    is four workgroups per compute unit of an MI355X, what the one-wave FP8 decode
    workgroup (up to 32 query heads per KV head) fits; the eight-wave workgroup (BF16, or
    larger groups) fits one, and its calls default to 256."""
    per = -(-max_kv_len * B * Hkv // target_workgroups)
    return max(256, -(-per // 64) * 64)


def _decode_common(q, k_cache, v_cache, kv_lens, block_table, max_kv_len, split_keys, o, lse, return_lse,
                   one_wave):
    B, Hq, Dqk = q.shape
    num_pages, Hkv, page_size, Dk = k_cache.shape
    if Dk != Dqk or tuple(v_cache.shape[:3]) != (num_pages, Hkv, page_size):
        raise ValueError(f"inconsistent shapes q {tuple(q.shape)} k_cache {tuple(k_cache.shape)} "
                         f"v_cache {tuple(v_cache.shape)}")
    pkl = _dev(kv_lens, "kv_lens", torch.int32, 1)
    pbt = _dev(block_table, "block_table", torch.int32, 2)
    if kv_lens.shape[0] != B or block_table.shape[0] != B:
        raise ValueError("kv_lens and block_table need one entry / row per sequence")
    max_pages = block_table.shape[1]
    Dv = v_cache.shape[3]
    if split_keys is None:
        split_keys = decode_split_keys(B, Hkv, int(max_kv_len), 1024 if one_wave else 256)
    if o is None:
        o = torch.empty((B, Hq, Dv), dtype=torch.bfloat16, device=q.device)
    po = _dev(o, "o", torch.bfloat16, 3)
    if tuple(o.shape) != (B, Hq, Dv):
        raise ValueError("o has the wrong shape")
    if lse is None and return_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    plse = None
    if lse is not None:
        plse = _dev(lse, "lse", torch.float32, 2)
        if tuple(lse.shape) != (B, Hq):
            raise ValueError("lse has the wrong shape")
    nbytes = load().zyfa_attn_decode_workspace_bytes(B, Hq, Dv, int(max_kv_len), int(split_keys))
    ws = torch.empty(max(nbytes, 0) + 256, dtype=torch.uint8, device=q.device) if nbytes > 0 else None
    pws = None if ws is None else (ws.data_ptr() + 255) // 256 * 256
    return (B, Hq, Hkv, Dqk, Dv, num_pages, page_size, max_pages, int(split_keys), pkl, pbt, o, po, lse, plse, ws,
            pws, max(nbytes, 0))


def attn_decode_fp8_paged(q, k_cache, v_cache, q_scale, k_cache_scale, v_cache_scale, scale_block: int, kv_lens,
                          block_table, max_kv_len: int, softmax_scale=None, split_keys=None, o=None, lse=None,
                          return_lse: bool = False, lean: bool = False):
    """Decode: one new token per sequence, q [B, Hq, Dqk] (e4m3 codes), at position
    kv_lens[b] - 1 of its sequence, against the paged cache (layout as attn_fwd_fp8_paged);
    q_scale [B, Hkv, ceil((Hq / Hkv) / scale_block)] (quantize_fp8 of q viewed as
    [B, Hkv, Hq / Hkv, Dqk]). max_kv_len bounds kv_lens; split_keys (keys per workgroup
    split, a multiple of 64) defaults to decode_split_keys. Returns (o bfloat16 [B, Hq, Dv],
    lse or None)."""
    pq = _dev(q, "q", torch.uint8, 3)
    pk = _dev(k_cache, "k_cache", torch.uint8, 4)
    pv = _dev(v_cache, "v_cache", torch.uint8, 4)
    (B, Hq, Hkv, Dqk, Dv, num_pages, page_size, max_pages, split_keys, pkl, pbt, o, po, lse, plse, ws, pws,
     nbytes) = _decode_common(q, k_cache, v_cache, kv_lens, block_table, max_kv_len, split_keys, o, lse, return_lse,
                              q.shape[1] <= 32 * k_cache.shape[1])
    g = Hq // Hkv if Hkv > 0 else 0
    nbg = (g + scale_block - 1) // scale_block if scale_block > 0 else 0
    nbp = page_size // scale_block if scale_block > 0 else 0
    psq = _dev(q_scale, "q_scale", torch.float32, 3)
    psk = _dev(k_cache_scale, "k_cache_scale", torch.float32, 3)
    psv = _dev(v_cache_scale, "v_cache_scale", torch.float32, 3)
    if (tuple(q_scale.shape) != (B, Hkv, nbg) or tuple(k_cache_scale.shape) != (num_pages, Hkv, nbp)
            or tuple(v_cache_scale.shape) != (num_pages, Hkv, nbp)):
        raise ValueError("scale tensors have the wrong shape")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(Dqk)
    stream = _stream(q, k_cache, v_cache, q_scale, k_cache_scale, v_cache_scale, kv_lens, block_table, o, lse, ws)
    st = load().zyfa_attn_decode_fp8_paged(pq, pk, pv, psq, psk, psv, scale_block, po, plse, pkl, pbt, B,
                                           int(max_kv_len), max_pages, num_pages, page_size, Hq, Hkv, Dqk, Dv,
                                           float(softmax_scale), split_keys, pws, nbytes, int(bool(lean)), stream)
    _lib.check(st, "zyfa_attn_decode_fp8_paged")
    del ws  # (the stream orders its reuse by the caching allocator after the kernels)
    return o, lse


NOALLOC_SCRATCH_BYTES = 8 << 20  # the library's per-GPU scratch array for the allocation-free decode


def attn_decode_fp8_paged_noalloc(q, k_cache, v_cache, q_scale, k_cache_scale, v_cache_scale, scale_block: int,
                                  kv_lens, block_table, max_kv_len: int, o, lse=None, softmax_scale=None,
                                  split_keys=None, lean: bool = False):
    """attn_decode_fp8_paged for callers that cannot allocate (graph capture, tight serving
    loops): the splits' partial results go to the library's per-GPU scratch array, and this
    wrapper allocates nothing either, so the caller passes o [B, Hq, Dv] bfloat16 and, if
    wanted, lse [B, Hq] float32. Calls that overlap on one GPU race. Returns (o, lse)."""
    if o is None:
        raise ValueError("the allocation-free decode writes into a caller's o")
    B, Hq, Dqk = q.shape
    num_pages, Hkv, page_size, Dk = k_cache.shape
    if Dk != Dqk or tuple(v_cache.shape[:3]) != (num_pages, Hkv, page_size):
        raise ValueError(f"inconsistent shapes q {tuple(q.shape)} k_cache {tuple(k_cache.shape)} "
                         f"v_cache {tuple(v_cache.shape)}")
    pq = _dev(q, "q", torch.uint8, 3)
    pk = _dev(k_cache, "k_cache", torch.uint8, 4)
    pv = _dev(v_cache, "v_cache", torch.uint8, 4)
    pkl = _dev(kv_lens, "kv_lens", torch.int32, 1)
    pbt = _dev(block_table, "block_table", torch.int32, 2)
    if kv_lens.shape[0] != B or block_table.shape[0] != B:
        raise ValueError("kv_lens and block_table need one entry / row per sequence")
    Dv = v_cache.shape[3]
    po = _dev(o, "o", torch.bfloat16, 3)
    if tuple(o.shape) != (B, Hq, Dv):
        raise ValueError("o has the wrong shape")
    plse = None
    if lse is not None:
        plse = _dev(lse, "lse", torch.float32, 2)
        if tuple(lse.shape) != (B, Hq):
            raise ValueError("lse has the wrong shape")
    if split_keys is None:
        split_keys = decode_split_keys(B, Hkv, int(max_kv_len), 1024 if Hq <= 32 * Hkv else 256)
    g = Hq // Hkv if Hkv > 0 else 0
    nbg = (g + scale_block - 1) // scale_block if scale_block > 0 else 0
    nbp = page_size // scale_block if scale_block > 0 else 0
    psq = _dev(q_scale, "q_scale", torch.float32, 3)
    psk = _dev(k_cache_scale, "k_cache_scale", torch.float32, 3)
    psv = _dev(v_cache_scale, "v_cache_scale", torch.float32, 3)
    if (tuple(q_scale.shape) != (B, Hkv, nbg) or tuple(k_cache_scale.shape) != (num_pages, Hkv, nbp)
            or tuple(v_cache_scale.shape) != (num_pages, Hkv, nbp)):
        raise ValueError("scale tensors have the wrong shape")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(Dqk)
    stream = _stream(q, k_cache, v_cache, q_scale, k_cache_scale, v_cache_scale, kv_lens, block_table, o, lse)
    st = load().zyfa_attn_decode_fp8_paged_noalloc(pq, pk, pv, psq, psk, psv, scale_block, po, plse, pkl, pbt, B,
                                                   int(max_kv_len), block_table.shape[1], num_pages, page_size, Hq,
                                                   Hkv, Dqk, Dv, float(softmax_scale), int(split_keys),
                                                   int(bool(lean)), stream)
    _lib.check(st, "zyfa_attn_decode_fp8_paged_noalloc")
    return o, lse


def attn_decode_bf16_paged(q, k_cache, v_cache, kv_lens, block_table, max_kv_len: int, softmax_scale=None,
                           split_keys=None, o=None, lse=None, return_lse: bool = False):
    """attn_decode_fp8_paged on bfloat16 tensors. Returns (o bfloat16 [B, Hq, Dv], lse or None)."""
    pq = _dev(q, "q", torch.bfloat16, 3)
    pk = _dev(k_cache, "k_cache", torch.bfloat16, 4)
    pv = _dev(v_cache, "v_cache", torch.bfloat16, 4)
    (B, Hq, Hkv, Dqk, Dv, num_pages, page_size, max_pages, split_keys, pkl, pbt, o, po, lse, plse, ws, pws,
     nbytes) = _decode_common(q, k_cache, v_cache, kv_lens, block_table, max_kv_len, split_keys, o, lse, return_lse,
                              False)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(Dqk)
    stream = _stream(q, k_cache, v_cache, kv_lens, block_table, o, lse, ws)
    st = load().zyfa_attn_decode_bf16_paged(pq, pk, pv, po, plse, pkl, pbt, B, int(max_kv_len), max_pages, num_pages,
                                            page_size, Hq, Hkv, Dqk, Dv, float(softmax_scale), split_keys, pws, nbytes,
                                            stream)
    _lib.check(st, "zyfa_attn_decode_bf16_paged")
    del ws
    return o, lse
