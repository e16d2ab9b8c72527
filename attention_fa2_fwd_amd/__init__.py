"""Python binding of the gfx950 attention library (libattn_fa2.so).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/attn_fa2.h.  PyTorch supplies
device memory (outputs are allocated with torch.empty when not given) and the
current stream.  There is no fallback: if the library is missing or a call
fails, an exception is raised.

Functions (same names as the C entry points):
    attn_fwd(q, k, v, ...)                      -> (out, lse)
    attn_build_block_mask(mask, B, Sq, Skv, ...) -> BlockMask
    attn_paged_decode_workspace_size(...)       -> int (bytes)
    attn_paged_decode(q, k_cache, v_cache, page_table, seq_lens, ...) -> (out, lse)
    attn_paged_decode_noalloc(q, k_cache, v_cache, page_table, seq_lens, ...) -> (out, lse)
    attn_block_mask_transpose(block_mask)       -> BlockMask with its lists by key block
    attn_bwd(q, k, v, out, lse, dout, ...)      -> (dq, dk, dv)

Every tensor's shape, dtype and device are checked against the sizes passed
to the C ABI before any call (the library sees only pointers and sizes).
"""

from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn_fa2.so")

F32, BF16 = 0, 1
MASK_KINDS = {"none": 0, "causal": 1, "sliding": 2, "prefix_lm": 3, "document": 4}
MASK_AND = 5   # masks joined with "&", e.g. "sliding&document&causal"
SCORE_KINDS = {"none": 0, "alibi": 1, "rel_pos": 2, "softcap": 3}
EXPORTED = ("attn_fwd", "attn_build_block_mask", "attn_block_mask_transpose",
            "attn_paged_decode_workspace_size", "attn_paged_decode", "attn_bwd_workspace_size",
            "attn_bwd", "attn_paged_decode_noalloc", "attn_last_error")


class AttnError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed with code {code}: {msg}")
        self.code = code


class MaskParams(ctypes.Structure):
    _fields_ = [("window", ctypes.c_int32), ("prefix_len", ctypes.c_int32),
                ("doc_ids", ctypes.c_void_p), ("and_kinds", ctypes.c_uint32)]


class ScoreParams(ctypes.Structure):
    _fields_ = [("alibi_slopes", ctypes.c_void_p), ("rel_scale", ctypes.c_float),
                ("softcap", ctypes.c_float)]


class BlockMaskC(ctypes.Structure):
    _fields_ = [("kv_num_blocks", ctypes.c_void_p), ("kv_indices", ctypes.c_void_p),
                ("kv_full", ctypes.c_void_p), ("q_block", ctypes.c_int32),
                ("kv_block", ctypes.c_int32), ("n_q_blocks", ctypes.c_int32),
                ("n_kv_blocks", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("q_num_blocks", ctypes.c_void_p), ("q_indices", ctypes.c_void_p),
                ("q_full", ctypes.c_void_p)]


@dataclass
class BlockMask:
    kv_num_blocks: torch.Tensor    # int32 [B, 1, nQB]
    kv_indices: torch.Tensor       # int32 [B, 1, nQB, nKVB]
    kv_full: Optional[torch.Tensor]  # uint8 [B, 1, nQB, nKVB]
    q_block: int
    kv_block: int
    # the same blocks listed by key block (attn_block_mask_transpose), for attn_bwd
    q_num_blocks: Optional[torch.Tensor] = None   # int32 [B, 1, nKVB]
    q_indices: Optional[torch.Tensor] = None      # int32 [B, 1, nKVB, nQB]
    q_full: Optional[torch.Tensor] = None         # uint8 [B, 1, nKVB, nQB]

    def to_c(self) -> BlockMaskC:
        b, _, nqb, nkb = self.kv_indices.shape
        return BlockMaskC(self.kv_num_blocks.data_ptr(), self.kv_indices.data_ptr(),
                          self.kv_full.data_ptr() if self.kv_full is not None else None,
                          self.q_block, self.kv_block, nqb, nkb, b, _ptr(self.q_num_blocks),
                          _ptr(self.q_indices), _ptr(self.q_full))


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libattn_fa2.so (built by attention_fa2_fwd_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m attention_fa2_fwd_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, f32,
                             i32, ctypes.POINTER(MaskParams), i32, ctypes.POINTER(ScoreParams),
                             ctypes.POINTER(BlockMaskC), vp]
    lib.attn_fwd.restype = i32
    lib.attn_build_block_mask.argtypes = [i32, ctypes.POINTER(MaskParams), i32, i32, i32, i32,
                                          i32, vp, vp, vp, vp]
    lib.attn_build_block_mask.restype = i32
    lib.attn_paged_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    lib.attn_paged_decode_workspace_size.restype = ctypes.c_size_t
    lib.attn_paged_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                      i32, i32, f32, i32, ctypes.POINTER(MaskParams), i32,
                                      ctypes.POINTER(ScoreParams), vp, ctypes.c_size_t, vp]
    lib.attn_paged_decode.restype = i32
    lib.attn_paged_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                              i32, i32, f32, i32, ctypes.POINTER(MaskParams), i32,
                                              ctypes.POINTER(ScoreParams), vp]
    lib.attn_paged_decode_noalloc.restype = i32
    lib.attn_block_mask_transpose.argtypes = [ctypes.POINTER(BlockMaskC), vp, vp, vp, vp]
    lib.attn_block_mask_transpose.restype = i32
    lib.attn_bwd_workspace_size.argtypes = [i32, i32, i32]
    lib.attn_bwd_workspace_size.restype = ctypes.c_size_t
    lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                             f32, i32, ctypes.POINTER(MaskParams), i32, ctypes.POINTER(ScoreParams),
                             ctypes.POINTER(BlockMaskC), vp, ctypes.c_size_t, vp]
    lib.attn_bwd.restype = i32
    lib.attn_last_error.argtypes = []
    lib.attn_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(fn: str, rc: int):
    if rc != 0:
        msg = load_library().attn_last_error().decode(errors="replace")
        raise AttnError(fn, rc, msg)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _need_device(*tensors):
    for t in tensors:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous device (GPU) tensors")


def _expect(t, name: str, shape, dtypes=None):
    """Refuse a tensor whose shape (or dtype) is not what the sizes passed to
    the C ABI say: the library cannot see tensor sizes, so a short buffer would
    be read or written out of bounds."""
    if t is None:
        return
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(int(x) for x in shape)}")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {tuple(dtypes)}")


def _same_device(ref, **named):
    for name, t in named.items():
        if t is not None and t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, not on {ref.device} with the other tensors")


def _dims(t, name: str, n: int):
    if t.dim() != n:
        raise ValueError(f"{name} must have {n} dimensions (got shape {tuple(t.shape)})")


def _check_block_mask(bm: BlockMask, B: int, Sq: int, Skv: int, ref, need_key_lists: bool):
    _dims(bm.kv_indices, "block_mask.kv_indices", 4)
    bb, one, nqb, nkb = bm.kv_indices.shape
    if one != 1 or bb not in (1, B):
        raise ValueError(f"block_mask.kv_indices has shape {tuple(bm.kv_indices.shape)}: "
                         f"expected [1 or B={B}, 1, nQB, nKVB]")
    if nqb != -(-Sq // bm.q_block) or nkb != -(-Skv // bm.kv_block):
        raise ValueError(f"block_mask of {nqb} x {nkb} blocks of {bm.q_block} x {bm.kv_block} does "
                         f"not cover Sq={Sq}, Skv={Skv}")
    i32, u8 = (torch.int32,), (torch.uint8,)
    _expect(bm.kv_num_blocks, "block_mask.kv_num_blocks", (bb, 1, nqb), i32)
    _expect(bm.kv_indices, "block_mask.kv_indices", (bb, 1, nqb, nkb), i32)
    _expect(bm.kv_full, "block_mask.kv_full", (bb, 1, nqb, nkb), u8)
    if need_key_lists:
        if bm.q_num_blocks is None or bm.q_indices is None:
            raise ValueError("block_mask needs its lists by key block (attn_block_mask_transpose)")
        _expect(bm.q_num_blocks, "block_mask.q_num_blocks", (bb, 1, nkb), i32)
        _expect(bm.q_indices, "block_mask.q_indices", (bb, 1, nkb, nqb), i32)
        _expect(bm.q_full, "block_mask.q_full", (bb, 1, nkb, nqb), u8)
    _same_device(ref, kv_num_blocks=bm.kv_num_blocks, kv_indices=bm.kv_indices, kv_full=bm.kv_full,
                 q_num_blocks=bm.q_num_blocks if need_key_lists else None,
                 q_indices=bm.q_indices if need_key_lists else None,
                 q_full=bm.q_full if need_key_lists else None)


def _check_mask_score_tensors(mask: str, doc_ids, alibi_slopes, B: int, Skv: int, Hq: int, ref):
    if doc_ids is not None:
        _expect(doc_ids, "doc_ids", (B, Skv), (torch.int32,))
    elif "document" in mask.split("&"):
        raise ValueError("a document mask needs doc_ids [B, S]")
    _expect(alibi_slopes, "alibi_slopes", (Hq,), (torch.float32,))
    _same_device(ref, doc_ids=doc_ids, alibi_slopes=alibi_slopes)


def _mask_params(mask: str, window: int, prefix_len: int, doc_ids: Optional[torch.Tensor]):
    kind, bits = _mask_kind(mask)
    if doc_ids is not None and doc_ids.dtype != torch.int32:
        raise ValueError("doc_ids must be int32")
    return kind, MaskParams(int(window), int(prefix_len), _ptr(doc_ids), bits)


def _mask_kind(mask: str):
    """(kind, and_kinds) of a mask name; names joined with "&" intersect."""
    if "&" not in mask:
        if mask not in MASK_KINDS:
            raise ValueError(f"unknown mask kind {mask!r}")
        return MASK_KINDS[mask], 0
    bits = 0
    for part in mask.split("&"):
        if part not in MASK_KINDS:
            raise ValueError(f"unknown mask kind {part!r} in {mask!r}")
        bits |= 1 << MASK_KINDS[part]
    return MASK_AND, bits


def _score_params(score: str, alibi_slopes: Optional[torch.Tensor], rel_scale: float,
                  softcap: float):
    if score not in SCORE_KINDS:
        raise ValueError(f"unknown score kind {score!r}")
    if alibi_slopes is not None and alibi_slopes.dtype != torch.float32:
        raise ValueError("alibi_slopes must be float32")
    return SCORE_KINDS[score], ScoreParams(_ptr(alibi_slopes), float(rel_scale), float(softcap))


def attn_fwd(q, k, v, *, scale: Optional[float] = None, mask: str = "none", window: int = 0,
             prefix_len: int = 0, doc_ids=None, score: str = "none", alibi_slopes=None,
             rel_scale: float = 1.0, softcap: float = 0.0, block_mask: Optional[BlockMask] = None,
             out=None, lse=None, out_dtype=None):
    """Fused attention forward.  q [B,Hq,Sq,D], k/v [B,Hkv,Skv,D] (bf16 or fp32).
    Returns (out [B,Hq,Sq,D], lse [B,Hq,Sq] float32).  out_dtype defaults to
    the input dtype; torch.float32 gives bf16 inputs an fp32 output."""
    lib = load_library()
    if q.dtype not in (torch.bfloat16, torch.float32) or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share dtype bf16 or float32")
    _dims(q, "q", 4)
    _dims(k, "k", 4)
    b, hq, sq, d = q.shape
    hkv, skv = k.shape[1], k.shape[2]
    _expect(k, "k", (b, hkv, skv, d))
    _expect(v, "v", (b, hkv, skv, d))
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((b, hq, sq), dtype=torch.float32, device=q.device)
    _expect(out, "out", q.shape, (torch.bfloat16, torch.float32))
    _expect(lse, "lse", (b, hq, sq), (torch.float32,))
    _check_mask_score_tensors(mask, doc_ids, alibi_slopes, b, skv, hq, q)
    _same_device(q, k=k, v=v, out=out, lse=lse)
    if block_mask is not None:
        _check_block_mask(block_mask, b, sq, skv, q, need_key_lists=False)
    _need_device(q, k, v, out, lse, doc_ids, alibi_slopes)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    mk, mp = _mask_params(mask, window, prefix_len, doc_ids)
    sk, sp = _score_params(score, alibi_slopes, rel_scale, softcap)
    bmc = block_mask.to_c() if block_mask is not None else None
    rc = lib.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                      BF16 if q.dtype == torch.bfloat16 else F32,
                      BF16 if out.dtype == torch.bfloat16 else F32, b, hq, hkv, sq, skv, d,
                      float(scale), mk, ctypes.byref(mp), sk, ctypes.byref(sp),
                      ctypes.byref(bmc) if bmc is not None else None, _stream(q.device))
    _check("attn_fwd", rc)
    return out, lse


def attn_build_block_mask(mask: str, B: int, Sq: int, Skv: int, *, q_block: int = 128,
                          kv_block: int = 128, window: int = 0, prefix_len: int = 0,
                          doc_ids=None, device="cuda", with_full: bool = True,
                          out: BlockMask = None) -> BlockMask:
    """Build the BlockMask of a mask kind on the GPU (into `out`'s buffers
    when given: a BlockMask of the same B, block sizes and block counts)."""
    lib = load_library()
    device = torch.device(device)
    nqb = -(-Sq // q_block)
    nkb = -(-Skv // kv_block)
    if out is not None:
        if (tuple(out.kv_indices.shape) != (B, 1, nqb, nkb) or out.q_block != q_block
                or out.kv_block != kv_block or (out.kv_full is None) == with_full):
            raise ValueError("out does not match the BlockMask being built")
        num, idx, full = out.kv_num_blocks, out.kv_indices, out.kv_full
    else:
        num = torch.empty((B, 1, nqb), dtype=torch.int32, device=device)
        idx = torch.empty((B, 1, nqb, nkb), dtype=torch.int32, device=device)
        full = torch.empty((B, 1, nqb, nkb), dtype=torch.uint8, device=device) if with_full else None
    _expect(num, "out.kv_num_blocks", (B, 1, nqb), (torch.int32,))
    _expect(idx, "out.kv_indices", (B, 1, nqb, nkb), (torch.int32,))
    _expect(full, "out.kv_full", (B, 1, nqb, nkb), (torch.uint8,))
    _check_mask_score_tensors(mask, doc_ids, None, B, Skv, 0, idx)
    _same_device(idx, kv_num_blocks=num, kv_full=full)
    _need_device(num, idx, full, doc_ids)
    mk, mp = _mask_params(mask, window, prefix_len, doc_ids)
    rc = lib.attn_build_block_mask(mk, ctypes.byref(mp), B, Sq, Skv, q_block, kv_block,
                                   num.data_ptr(), idx.data_ptr(), _ptr(full), _stream(device))
    _check("attn_build_block_mask", rc)
    return BlockMask(num, idx, full, q_block, kv_block)


def attn_block_mask_transpose(bm: BlockMask) -> BlockMask:
    """The BlockMask with its lists by key block filled in (for attn_bwd)."""
    lib = load_library()
    _dims(bm.kv_indices, "block_mask.kv_indices", 4)
    b, _, nqb, nkb = bm.kv_indices.shape
    _check_block_mask(bm, b, nqb * bm.q_block, nkb * bm.kv_block, bm.kv_indices, need_key_lists=False)
    dev = bm.kv_indices.device
    qnum = torch.empty((b, 1, nkb), dtype=torch.int32, device=dev)
    qidx = torch.empty((b, 1, nkb, nqb), dtype=torch.int32, device=dev)
    qfull = torch.empty((b, 1, nkb, nqb), dtype=torch.uint8, device=dev)
    _need_device(bm.kv_num_blocks, bm.kv_indices, bm.kv_full, qnum, qidx, qfull)
    c = bm.to_c()
    rc = lib.attn_block_mask_transpose(ctypes.byref(c), qnum.data_ptr(), qidx.data_ptr(),
                                       qfull.data_ptr(), _stream(dev))
    _check("attn_block_mask_transpose", rc)
    return BlockMask(bm.kv_num_blocks, bm.kv_indices, bm.kv_full, bm.q_block, bm.kv_block,
                     qnum, qidx, qfull)


def attn_paged_decode_workspace_size(num_seqs: int, Hq: int, D: int, max_pages_per_seq: int,
                                     page_size: int = 16) -> int:
    return int(load_library().attn_paged_decode_workspace_size(num_seqs, Hq, D,
                                                                max_pages_per_seq, page_size))


def _decode_args(q, k_cache, v_cache, page_table, seq_lens, scale, mask, window, score,
                 alibi_slopes, rel_scale, softcap, out, lse):
    """Checks shared by the two decode calls; returns the C arguments up to
    the score params."""
    if q.dtype != torch.bfloat16 or k_cache.dtype != torch.bfloat16 or v_cache.dtype != torch.bfloat16:
        raise ValueError("paged decode takes bf16 q and caches")
    if page_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("page_table and seq_lens must be int32")
    _dims(q, "q", 3)
    _dims(k_cache, "k_cache", 4)
    _dims(page_table, "page_table", 2)
    n, hq, d = q.shape
    pages, hkv, page_size, dc = k_cache.shape
    if dc != d:
        raise ValueError(f"k_cache rows hold {dc} values, q has D={d}")
    _expect(v_cache, "v_cache", k_cache.shape)
    if page_table.shape[0] != n:
        raise ValueError(f"page_table has {page_table.shape[0]} rows for {n} sequences")
    max_pages = page_table.shape[1]
    _expect(seq_lens, "seq_lens", (n,))
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((n, hq), dtype=torch.float32, device=q.device)
    _expect(out, "out", q.shape, (torch.bfloat16,))
    _expect(lse, "lse", (n, hq), (torch.float32,))
    _expect(alibi_slopes, "alibi_slopes", (hq,), (torch.float32,))
    _same_device(q, k_cache=k_cache, v_cache=v_cache, page_table=page_table, seq_lens=seq_lens,
                 out=out, lse=lse, alibi_slopes=alibi_slopes)
    _need_device(q, k_cache, v_cache, page_table, seq_lens, out, lse, alibi_slopes)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    sk, sp = _score_params(score, alibi_slopes, rel_scale, softcap)
    mk, bits = _mask_kind(mask)
    mp = MaskParams(int(window), 0, None, bits)
    args = (q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), page_table.data_ptr(),
            seq_lens.data_ptr(), out.data_ptr(), lse.data_ptr(), BF16, n, hq, hkv, d, page_size,
            max_pages, pages, float(scale), mk, mp, sk, sp)
    return args, out, lse


def attn_paged_decode(q, k_cache, v_cache, page_table, seq_lens, *, scale: Optional[float] = None,
                      mask: str = "none", window: int = 0, score: str = "none", alibi_slopes=None,
                      rel_scale: float = 1.0, softcap: float = 0.0, workspace=None, out=None,
                      lse=None):
    """Paged split-KV decode.  q [N,Hq,D] bf16; caches [pages,Hkv,page,D] bf16;
    page_table int32 [N,max_pages]; seq_lens int32 [N]; mask "none" or
    "sliding" (the query at seq_lens-1 sees the last `window` keys).
    Returns (out, lse)."""
    lib = load_library()
    args, out, lse = _decode_args(q, k_cache, v_cache, page_table, seq_lens, scale, mask, window,
                                  score, alibi_slopes, rel_scale, softcap, out, lse)
    n, hq, d, page_size, max_pages = args[8], args[9], args[11], args[12], args[13]
    need = attn_paged_decode_workspace_size(n, hq, d, max_pages, page_size)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _same_device(q, workspace=workspace)
    _need_device(workspace)
    mp, sp = args[17], args[19]
    rc = lib.attn_paged_decode(*args[:17], ctypes.byref(mp), args[18], ctypes.byref(sp),
                               workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                               _stream(q.device))
    _check("attn_paged_decode", rc)
    return out, lse


def attn_paged_decode_noalloc(q, k_cache, v_cache, page_table, seq_lens, *,
                              scale: Optional[float] = None, mask: str = "none", window: int = 0,
                              score: str = "none", alibi_slopes=None, rel_scale: float = 1.0,
                              softcap: float = 0.0, out=None, lse=None):
    """attn_paged_decode without a workspace: the split partials go to the
    library's fixed per-GPU scratch (64 MiB), so the C call allocates
    nothing (pass out and lse to allocate nothing here either).  Calls that
    overlap on one GPU race for that scratch."""
    lib = load_library()
    args, out, lse = _decode_args(q, k_cache, v_cache, page_table, seq_lens, scale, mask, window,
                                  score, alibi_slopes, rel_scale, softcap, out, lse)
    mp, sp = args[17], args[19]
    rc = lib.attn_paged_decode_noalloc(*args[:17], ctypes.byref(mp), args[18], ctypes.byref(sp),
                                       _stream(q.device))
    _check("attn_paged_decode_noalloc", rc)
    return out, lse


def attn_bwd(q, k, v, out, lse, dout, *, scale: Optional[float] = None, mask: str = "none",
             window: int = 0, prefix_len: int = 0, doc_ids=None, score: str = "none",
             alibi_slopes=None, rel_scale: float = 1.0, softcap: float = 0.0,
             block_mask: Optional[BlockMask] = None, workspace=None, dq=None, dk=None, dv=None):
    """Gradients of attn_fwd from its output and LSE.  q, out, dout
    [B,Hq,Sq,D] and k, v [B,Hkv,Skv,D] bf16; lse [B,Hq,Sq] float32.  Returns
    (dq, dk, dv) float32.  The mask and score arguments are the forward's."""
    lib = load_library()
    for t in (q, k, v, out, dout):
        if t.dtype != torch.bfloat16:
            raise ValueError("attn_bwd takes bf16 q, k, v, out, dout")
    _dims(q, "q", 4)
    _dims(k, "k", 4)
    b, hq, sq, d = q.shape
    hkv, skv = k.shape[1], k.shape[2]
    _expect(k, "k", (b, hkv, skv, d))
    _expect(v, "v", (b, hkv, skv, d))
    _expect(out, "out", q.shape)
    _expect(dout, "dout", q.shape)
    _expect(lse, "lse", (b, hq, sq), (torch.float32,))
    dq = torch.empty(q.shape, dtype=torch.float32, device=q.device) if dq is None else dq
    dk = torch.empty(k.shape, dtype=torch.float32, device=q.device) if dk is None else dk
    dv = torch.empty(v.shape, dtype=torch.float32, device=q.device) if dv is None else dv
    _expect(dq, "dq", q.shape, (torch.float32,))
    _expect(dk, "dk", k.shape, (torch.float32,))
    _expect(dv, "dv", k.shape, (torch.float32,))
    _check_mask_score_tensors(mask, doc_ids, alibi_slopes, b, skv, hq, q)
    need = int(lib.attn_bwd_workspace_size(b, hq, sq))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _same_device(q, k=k, v=v, out=out, lse=lse, dout=dout, dq=dq, dk=dk, dv=dv, workspace=workspace)
    if block_mask is not None:
        _check_block_mask(block_mask, b, sq, skv, q, need_key_lists=block_mask.q_indices is not None)
    _need_device(q, k, v, out, lse, dout, dq, dk, dv, workspace, doc_ids, alibi_slopes)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    mk, mp = _mask_params(mask, window, prefix_len, doc_ids)
    sk, sp = _score_params(score, alibi_slopes, rel_scale, softcap)
    if block_mask is not None and block_mask.q_indices is None:
        block_mask = attn_block_mask_transpose(block_mask)
    bmc = block_mask.to_c() if block_mask is not None else None
    rc = lib.attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                      dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), BF16, b, hq, hkv,
                      sq, skv, d, float(scale), mk, ctypes.byref(mp), sk, ctypes.byref(sp),
                      ctypes.byref(bmc) if bmc is not None else None,
                      workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                      _stream(q.device))
    _check("attn_bwd", rc)
    return dq, dk, dv
