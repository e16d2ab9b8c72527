"""C-ABI checks that need no GPU: the library loads, exports every entry point
include/attn_fa2.h declares, and rejects bad arguments on the host with the
documented error codes before any launch (null device pointers are passed, so
any launch would fault; none happens)."""

import ctypes
import os
import re

import pytest

import attention_fa2_fwd_amd as af

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_fa2.h")

pytestmark = pytest.mark.skipif(not os.path.exists(af.LIB_PATH), reason="library not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = af.load_library()
    names = declared_functions()
    assert names == sorted(af.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def _fwd(lib, dt=1, out_dt=None, B=1, Hq=4, Hkv=2, Sq=16, Skv=16, D=64, scale=0.125, mk=0, window=0,
         prefix=0, sk=0, bm=None, null_score=False, softcap=0.0, and_kinds=0):
    mp = af.MaskParams(window, prefix, None, and_kinds)
    sp = af.ScoreParams(None, 1.0, softcap)
    out_dt = dt if out_dt is None else out_dt
    return lib.attn_fwd(None, None, None, None, None, dt, out_dt, B, Hq, Hkv, Sq, Skv, D, scale, mk,
                        ctypes.byref(mp), sk, None if null_score else ctypes.byref(sp),
                        ctypes.byref(bm) if bm is not None else None, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(Hq=4, Hkv=3), -1),
    (dict(Hkv=0), -1),
    (dict(B=-1), -1),
    (dict(D=96), -2),
    (dict(dt=0, D=48), -2),
    (dict(dt=7), -1),
    (dict(out_dt=5), -1),
    (dict(dt=0, out_dt=1), -2),
    (dict(mk=9), -1),
    (dict(sk=5), -1),
    (dict(mk=2, window=0), -1),
    (dict(mk=3, prefix=-1), -1),
    (dict(mk=4), -1),                   # DOCUMENT without doc_ids
    (dict(sk=2, null_score=True), -1),  # REL_POS without params
    (dict(sk=3, null_score=True), -1),  # SOFTCAP without params
    (dict(sk=3, softcap=0.0), -1),      # cap must be > 0
    (dict(sk=3, softcap=-2.0), -1),
    (dict(sk=3, softcap=float("inf")), -1),
    (dict(sk=3, softcap=float("nan")), -1),
    (dict(sk=3, softcap=30.0), -1),     # valid cap, null tensors
    (dict(mk=5, and_kinds=1 << 5), -1),           # AND names no kind
    (dict(mk=5, and_kinds=1 << 2), -1),           # AND with a window of 0
    (dict(mk=5, and_kinds=(1 << 2) | (1 << 4), window=8), -1),   # no doc_ids
    (dict(mk=5, and_kinds=(1 << 3), prefix=-2), -1),
    (dict(mk=5, and_kinds=0), -1),                # empty AND is no mask; null tensors
    (dict(mk=5, and_kinds=(1 << 1) | (1 << 2) | (1 << 3), window=8), -1),   # null tensors
    (dict(scale=float("nan")), -1),
    (dict(), -1),                       # valid shapes but null tensors
])
def test_fwd_rejects_bad_arguments(kwargs, code):
    lib = af.load_library()
    assert _fwd(lib, **kwargs) == code
    assert lib.attn_last_error().decode()


def test_fwd_block_mask_checks():
    lib = af.load_library()
    bm = af.BlockMaskC(None, None, None, 128, 128, 1, 1, 1)
    assert _fwd(lib, bm=bm) == -1                          # null lists
    dummy = ctypes.c_int32(0)
    p = ctypes.addressof(dummy)
    bm = af.BlockMaskC(p, p, None, 64, 128, 1, 1, 1)
    assert _fwd(lib, bm=bm) == -2                          # block size
    bm = af.BlockMaskC(p, p, None, 128, 128, 2, 1, 1)
    assert _fwd(lib, bm=bm) == -1                          # shape mismatch
    bm = af.BlockMaskC(p, p, None, 128, 128, 1, 1, 3)
    assert _fwd(lib, bm=bm) == -1                          # batch mismatch
    # The bf16 kernel stages one row of the block list in LDS: at most 1024
    # key blocks (Skv <= 131072); the fp32 path has no such limit.
    bm = af.BlockMaskC(p, p, None, 128, 128, 1, 1025, 1)
    assert _fwd(lib, Sq=16, Skv=1025 * 128, bm=bm) == -2
    assert "1024" in lib.attn_last_error().decode()


def test_fwd_empty_problem_is_a_no_op():
    lib = af.load_library()
    assert _fwd(lib, Sq=0) == 0
    assert _fwd(lib, B=0) == 0


def test_block_mask_builder_checks():
    lib = af.load_library()
    mp = af.MaskParams(0, 0, None)
    assert lib.attn_build_block_mask(1, ctypes.byref(mp), 1, 256, 256, 100, 128, None, None, None, None) == -2
    assert lib.attn_build_block_mask(1, ctypes.byref(mp), 1, 256, 256, 128, 2048, None, None, None, None) == -2
    assert lib.attn_build_block_mask(1, ctypes.byref(mp), 1, 256, 256, 128, 128, None, None, None, None) == -1
    assert lib.attn_build_block_mask(2, ctypes.byref(mp), 1, 256, 256, 128, 128, None, None, None, None) == -1
    assert lib.attn_build_block_mask(1, ctypes.byref(mp), 0, 256, 256, 128, 128, None, None, None, None) == 0


def _dec(lib, N=2, Hq=8, Hkv=2, D=128, page=16, max_pages=4, pool=8, dt=1, mk=0, window=0, sk=0,
         ws=None, ws_bytes=0, softcap=0.0, and_kinds=0, doc=None):
    mp = af.MaskParams(window, 0, doc, and_kinds)
    sp = af.ScoreParams(None, 1.0, softcap)
    return lib.attn_paged_decode(None, None, None, None, None, None, None, dt, N, Hq, Hkv, D, page,
                                 max_pages, pool, 0.1, mk, ctypes.byref(mp), sk, ctypes.byref(sp), ws,
                                 ws_bytes, None)


def test_paged_decode_checks():
    lib = af.load_library()
    assert _dec(lib, Hq=6, Hkv=4) == -1
    assert _dec(lib, D=64) == -2
    assert _dec(lib, page=32) == -2
    assert _dec(lib, dt=0) == -2
    assert _dec(lib, Hq=34, Hkv=2) == -2
    assert _dec(lib, mk=1) == -2                           # only NONE and SLIDING
    assert _dec(lib, sk=3) == -1                           # SOFTCAP needs a cap > 0
    assert _dec(lib, mk=5, and_kinds=(1 << 1) | (1 << 2), window=9) == -1   # a window: null tensors
    assert _dec(lib, mk=5, and_kinds=1 << 1) == -2                          # causal alone
    assert _dec(lib, mk=5, and_kinds=1 << 4, doc=8) == -2                   # a document mask
    assert _dec(lib, mk=9) == -1
    assert _dec(lib, mk=2, window=0) == -1                 # window must be >= 1
    assert _dec(lib, mk=2, window=100) == -1               # valid mask, null tensors
    assert _dec(lib, N=0) == 0
    assert _dec(lib) == -1                                 # null tensors
    # rows = N * Hq * ceil(max_pages / 16); O part rounded up to 256 bytes
    for max_pages, splits in ((4, 1), (16, 1), (17, 2), (300, 19)):
        need = lib.attn_paged_decode_workspace_size(2, 8, 128, max_pages, 16)
        rows = 2 * 8 * splits
        assert need == (rows * 128 * 4 + 255) // 256 * 256 + rows * 4
    assert lib.attn_paged_decode_workspace_size(0, 8, 128, 4, 16) == 0


def _bwd(lib, dt=1, B=1, Hq=4, Hkv=2, Sq=16, Skv=16, D=64, mk=0, window=0, sk=0, bm=None,
         ws=None, ws_bytes=0, null_tensors=True):
    mp = af.MaskParams(window, 0, None, 0)
    sp = af.ScoreParams(None, 1.0, 0.0)
    return lib.attn_bwd(None, None, None, None, None, None, None, None, None, dt, B, Hq, Hkv, Sq, Skv,
                        D, 0.125, mk, ctypes.byref(mp), sk, ctypes.byref(sp),
                        ctypes.byref(bm) if bm is not None else None, ws, ws_bytes, None)


def test_bwd_checks():
    lib = af.load_library()
    assert _bwd(lib, dt=0) == -2                      # bf16 only
    assert _bwd(lib, D=96) == -2
    assert _bwd(lib, Hq=3) == -1
    assert _bwd(lib, mk=2) == -1                      # window 0
    assert _bwd(lib, sk=9) == -1
    assert _bwd(lib, B=0) == 0
    assert _bwd(lib) == -4                            # no workspace
    assert _bwd(lib, ws=256, ws_bytes=1 << 20) == -1  # workspace given, null tensors
    assert lib.attn_bwd_workspace_size(2, 3, 100) == (2 * 3 * 100 * 4 + 255) // 256 * 256
    assert lib.attn_bwd_workspace_size(0, 3, 100) == 0
    # a BlockMask without the lists by key block, or with other block sizes
    half = af.BlockMaskC(8, 8, None, 128, 128, 1, 1, 1, None, None, None)
    assert _bwd(lib, bm=half) == -1
    both = af.BlockMaskC(8, 8, None, 64, 64, 1, 1, 1, 8, 8, None)
    assert _bwd(lib, bm=both) == -2
    wrong = af.BlockMaskC(8, 8, None, 128, 128, 2, 1, 1, 8, 8, None)
    assert _bwd(lib, bm=wrong) == -1                  # 2 query blocks for Sq = 16


def test_block_mask_transpose_checks():
    lib = af.load_library()
    assert lib.attn_block_mask_transpose(None, None, None, None, None) == -1
    bm = af.BlockMaskC(None, None, None, 128, 128, 2, 2, 1, None, None, None)
    assert lib.attn_block_mask_transpose(ctypes.byref(bm), None, None, None, None) == -1
    empty = af.BlockMaskC(None, None, None, 128, 128, 2, 0, 1, None, None, None)
    assert lib.attn_block_mask_transpose(ctypes.byref(empty), None, None, None, None) == 0


def test_paged_decode_noalloc_rejects_more_than_its_scratch():
    # Non-null stand-in pointers: the size check refuses the request on the
    # host before any HIP call, so nothing is dereferenced.  1024 sequences x
    # 32 heads x 32 splits of 64 pages need 541 MB of partials (> 64 MiB).
    lib = af.load_library()
    mp = af.MaskParams(0, 0, None, 0)
    sp = af.ScoreParams(None, 1.0, 0.0)
    fake = 256
    rc = lib.attn_paged_decode_noalloc(fake, fake, fake, fake, fake, fake, fake, 1, 1024, 32, 8, 128,
                                       16, 2048, 1, 0.1, 0, ctypes.byref(mp), 0, ctypes.byref(sp), None)
    assert rc == -4
    msg = lib.attn_last_error().decode()
    assert "scratch" in msg and "67108864" in msg
    # the same validation as attn_paged_decode before that
    assert lib.attn_paged_decode_noalloc(None, None, None, None, None, None, None, 1, 2, 8, 2, 128, 16,
                                         4, 1, 0.1, 0, ctypes.byref(mp), 0, ctypes.byref(sp), None) == -1
    assert lib.attn_paged_decode_noalloc(fake, fake, fake, fake, fake, fake, fake, 1, 2, 8, 2, 64, 16,
                                         4, 1, 0.1, 0, ctypes.byref(mp), 0, ctypes.byref(sp), None) == -2
    assert lib.attn_paged_decode_noalloc(None, None, None, None, None, None, None, 1, 0, 8, 2, 128, 16,
                                         4, 1, 0.1, 0, ctypes.byref(mp), 0, ctypes.byref(sp), None) == 0


# ---- the binding refuses tensors that do not match the sizes it passes to C
# (CPU tensors: every shape check runs before the device check, so a refusal
# here names the shape, and a consistent call gets as far as the device check)

import torch  # noqa: E402


def _qkv(B=1, Hq=4, Hkv=2, S=32, D=64, dt=torch.bfloat16):
    return (torch.zeros(B, Hq, S, D, dtype=dt), torch.zeros(B, Hkv, S, D, dtype=dt),
            torch.zeros(B, Hkv, S, D, dtype=dt))


@pytest.mark.parametrize("change,what", [
    (dict(out=torch.zeros(1, 4, 31, 64, dtype=torch.bfloat16)), "out"),
    (dict(lse=torch.zeros(1, 4, 16)), "lse"),
    (dict(lse=torch.zeros(1, 4, 32, dtype=torch.float64)), "lse"),
    (dict(k=torch.zeros(2, 2, 32, 64, dtype=torch.bfloat16)), "k"),
    (dict(k=torch.zeros(1, 2, 32, 128, dtype=torch.bfloat16)), "k"),
    (dict(v=torch.zeros(1, 2, 16, 64, dtype=torch.bfloat16)), "v"),
    (dict(mask="document", doc_ids=torch.zeros(1, 16, dtype=torch.int32)), "doc_ids"),
    (dict(mask="document"), "doc_ids"),
    (dict(score="alibi", alibi_slopes=torch.zeros(3)), "alibi_slopes"),
])
def test_binding_fwd_refuses_mismatched_tensors(change, what):
    q, k, v = _qkv()
    kw = dict(change)
    k = kw.pop("k", k)
    v = kw.pop("v", v)
    with pytest.raises(ValueError, match=what):
        af.attn_fwd(q, k, v, **kw)


def test_binding_fwd_block_mask_shapes_and_device_check_last():
    q, k, v = _qkv(S=300)
    num = torch.zeros(1, 1, 3, dtype=torch.int32)
    idx = torch.zeros(1, 1, 3, 3, dtype=torch.int32)
    full = torch.zeros(1, 1, 3, 3, dtype=torch.uint8)
    with pytest.raises(ValueError, match="kv_num_blocks"):
        af.attn_fwd(q, k, v, block_mask=af.BlockMask(torch.zeros(1, 1, 2, dtype=torch.int32), idx, full,
                                                     128, 128))
    with pytest.raises(ValueError, match="kv_full"):
        af.attn_fwd(q, k, v, block_mask=af.BlockMask(num, idx, torch.zeros(1, 1, 3, 2, dtype=torch.uint8),
                                                     128, 128))
    with pytest.raises(ValueError, match="does not cover"):
        af.attn_fwd(q, k, v, block_mask=af.BlockMask(num[:, :, :2], idx[:, :, :2], None, 128, 128))
    with pytest.raises(ValueError, match="expected \\[1 or B"):
        af.attn_fwd(q, k, v, block_mask=af.BlockMask(num.expand(3, 1, 3).contiguous(),
                                                     idx.expand(3, 1, 3, 3).contiguous(), None, 128, 128))
    # consistent shapes: refused only because the tensors are not on a GPU
    with pytest.raises(ValueError, match="device"):
        af.attn_fwd(q, k, v, block_mask=af.BlockMask(num, idx, full, 128, 128))


def _dec_inputs(N=3, Hq=8, Hkv=2, D=128, pages=10, max_pages=4):
    return (torch.zeros(N, Hq, D, dtype=torch.bfloat16),
            torch.zeros(pages, Hkv, 16, D, dtype=torch.bfloat16),
            torch.zeros(pages, Hkv, 16, D, dtype=torch.bfloat16),
            torch.zeros(N, max_pages, dtype=torch.int32), torch.zeros(N, dtype=torch.int32))


@pytest.mark.parametrize("fn", ["attn_paged_decode", "attn_paged_decode_noalloc"])
@pytest.mark.parametrize("change,what", [
    (dict(page_table=torch.zeros(2, 4, dtype=torch.int32)), "page_table"),
    (dict(seq_lens=torch.zeros(4, dtype=torch.int32)), "seq_lens"),
    (dict(out=torch.zeros(3, 8, 64, dtype=torch.bfloat16)), "out"),
    (dict(lse=torch.zeros(3, 4)), "lse"),
    (dict(v_cache=torch.zeros(9, 2, 16, 128, dtype=torch.bfloat16)), "v_cache"),
    (dict(k_cache=torch.zeros(10, 2, 16, 64, dtype=torch.bfloat16),
          v_cache=torch.zeros(10, 2, 16, 64, dtype=torch.bfloat16)), "k_cache"),
    (dict(alibi_slopes=torch.zeros(4)), "alibi_slopes"),
    (dict(), "device"),
])
def test_binding_decode_refuses_mismatched_tensors(fn, change, what):
    q, kc, vc, table, lens = _dec_inputs()
    kw = dict(change)
    q = kw.pop("q", q)
    kc = kw.pop("k_cache", kc)
    vc = kw.pop("v_cache", vc)
    table = kw.pop("page_table", table)
    lens = kw.pop("seq_lens", lens)
    with pytest.raises(ValueError, match=what):
        getattr(af, fn)(q, kc, vc, table, lens, **kw)


@pytest.mark.parametrize("change,what", [
    (dict(dq=torch.zeros(1, 4, 32, 64, dtype=torch.bfloat16)), "dq"),
    (dict(dk=torch.zeros(1, 4, 32, 64)), "dk"),
    (dict(dv=torch.zeros(1, 2, 31, 64)), "dv"),
    (dict(lse=torch.zeros(1, 4, 31)), "lse"),
    (dict(out=torch.zeros(1, 4, 31, 64, dtype=torch.bfloat16)), "out"),
    (dict(dout=torch.zeros(1, 4, 32, 128, dtype=torch.bfloat16)), "dout"),
    (dict(mask="document", doc_ids=torch.zeros(2, 32, dtype=torch.int32)), "doc_ids"),
    (dict(), "device"),
])
def test_binding_bwd_refuses_mismatched_tensors(change, what):
    q, k, v = _qkv()
    kw = dict(change)
    out = kw.pop("out", torch.zeros_like(q))
    dout = kw.pop("dout", torch.zeros_like(q))
    lse = kw.pop("lse", torch.zeros(1, 4, 32))
    with pytest.raises(ValueError, match=what):
        af.attn_bwd(q, k, v, out, lse, dout, **kw)


def test_binding_build_block_mask_refuses_short_doc_ids():
    with pytest.raises(ValueError, match="doc_ids"):
        af.attn_build_block_mask("document", 1, 300, 300, doc_ids=torch.zeros(1, 200, dtype=torch.int32),
                                 device="cpu")
    with pytest.raises(ValueError, match="doc_ids"):
        af.attn_build_block_mask("document", 1, 300, 300, device="cpu")
