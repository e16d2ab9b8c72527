"""attn_paged_decode_noalloc (the decode entry point that allocates nothing,
its split partials in the library's fixed per-GPU scratch) against
attn_paged_decode (caller workspace), through the C ABI: two calls in a row,
the second with a smaller input, each equal to the workspace call's result
and within the parity bars of the oracle on sampled sequences."""

import math

import numpy as np
import pytest
import torch

import attention_fa2_fwd_amd as af
import oracle
import workloads
from gpu_util import announce, compare, f64, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]


def _both(inp, **kw):
    dev = torch.device("cuda")
    args = tuple(inp[n].to(dev) for n in ("q", "k_cache", "v_cache", "page_table", "seq_lens"))
    n, hq, d = args[0].shape
    out_a = torch.empty_like(args[0])
    lse_a = torch.empty((n, hq), dtype=torch.float32, device=dev)
    out_b = torch.full_like(args[0], float("nan"))
    lse_b = torch.full((n, hq), float("nan"), dtype=torch.float32, device=dev)
    af.attn_paged_decode(*args, out=out_a, lse=lse_a, **kw)
    af.attn_paged_decode_noalloc(*args, out=out_b, lse=lse_b, **kw)
    torch.cuda.synchronize()
    return args, (out_a, lse_a), (out_b, lse_b)


def _oracle_rows(args, seqs, scale, score=oracle.SCORE_NONE, window=0):
    q, kc, vc, table, seq_lens = args
    table = table.cpu().numpy()
    lengths = seq_lens.cpu().numpy()
    o_ref = np.zeros((len(seqs), q.shape[1], q.shape[2]))
    l_ref = np.zeros((len(seqs), q.shape[1]))
    mask = oracle.MaskSpec(oracle.MASK_SLIDING, window=window) if window else None
    for i, s in enumerate(seqs):
        L = int(lengths[s])
        pages = table[s, :(L + 15) // 16]
        pid = torch.from_numpy(pages.astype(np.int64)).to(kc.device)
        kp = kc.index_select(0, pid).cpu()
        vp = vc.index_select(0, pid).cpu()
        local = np.arange(len(pages), dtype=np.int32)[None, :]
        kw = {} if mask is None else {"mask": mask}
        o1, l1 = oracle.paged_decode_ref(f64(q[s:s + 1]), f64(kp), f64(vp), local,
                                         np.array([L], dtype=np.int32), scale,
                                         oracle.ScoreSpec(score), **kw)
        o_ref[i], l_ref[i] = o1[0], l1[0]
    return o_ref, l_ref


def test_noalloc_decode_two_calls_second_smaller():
    dev = torch.device("cuda")
    # Call 1: the 64-sequence workload (33.8 MB of partials in the scratch).
    w = workloads.PAGED_DECODE
    announce("noalloc decode call 1: 64-sequence workload, generating")
    inp = workloads.decode_inputs(w, device=dev)
    scale = 1.0 / math.sqrt(w.D)
    announce("noalloc decode call 1: run")
    args, (oa, la), (ob, lb) = _both(inp, scale=scale)
    assert torch.equal(oa, ob) and torch.equal(la, lb), "noalloc differs from the workspace call"
    seqs = [0, 31, 63, int(np.argmax(inp["lengths"]))]
    o_ref, l_ref = _oracle_rows(args, seqs, scale)
    compare(f64(ob)[seqs], f64(lb)[seqs], o_ref, l_ref, torch.bfloat16, "noalloc call 1")
    del inp, args, oa, la, ob, lb

    # Call 2: a smaller input on the same scratch (5 sequences, window + ALiBi);
    # whatever call 1 left there must not show through.
    announce("noalloc decode call 2: 5 sequences, window 300 + alibi")
    small = workloads.DecodeWorkload("noalloc_small", 5, 8, 2, 128, max_pages=80, seed=3)
    inp = workloads.decode_inputs(small, device="cpu", lengths=np.array([1, 17, 300, 1100, 1280]))
    args, (oa, la), (ob, lb) = _both(inp, scale=scale, mask="sliding", window=300, score="alibi")
    assert torch.equal(oa, ob) and torch.equal(la, lb), "noalloc differs from the workspace call"
    seqs = list(range(5))
    o_ref, l_ref = _oracle_rows(args, seqs, scale, oracle.SCORE_ALIBI, window=300)
    compare(f64(ob), f64(lb), o_ref, l_ref, torch.bfloat16, "noalloc call 2")


def test_noalloc_decode_rejects_more_than_its_scratch():
    dev = torch.device("cuda")
    # 1024 sequences x 32 heads x 32 splits of 2048 pages: 541 MB of partials.
    q = torch.zeros((1024, 32, 128), dtype=torch.bfloat16, device=dev)
    kc = torch.zeros((1, 8, 16, 128), dtype=torch.bfloat16, device=dev)
    table = torch.zeros((1024, 2048), dtype=torch.int32, device=dev)
    lens = torch.ones((1024,), dtype=torch.int32, device=dev)
    announce("noalloc decode: oversized request")
    with pytest.raises(af.AttnError) as e:
        af.attn_paged_decode_noalloc(q, kc, kc, table, lens)
    assert e.value.code == -4
    assert "scratch" in str(e.value)
