"""Shared helpers of the GPU parity tests: tolerances, conversions, case
labels printed (and flushed) before each GPU step."""

import sys

import numpy as np
import pytest
import torch

# Tolerances of the parity contract: bf16 inputs O max-abs <= 1e-2 and
# mean-abs <= 1e-3; fp32 inputs O <= 1e-5 (both norms); LSE max-abs <= 1e-3.
TOL = {
    torch.bfloat16: dict(o_max=1e-2, o_mean=1e-3, lse=1e-3),
    torch.float32: dict(o_max=1e-5, o_mean=1e-5, lse=1e-3),
}


def have_gpu():
    return torch.cuda.is_available()


requires_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def announce(msg: str):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


# Relative error of rounding a real number to bf16 (round to nearest even,
# 8 significant bits): at most half a unit in the last place, 2^-9.
BF16_ROUND_REL = 2.0 ** -9


def compare(o_gpu, lse_gpu, o_ref, lse_ref, dtype, label="", out_rounding=False):
    """Element-wise comparison against the oracle; returns the error summary.

    out_rounding: the output was rounded to bf16 after the computation; the
    bound then also admits that final rounding, BF16_ROUND_REL * |O|, on top
    of the tolerance (the same values before rounding are gated separately at
    the plain tolerance)."""
    tol = TOL[dtype]
    o = f64(o_gpu) if isinstance(o_gpu, torch.Tensor) else o_gpu
    l = f64(lse_gpu) if isinstance(lse_gpu, torch.Tensor) else lse_gpu
    assert o.shape == o_ref.shape, (o.shape, o_ref.shape)
    assert np.all(np.isfinite(o)), f"{label}: non-finite output"
    err = np.abs(o - o_ref)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(l), fin), f"{label}: -inf LSE pattern differs"
    lerr = np.abs(l[fin] - lse_ref[fin]) if fin.any() else np.zeros(1)
    summary = dict(o_max=float(err.max()), o_mean=float(err.mean()), lse_max=float(lerr.max()))
    print(f"{label}: {summary}", flush=True)
    if out_rounding:
        excess = err - (tol["o_max"] + BF16_ROUND_REL * np.abs(o_ref))
        summary["o_max_beyond_rounding"] = float(excess.max())
        assert summary["o_max_beyond_rounding"] <= 0.0, f"{label}: {summary}"
    else:
        assert summary["o_max"] <= tol["o_max"], f"{label}: {summary}"
    assert summary["o_mean"] <= tol["o_mean"], f"{label}: {summary}"
    assert summary["lse_max"] <= tol["lse"], f"{label}: {summary}"
    return summary


def mask_spec(mask: str, window=0, prefix_len=0, doc_ids=None):
    """The oracle's MaskSpec for a mask name of the binding ("&" joins the
    kinds of an intersection)."""
    import oracle
    import workloads
    doc = None if doc_ids is None else (doc_ids.cpu().numpy() if hasattr(doc_ids, "cpu") else doc_ids)
    if "&" in mask:
        kinds = tuple(workloads.MASK_NAMES[p] for p in mask.split("&"))
        return oracle.MaskSpec(oracle.MASK_AND, window=window, prefix_len=prefix_len, doc_ids=doc,
                               and_kinds=kinds)
    return oracle.MaskSpec(workloads.MASK_NAMES[mask], window=window, prefix_len=prefix_len, doc_ids=doc)


def has_document(mask: str) -> bool:
    return "document" in mask.split("&")
