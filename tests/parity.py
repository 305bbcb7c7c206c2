"""Parity helpers: move a workloads.DecodeCase to the GPU, run the HIP library on
it, and compare with the float64 oracle under the stated tolerance.

Tolerance (written here, used by every GPU test):
  fp16 storage: max |gpu - ref| <= 2e-3 over all elements, and
                max |gpu - ref| / |ref| <= 1e-2 over elements with |ref| >= 2e-3
                (elements below 2e-3 are covered by the absolute bound; relative
                error is not meaningful near zero).
  bf16 storage: max |gpu - ref| <= 1e-2.
"""
from __future__ import annotations

import numpy as np
import torch

TOL = {"f16": {"atol": 2e-3, "rtol": 1e-2}, "bf16": {"atol": 1e-2, "rtol": None}}

_TORCH = {"f16": torch.float16, "bf16": torch.bfloat16}


def bits_to_device(bits: np.ndarray, dtype: str, device) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device).view(_TORCH[dtype])


def case_to_device(case, device, copies: int = 1):
    """Device tensors of a case.  ``copies`` > 1 adds extra K/V copies (list)."""
    dev = {"case": case, "q": bits_to_device(case.q, case.dtype, device)}
    dev["k"] = bits_to_device(case.k, case.dtype, device)
    dev["v"] = bits_to_device(case.v, case.dtype, device)
    if case.layout in ("paged", "paged_xsplit"):
        dev["block_table"] = torch.from_numpy(case.block_table).to(device)
        dev["ctx_lens"] = torch.from_numpy(case.ctx_lens).to(device)
    return dev


def run_case(dev, policy=None, out=None, workspace=None, k=None, v=None) -> np.ndarray:
    """Run the library on a device case; return the output as float64 numpy."""
    import decode_attention_08_amd as gq
    case = dev["case"]
    k = dev["k"] if k is None else k
    v = dev["v"] if v is None else v
    if case.layout == "paged":
        res = gq.decode(dev["q"], k, v, dev["block_table"], dev["ctx_lens"], scale=case.scale,
                        out=out, workspace=workspace, policy=policy)
    elif case.layout == "paged_xsplit":
        res = gq.decode_xsplit(dev["q"], k, v, dev["block_table"], dev["ctx_lens"],
                               scale=case.scale, out=out, workspace=workspace, policy=policy)
    else:
        res = gq.decode_contiguous(dev["q"], k, v, scale=case.scale, out=out,
                                   workspace=workspace, policy=policy)
    torch.cuda.synchronize()
    return res.float().cpu().numpy().astype(np.float64)


def errors(got: np.ndarray, ref: np.ndarray, atol: float):
    diff = np.abs(got - ref)
    max_abs = float(diff.max()) if diff.size else 0.0
    big = np.abs(ref) >= atol
    max_rel = float((diff[big] / np.abs(ref[big])).max()) if big.any() else 0.0
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    normwise = max_abs / scale if scale > 0 else max_abs
    return max_abs, max_rel, normwise


def assert_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    mask = ~np.isnan(ref)                      # rows the oracle was asked for
    g, r = got[mask], ref[mask]
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    tol = TOL[dtype]
    max_abs, max_rel, normwise = errors(g, r, tol["atol"])
    msg = (f"{what}: max_abs={max_abs:.3e} max_rel={max_rel:.3e} "
           f"normwise={normwise:.3e} (dtype {dtype})")
    assert max_abs <= tol["atol"], msg
    if tol["rtol"] is not None:
        assert max_rel <= tol["rtol"], msg
    return max_abs, max_rel, normwise
