"""Shared helpers of the GPU tests: move a workloads Case to the device, run the
C-ABI path through the binding, compare with the oracle."""

from __future__ import annotations

import sys

import numpy as np
import torch

import speculative_decoding_mla_amd as mv
from oracle import bf16_bits_to_f64, oracle_case

OUT_TOL = 1e-2  # max-abs on out when |out| < 4 (bf16 half-ulp there is <= 7.8e-3)
LSE_TOL = 1e-3


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def bf16(u16: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16)


def device_case(case, dev="cuda"):
    return dict(
        q=bf16(case.q).to(dev),
        kv=bf16(case.kv).to(dev),
        page_table=torch.from_numpy(np.ascontiguousarray(case.page_table, dtype=np.int32)).to(dev),
        seq_lens=torch.from_numpy(np.ascontiguousarray(case.seq_lens, dtype=np.int32)).to(dev),
        tree_parent=torch.from_numpy(np.ascontiguousarray(case.tree_parent, dtype=np.int32)).to(dev),
    )


def run_gpu(case, nsplit: int | None = None, dc=None, workspace=None):
    """One verify call on the GPU. Returns (out bits uint16, lse float32, device error word)."""
    nsplit = case.nsplit if nsplit is None else nsplit
    dc = dc or device_case(case)
    b, t, h, _ = case.q.shape
    out = torch.empty((b, t, h, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((b, t, h), dtype=torch.float32, device="cuda")
    if workspace is None:
        desc = mv.desc_for(dc["q"], dc["kv"], dc["page_table"], page_size=case.page_size, nsplit=nsplit,
                           sm_scale=case.sm_scale)
        workspace = mv.alloc_workspace(desc)
    mv.verify_attention(dc["q"], dc["kv"], dc["page_table"], dc["seq_lens"], dc["tree_parent"], out, lse,
                        workspace, page_size=case.page_size, nsplit=nsplit, sm_scale=case.sm_scale)
    torch.cuda.synchronize()
    out_bits = out.view(torch.int16).cpu().numpy().view(np.uint16)
    return out_bits, lse.cpu().numpy(), mv.device_error(workspace)


def check_parity(case, out_bits, lse, ref=None, label=""):
    """out within OUT_TOL (or one bf16 ulp where |out| >= 4) and lse within
    LSE_TOL of the oracle; returns the observed maxima."""
    ref_out, ref_lse = oracle_case(case) if ref is None else ref
    out = bf16_bits_to_f64(out_bits)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse)), label
    err = np.abs(out - ref_out)
    # one bf16 ulp at the reference magnitude, for the rare |out| >= 4
    ulp = np.where(np.abs(ref_out) >= 4, 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref_out), 1e-30))) - 7), 0)
    tol = np.maximum(OUT_TOL, ulp)
    e_out = float(err.max())
    e_lse = float(np.abs(lse.astype(np.float64) - ref_lse).max())
    assert np.all(err <= tol), f"{label}: out max-abs error {e_out}"
    assert e_lse <= LSE_TOL, f"{label}: lse max-abs error {e_lse}"
    return e_out, e_lse
