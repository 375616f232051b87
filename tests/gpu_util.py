"""Helpers shared by the GPU parity tests."""

from __future__ import annotations

import sys

import numpy as np
import torch

import workloads as W

# Pass criteria: worst per-(row, head) relative error ("worst relative error ...
# limit 1e-3", "perf(gfx1100): share Q8 KV scans across verifier rows", Kernel
# evidence) and the largest error as a fraction of the output scale ("error vs
# FP64 (output scale ...)", "hip: gfx12 (RDNA4) WMMA kernel for the int8-KV QSA
# prompt attention", Measurements).
E_ROW_TOL = 1e-3
E_SCALE_TOL = 1e-5


def note(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(inp: W.Inputs, device="cuda"):
    return (
        torch.from_numpy(np.ascontiguousarray(inp.q)).to(device),
        torch.from_numpy(inp.k_codes).to(device),
        torch.from_numpy(inp.k_scales).to(device),
        torch.from_numpy(inp.v_codes).to(device),
        torch.from_numpy(inp.v_scales).to(device),
    )


def errors(got, ref):
    """(E_row, E_scale) of got vs ref, both [rows][heads][hd]."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = np.abs(got - ref)
    row_scale = np.max(np.abs(ref), axis=-1)
    e_row = float(np.max(np.max(diff, axis=-1) / np.maximum(row_scale, 1e-300)))
    e_scale = float(np.max(diff) / max(np.max(np.abs(ref)), 1e-300))
    return e_row, e_scale


# (test id, what, E_row, E_scale) of every comparison in this session, for the
# terminal summary
PARITY = []


def assert_parity(got, ref, what: str, e_row_tol=E_ROW_TOL, e_scale_tol=E_SCALE_TOL):
    import os

    e_row, e_scale = errors(got, ref)
    note(f"  {what}: E_row={e_row:.3e} E_scale={e_scale:.3e}")
    PARITY.append((os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0], what, e_row, e_scale))
    assert np.all(np.isfinite(np.asarray(got))), f"{what}: non-finite output"
    assert e_row <= e_row_tol, f"{what}: E_row {e_row:.3e} > {e_row_tol}"
    assert e_scale <= e_scale_tol, f"{what}: E_scale {e_scale:.3e} > {e_scale_tol}"
    return e_row, e_scale
