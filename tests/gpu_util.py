"""Helpers shared by the GPU tests: device transfer of bf16 bit arrays and tolerance checks."""
from __future__ import annotations

import numpy as np
import torch

import oracle

TOL = 1e-3  # max |out - ref| <= TOL * RMS(ref), per output buffer


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def dev_f32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def dev_i32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def assert_close(out, ref, what: str, tol: float = TOL):
    assert np.shape(out) == np.shape(ref), f"{what}: shape {np.shape(out)} vs {np.shape(ref)}"
    assert not np.isnan(np.asarray(out)).any(), f"{what}: NaN in output"
    err = oracle.max_rel_err(np.asarray(out, np.float64), ref)
    print(f"{what}: max|out-ref|/RMS(ref) = {err:.3e} over {np.size(ref)} elements", flush=True)
    assert err <= tol, f"{what}: max|out-ref|/RMS(ref) = {err:.3e} > {tol:.1e}"
    return err


def assert_exact(out, ref, what: str):
    out = np.asarray(out)
    ref = np.asarray(ref)
    assert out.shape == ref.shape, f"{what}: shape {out.shape} vs {ref.shape}"
    bad = np.argwhere(out != ref)
    assert bad.size == 0, f"{what}: {len(bad)} mismatches, first at {bad[0].tolist()}"


def log(msg: str):
    print(msg, flush=True)
