"""Shared helpers of the GPU parity tests (device transfer, seeded inputs, GEMM metrics).

Expected values always come from ``oracle/`` applied to the same input bytes the GPU receives.
"""
from __future__ import annotations

import functools
import sys

import numpy as np
import torch

import workloads as W
from oracle import activations as A

DEV = "cuda"

# GEMM tolerances (fp32 accumulation of exact fp16/e4m3 products, then one bf16 rounding)
REL_FRO = 1e-3      # relative Frobenius error
MAX_REL = 8e-3      # max |C - ref| / max |ref| after the bf16 cast


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_u8(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().cpu().numpy()


def dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def scalar(v) -> torch.Tensor:
    return torch.tensor([float(np.float32(v))], dtype=torch.float32, device=DEV)


@functools.lru_cache(maxsize=8)
def tensor_bits(cfg: int, name: str) -> np.ndarray:
    return W.generate(W.config(cfg).tensor(name))


def bf16_of(ref: np.ndarray) -> np.ndarray:
    return W.bf16_bits_to_f32(A.f64_to_bf16_bits(ref)).astype(np.float64)


def gemm_metrics(c: np.ndarray, ref: np.ndarray) -> dict:
    c = np.asarray(c, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    nref = np.linalg.norm(ref)
    mref = np.max(np.abs(ref))
    return {
        "rel_fro": float(np.linalg.norm(c - ref) / nref) if nref else float(np.linalg.norm(c)),
        "rel_fro_vs_bf16_ref": float(np.linalg.norm(c - bf16_of(ref)) / nref) if nref else 0.0,
        "max_rel": float(np.max(np.abs(c - ref)) / mref) if mref else float(np.max(np.abs(c))),
    }


def assert_gemm_f32(c: np.ndarray, ref: np.ndarray, what: str = ""):
    m = gemm_metrics(c, ref)
    say(what, "fp32 out", m)
    assert m["rel_fro"] <= REL_FRO, (what, m)


def assert_gemm_bf16(c: np.ndarray, ref: np.ndarray, what: str = ""):
    m = gemm_metrics(c, ref)
    say(what, "bf16 out", m)
    assert m["rel_fro_vs_bf16_ref"] <= REL_FRO, (what, m)
    assert m["max_rel"] <= MAX_REL, (what, m)


def sample_entries(m: int, n: int, count: int, seed: int):
    """Random (row, col) pairs plus the four corners and the last rows/cols (ragged tails)."""
    rng = np.random.default_rng(seed)
    r = rng.integers(0, m, count)
    c = rng.integers(0, n, count)
    extra_r = np.array([0, 0, m - 1, m - 1] + [m - 1 - i for i in range(16)])
    extra_c = np.array([0, n - 1, 0, n - 1] + [n - 1 - 3 * i % n for i in range(16)])
    return np.concatenate([r, extra_r]), np.concatenate([c, extra_c])


def gather(t: torch.Tensor, rows: np.ndarray, cols: np.ndarray) -> np.ndarray:
    ri = torch.from_numpy(rows).to(DEV)
    ci = torch.from_numpy(cols).to(DEV)
    return t[ri, ci].float().cpu().numpy().astype(np.float64)
