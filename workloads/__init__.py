"""Seeded synthetic inputs for the NVFP4 / MXFP8 linear-layer workloads.

This module only draws random numbers and rounds them to bf16 storage. It holds
none of the quantization or GEMM arithmetic, so both the CPU oracle and the HIP
path can be fed from it without sharing any of the method's code.

The shapes stand in for the Wan-2.1 attention and FFN projections that the
FastVideo nvfp4_qat_config.py page targets (its default FP4 layer list: to_q,
to_k, to_v, to_out, ffn.fc_in, ffn.fc_out). No checkpoint or dataset is used:
every tensor is drawn from a numpy PCG64 generator seeded with
``1000 * config + tensor_id`` (X=1, W=2, W2=3, outlier-channel permutation=4,
W3=5), in fp32, row chunk by row chunk, then rounded to bf16 with
round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Tuple

import numpy as np

ROW_CHUNK = 4096  # rows drawn per generator call; part of the recipe

TID_X, TID_W, TID_W2, TID_PERM, TID_W3 = 1, 2, 3, 4, 5


@dataclasses.dataclass(frozen=True)
class Tensor:
    """Recipe for one synthetic bf16 tensor."""
    name: str
    rows: int
    cols: int
    dist: str            # "normal" or "student_t4"
    std: float           # scale applied to the draw
    seed: int
    outlier_frac: float = 0.0   # fraction of columns multiplied by outlier_gain
    outlier_gain: float = 20.0
    perm_seed: int = 0


@dataclasses.dataclass(frozen=True)
class Config:
    idx: int
    name: str
    tensors: Tuple[Tensor, ...]
    gemms: Tuple[Tuple[str, str], ...]   # (activation tensor, weight tensor)
    fmt: str = "nvfp4"                   # "nvfp4" or "mxfp8"

    def tensor(self, name: str) -> Tensor:
        for t in self.tensors:
            if t.name == name:
                return t
        raise KeyError(name)


def _seed(cfg: int, tid: int) -> int:
    return 1000 * cfg + tid


def _x(cfg, rows, cols, dist="normal", outliers=0.0):
    return Tensor("X", rows, cols, dist, 1.0, _seed(cfg, TID_X), outliers, 20.0,
                  _seed(cfg, TID_PERM))


def _w(cfg, name, tid, rows, cols, std):
    return Tensor(name, rows, cols, "normal", std, _seed(cfg, tid))


M_TOK = 32760  # tokens per call in the Wan-shaped configurations

CONFIGS: Dict[int, Config] = {
    1: Config(1, "tiny NVFP4 linear 128x256x512",
              (_x(1, 128, 512), _w(1, "W", TID_W, 256, 512, 0.02)),
              (("X", "W"),)),
    2: Config(2, "Wan-1.3B attention projection 32760x1536x1536",
              (_x(2, M_TOK, 1536, outliers=0.01), _w(2, "W", TID_W, 1536, 1536, 0.02)),
              (("X", "W"),)),
    3: Config(3, "Wan-1.3B FFN fc_in 32760x8960x1536 -> GELU -> fc_out 32760x1536x8960",
              (_x(3, M_TOK, 1536, dist="student_t4"),
               _w(3, "W", TID_W, 8960, 1536, 0.02),
               _w(3, "W2", TID_W2, 1536, 8960, 0.02)),
              (("X", "W"), ("H", "W2"))),
    4: Config(4, "Wan-14B layers: to_q 32760x5120x5120, fc_in 32760x13824x5120, fc_out 32760x5120x13824",
              (_x(4, M_TOK, 5120, outliers=0.01),
               _w(4, "W", TID_W, 13824, 5120, 0.01),
               _w(4, "W2", TID_W2, 5120, 13824, 0.01),
               _w(4, "W3", TID_W3, 5120, 5120, 0.01)),
              (("X", "W"), ("H", "W2"), ("X", "W3"))),
    5: Config(5, "MXFP8 W8A8 at the Wan-14B FFN shape 32760x13824x5120",
              (_x(5, M_TOK, 5120, outliers=0.01), _w(5, "W", TID_W, 13824, 5120, 0.01)),
              (("X", "W"),), fmt="mxfp8"),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bit patterns.

    Inputs here are finite draws, so no NaN handling is needed.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to fp32 values (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def outlier_columns(t: Tensor) -> np.ndarray:
    """Columns that carry the outlier gain: floor(frac * cols) picks of a seeded permutation."""
    n = int(np.floor(t.outlier_frac * t.cols + 1e-9))
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    perm = np.random.Generator(np.random.PCG64(t.perm_seed)).permutation(t.cols)
    return np.sort(perm[:n])


def generate(t: Tensor, rows: int | None = None) -> np.ndarray:
    """Draw tensor ``t`` as bf16 bits, shape [rows, cols] (uint16).

    ``rows`` (default: all) takes only the first rows; because the draw is made
    in fixed row chunks from one generator stream, the first rows are the same
    whatever ``rows`` is.
    """
    rows = t.rows if rows is None else min(rows, t.rows)
    rng = np.random.Generator(np.random.PCG64(t.seed))
    out = np.empty((rows, t.cols), dtype=np.uint16)
    cols = outlier_columns(t)
    for r0 in range(0, rows, ROW_CHUNK):
        r1 = min(r0 + ROW_CHUNK, t.rows)
        if t.dist == "normal":
            v = rng.standard_normal((r1 - r0, t.cols), dtype=np.float32)
        elif t.dist == "student_t4":
            v = rng.standard_t(4.0, (r1 - r0, t.cols)).astype(np.float32)
        else:
            raise ValueError(t.dist)
        if t.std != 1.0:
            v *= np.float32(t.std)
        if cols.size:
            v[:, cols] *= np.float32(t.outlier_gain)
        n = min(r1, rows) - r0
        out[r0:r0 + n] = f32_to_bf16_bits(v[:n])
    return out


def small_case(rows: int, cols: int, seed: int, std: float = 1.0,
               dist: str = "normal", outlier_frac: float = 0.0) -> np.ndarray:
    """A free-form seeded tensor for tests (same recipe, arbitrary shape)."""
    return generate(Tensor("T", rows, cols, dist, std, seed, outlier_frac, 20.0, seed + 7))


def special_values_block(seed: int, rows: int, cols: int) -> np.ndarray:
    """bf16 tensor mixing zeros, signed zeros, tiny, huge and tie-prone values.

    Used for edge-case parity: whole 16-blocks of zeros, blocks of -0.0, blocks whose
    amax saturates the e4m3 scale, subnormal bf16 inputs and exact e2m1 grid points.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    v = rng.standard_normal((rows, cols), dtype=np.float32)
    nb = cols // 16
    kind = rng.integers(0, 8, size=(rows, nb))
    blocks = v[:, : nb * 16].reshape(rows, nb, 16)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float32)
    for k in range(8):
        sel = kind == k
        if k == 0:
            blocks[sel] = 0.0
        elif k == 1:
            blocks[sel] = -0.0
        elif k == 2:
            blocks[sel] *= np.float32(1e4)       # saturating scales at gsf=1
        elif k == 3:
            blocks[sel] *= np.float32(1e-39)     # bf16 subnormals
        elif k == 4:
            g = grid[rng.integers(0, 8, size=(int(sel.sum()), 16))]
            sg = np.where(rng.integers(0, 2, size=g.shape) == 1, -1, 1).astype(np.float32)
            blocks[sel] = g * sg                 # exact grid points, amax often 6
        elif k == 5:
            blocks[sel] *= np.float32(1e-6)      # tiny blocks: scale underflows to 0
        elif k == 6:
            blocks[sel] *= np.float32(3e3)       # large: near the 448*6 boundary at gsf=1
        # k == 7: plain N(0,1)
    v[:, : nb * 16] = blocks.reshape(rows, nb * 16)
    return f32_to_bf16_bits(v)


def nonfinite_block(seed: int, rows: int, cols: int) -> np.ndarray:
    """bf16 bits: ``special_values_block`` with infinities and NaNs written in.

    About 1 % of the elements become +inf, -inf, a quiet NaN (0x7FC0 / 0xFFC0) or a signalling NaN
    pattern (0x7F81 / 0xFF81); row 0 is all NaN, row 1 holds one +inf, row 2 one -inf among zeros.
    """
    b = special_values_block(seed, rows, cols)
    rng = np.random.Generator(np.random.PCG64(seed + 1))
    hit = rng.random((rows, cols)) < 0.01
    pats = np.array([0x7F80, 0xFF80, 0x7FC0, 0xFFC0, 0x7F81, 0xFF81], dtype=np.uint16)
    b[hit] = pats[rng.integers(0, pats.size, size=int(hit.sum()))]
    if rows > 2:
        b[0] = 0x7FC0
        b[1] = 0
        b[1, cols // 3] = 0x7F80
        b[2] = 0
        b[2, cols - 1] = 0xFF80
    return b


def config(idx: int) -> Config:
    return CONFIGS[idx]


def all_configs() -> List[Config]:
    return [CONFIGS[i] for i in sorted(CONFIGS)]
