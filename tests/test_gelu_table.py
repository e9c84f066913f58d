"""The GELU lookup table compiled into the kernels (csrc/gelu_table.inc): reproducible from its
generator, and equal on every one of its 4608 inputs to the oracle's GELU rounded once to bf16."""
import os
import re
import subprocess
import sys

import numpy as np

from oracle import activations as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_scaled_precision_nvfp4_amd", "csrc")


def _entries(text: str) -> np.ndarray:
    body = text.split("{", 1)[1]
    return np.array([int(v, 16) for v in re.findall(r"0x([0-9A-F]{4})", body)], dtype=np.uint16)


def test_committed_table_is_what_the_generator_writes(tmp_path):
    out = tmp_path / "gelu_table.inc"
    subprocess.run([sys.executable, os.path.join(CSRC, "gen_gelu_table.py"), str(out)], check=True,
                   timeout=120)
    assert out.read_text() == open(os.path.join(CSRC, "gelu_table.inc")).read()


def test_table_equals_the_oracle_gelu():
    v = _entries(open(os.path.join(CSRC, "gelu_table.inc")).read())
    assert v.size == 4608
    i = np.arange(4608)
    s = (i >= 2304).astype(np.int64)
    x_bits = ((s << 15) + (115 << 7) + i - s * 2304).astype(np.uint16)
    assert np.array_equal(v, A.gelu_tanh_bf16_bits(x_bits))
    # the range: 2^-12 .. just below 2^6, both signs
    xf = (x_bits.astype(np.uint32) << 16).view(np.float32)
    assert xf[0] == 2.0 ** -12 and xf[2303] < 64.0 and xf[2304] == -(2.0 ** -12)
