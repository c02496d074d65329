"""Writes the stored expected values under tests/golden/ by calling only the oracle.

Run from the repository root: ``python tests/golden/make_golden.py``.  The
fixtures guard the oracle against unintended changes; a change of any stored
value must name, in its commit message, the passage or reading that justifies it.
"""
import hashlib
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
from mxfp4_bit_weight_amd import workloads as W  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))


def sha(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def single_linear(fmt: int) -> dict:
    """Single linear, seed 0: W 256x512 ~ N(0, 0.02), x 1x512 ~ N(0, 1), LoRA r = 16."""
    w, x, a, b = W.linear_inputs(0, 256, 512, 1)
    codes, scales, st = O.quantize(fmt, w)
    y = O.linear(fmt, x, codes, scales, st, a, b)
    return {
        "format": "nvfp4" if fmt == O.NVFP4 else "mxfp4",
        "inputs_sha256": {"w": sha(w), "x": sha(x), "a": sha(a), "b": sha(b)},
        "codes_sha256": sha(codes),
        "scales_sha256": sha(scales),
        "tensor_scale_hex": float(st).hex(),
        "scales_row0": scales[0].tolist(),
        "codes_row0_first16": codes[0, :16].tolist(),
        "y_first8_hex": [float(v).hex() for v in y[0, :8]],
        "y_sha256": sha(y),
    }


def main():
    out = {"single_linear_256x512_seed0": {"nvfp4": single_linear(O.NVFP4),
                                            "mxfp4": single_linear(O.MXFP4)}}
    path = os.path.join(HERE, "single_linear_seed0.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
        f.write("\n")
    print(path)


if __name__ == "__main__":
    main()
