"""Write the shared 2D Lloyd-Max codebook files (run once, offline, on CPU).

    python -m oracle.make_codebooks [K ...]

For each K the script trains the codebook with ``oracle.lloyd.train`` on
2^16 samples of the unit circular Gaussian (seed 1, 50 rounds) and writes

    vector_codebook_codec_amd/codebooks/qamw_K<K>.f32   K x 2 float32, little-endian,
                                                        interleaved (cx, cy)
    vector_codebook_codec_amd/codebooks/qamw_K<K>.json  K, seed, n, iters, the
                                                        distortion history, numpy
                                                        version and sha256 of .f32

The codebook is an input of the codec -- the pages train it once on
synthetic samples, not per checkpoint -- so both the oracle's tests and the
GPU path read these files.  This script calls only ``oracle`` and the input
generators in ``workloads``.
"""
from __future__ import annotations

import hashlib
import json
import os
import sys
import time

import numpy as np

from oracle import lloyd
import workloads

DEFAULT_KS = (2, 4, 16, 128, 256, 1024, 2048, 4096)
N_SAMPLES = 1 << 16
SEED = 1
ITERS = 50
OUT_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                       "vector_codebook_codec_amd", "codebooks")


def main(ks) -> None:
    os.makedirs(OUT_DIR, exist_ok=True)
    X = workloads.gaussian_samples(N_SAMPLES, SEED)
    for K in ks:
        t0 = time.time()
        C, hist = lloyd.train(X, K, ITERS)
        raw = np.ascontiguousarray(C.astype(np.float32), dtype="<f4").tobytes()
        base = os.path.join(OUT_DIR, f"qamw_K{K}")
        with open(base + ".f32", "wb") as f:
            f.write(raw)
        meta = {
            "K": K, "seed": SEED, "n_samples": N_SAMPLES, "iters": ITERS,
            "distribution": "N(0, I_2)", "init": "first K samples",
            "distortion_history": hist,
            "numpy_version": np.__version__,
            "sha256": hashlib.sha256(raw).hexdigest(),
        }
        with open(base + ".json", "w") as f:
            json.dump(meta, f, indent=1)
        print(f"K={K}: D={hist[-1]:.6g} ({time.time() - t0:.1f} s)", flush=True)


if __name__ == "__main__":
    main([int(k) for k in sys.argv[1:]] or DEFAULT_KS)
