"""Write the shared 2D Lloyd-Max codebook files (run once, offline, on CPU).

    python -m oracle.make_codebooks [K ...]
    python -m oracle.make_codebooks --polar

For each K the script trains the codebook with ``oracle.lloyd.train`` on
2^16 samples of the unit circular Gaussian (seed 1, 50 rounds) and writes

    vector_codebook_codec_amd/codebooks/qamw_K<K>.f32   K x 2 float32, little-endian,
                                                        interleaved (cx, cy)
    vector_codebook_codec_amd/codebooks/qamw_K<K>.json  K, seed, n, iters, the
                                                        distortion history, numpy
                                                        version and sha256 of .f32

and, for the polar baseline (``oracle.polar``), for each split Ka x Kp

    polar_A<Ka>_P<Kp>.f32         decode table, Ka Kp x 2 float32 (entry ia Kp + ip)
    polar_A<Ka>_P<Kp>_levels.f32  Ka amplitude levels, float32, ascending
    polar_A<Ka>_P<Kp>_dirs.f32    Kp x 2 float32 unit directions (cos, sin)
    polar_A<Ka>_P<Kp>.json        the fp64 levels, solver iterations, sha256s

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

from oracle import lloyd, polar
import workloads

DEFAULT_KS = (2, 4, 16, 128, 256, 1024, 2048, 4096)
# 7, 8 and 11 bits per pair at their least-distortion splits, plus small and
# degenerate splits (one level, one direction) for the tests
DEFAULT_POLAR = ((8, 16), (8, 32), (32, 64), (16, 256), (1, 8), (2, 2), (4, 1), (4, 8))
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


def f32_bytes(a) -> bytes:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32), dtype="<f4").tobytes()


def main_polar(splits) -> None:
    os.makedirs(OUT_DIR, exist_ok=True)
    for Ka, Kp in splits:
        a, iters = polar.rayleigh_lloyd_max(Ka)
        u = polar.phase_directions(Kp)
        files = {"table": polar.product_table(a, u), "levels": a, "dirs": u}
        base = os.path.join(OUT_DIR, f"polar_A{Ka}_P{Kp}")
        sha = {}
        for key, arr in files.items():
            raw = f32_bytes(arr)
            name = base + (".f32" if key == "table" else f"_{key}.f32")
            with open(name, "wb") as f:
                f.write(raw)
            sha[key] = hashlib.sha256(raw).hexdigest()
        meta = {
            "Ka": Ka, "Kp": Kp, "K": Ka * Kp,
            "amplitude": "Lloyd-Max on Rayleigh(1), closed-form cell means",
            "levels_f64": [float(v) for v in a], "solver_iterations": iters,
            "phase": "angles 2 pi j / Kp",
            "numpy_version": np.__version__, "sha256": sha,
        }
        with open(base + ".json", "w") as f:
            json.dump(meta, f, indent=1)
        print(f"polar {Ka}x{Kp}: {iters} Lloyd-Max steps", flush=True)


if __name__ == "__main__":
    if sys.argv[1:2] == ["--polar"]:
        main_polar(DEFAULT_POLAR)
    else:
        main([int(k) for k in sys.argv[1:]] or DEFAULT_KS)
