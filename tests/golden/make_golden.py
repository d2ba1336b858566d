"""Writes tests/golden/tiny_layer.json from the CPU oracle alone.

The fixture freezes the oracle's routing, permutation and output for the
tiny layer (hidden 256, 8 experts, top-2, intermediate 512, group 64,
16 tokens, seed 0) so later edits of the oracle's arithmetic show up as a
diff.  Run: python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import moe_inputs as MI  # noqa: E402
import oracle as O  # noqa: E402


def tiny_layer():
    cfg = MI.TINY
    T = cfg.T[0]
    x = MI.gen_x(cfg, T)
    wr = MI.gen_router(cfg)
    blobs = [O.pack_expert(*MI.gen_expert(cfg, 0, e), cfg.g) for e in range(cfg.E)]
    r = O.moe_layer(x, wr, blobs, cfg.H, cfg.I, cfg.E, cfg.k, cfg.g)
    return cfg, blobs, r


def main():
    cfg, blobs, r = tiny_layer()
    doc = {
        "config": "tiny: H=256 E=8 k=2 I=512 g=64 T=16 seed 0",
        "written_by": "tests/golden/make_golden.py (oracle only)",
        "blob_sha256": [hashlib.sha256(b.tobytes()).hexdigest() for b in blobs],
        "idx": r["idx"].tolist(),
        "w": [float(v) for v in r["w"].reshape(-1)],
        "counts": r["counts"].tolist(),
        "offsets": r["offsets"].tolist(),
        "perm": r["perm"].tolist(),
        "out_f16_bits_sha256": hashlib.sha256(r["out"].view(np.uint16).tobytes()).hexdigest(),
        "out_row0_first8": [float(v) for v in r["out"][0, :8].astype(np.float64)],
    }
    with open(os.path.join(HERE, "tiny_layer.json"), "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
