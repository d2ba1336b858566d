"""Golden fixtures: the pages' worked byte arithmetic, and the frozen oracle
output of the tiny layer (written by tests/golden/make_golden.py, which calls
only the oracle)."""
import hashlib
import json
import os

import numpy as np

import oracle as O

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_pages_bytes_formula():
    doc = json.load(open(os.path.join(GOLD, "pages_worked_examples.json")))
    for c in doc["cases"]:
        assert c["params"] * c["bits"] // 8 == c["bytes"]
    # the blob of an expert obeys the same formula plus one fp16 scale per
    # block of g weights: H=2048, I=1024, g=128
    P = 3 * 2048 * 1024
    assert O.blob_layout(2048, 1024, 128)[1] == P * 4 // 8 + P // 128 * 2


def test_tiny_layer_regression():
    from tests.golden.make_golden import tiny_layer
    doc = json.load(open(os.path.join(GOLD, "tiny_layer.json")))
    cfg, blobs, r = tiny_layer()
    assert [hashlib.sha256(b.tobytes()).hexdigest() for b in blobs] == doc["blob_sha256"]
    assert r["idx"].tolist() == doc["idx"]
    assert [float(v) for v in r["w"].reshape(-1)] == doc["w"]
    assert r["counts"].tolist() == doc["counts"]
    assert r["offsets"].tolist() == doc["offsets"]
    assert r["perm"].tolist() == doc["perm"]
    assert hashlib.sha256(r["out"].view(np.uint16).tobytes()).hexdigest() == \
        doc["out_f16_bits_sha256"]
