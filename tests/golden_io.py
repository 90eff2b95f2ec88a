"""Readers for the small text fixtures under tests/golden (values printed on the pages)."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return [l.split() for l in fh if l.strip() and not l.startswith("#")]


def attention_example():
    d = {l[0]: np.array(l[1:], dtype=np.float64) for l in _lines("attention_softmax_example.txt")}
    return d


def normalize_example():
    rows = _lines("normalize_keypoints_example.txt")
    kv = {r[0]: float(r[1]) for r in rows if r[0] in ("width", "height")}
    tab = np.array([r for r in rows if r[0] not in ("width", "height")], dtype=np.float64)
    return kv["width"], kv["height"], tab[:, :2], tab[:, 2:]


def sinkhorn_demo():
    rows = _lines("sinkhorn_demo_matrix.txt")
    S = np.array([r[1:] for r in rows if r[0] == "S"], dtype=np.float64)
    dust = float([r for r in rows if r[0] == "dust"][0][1])
    return S, dust


def confidence_threshold_example():
    """(layer, n_layers, threshold) rows of the page's adaptive-depth example."""
    return [(int(a), int(b), float(c)) for a, b, c in _lines("confidence_threshold_example.txt")]
