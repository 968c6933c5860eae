"""Loader for tests/golden/hand_examples.json (hand-derived verification rounds)."""

import json
import os

import numpy as np

PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_examples.json")


def load():
    with open(PATH) as f:
        return json.load(f)


def sample_arrays(c):
    tgt = np.asarray(c["target"], np.float32)[None]
    K = tgt.shape[1] - 1
    V = tgt.shape[2]
    dr = np.asarray(c["draft"], np.float32).reshape(1, K, V)
    x = np.asarray(c["draft_tokens"], np.int32).reshape(1, K)
    ua = np.asarray(c["u_accept"], np.float32).reshape(1, K)
    us = np.asarray(c["u_sample"], np.float32).reshape(1, K + 1)
    return tgt, dr, x, ua, us


def greedy_arrays(c):
    tgt = np.asarray(c["target"], np.float32)[None]
    return tgt, np.asarray(c["draft_tokens"], np.int32).reshape(1, tgt.shape[1] - 1)


def tree_arrays(c):
    tgt = np.asarray(c["target"], np.float32)[None]
    return (tgt, np.asarray(c["node_tokens"], np.int32)[None],
            np.asarray(c["parents"], np.int32)[None])
