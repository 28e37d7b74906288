"""Parity at the layer's real sizes (hidden 7168, intermediate 3072, 48
experts, top-8): the decode, prefill and skewed configs through the same
nvfp4_moe_forward launch configuration bench.py times, against the full oracle
(per-expert work spread over CPU worker processes)."""
import time

import numpy as np
import pytest

import workloads as W
from fullsize import layer_inputs, make_pool, oracle_weights
from test_gpu_moe import compare_layer

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module")
def pool():
    p = make_pool()
    yield p
    p.close()
    p.join()


@pytest.fixture(scope="module")
def weights(pool):
    t0 = time.time()
    w = oracle_weights(W.PREFILL, pool)        # decode / prefill / skewed share them
    print(f"oracle weights: {time.time() - t0:.1f} s")
    return w


def _run(nv, cfg, weights, pool, label):
    t0 = time.time()
    L = layer_inputs(cfg, weights)
    g, r, st = compare_layer(nv, L, label, pool=pool)
    print(f"{label}: {time.time() - t0:.1f} s")
    return g, r, st


def test_decode_full_size(nv, weights, pool):
    _, _, st = _run(nv, W.DECODE, weights, pool, "decode full size")
    assert st["cos"] >= 0.9999


def test_prefill_full_size(nv, weights, pool):
    _, _, st = _run(nv, W.PREFILL, weights, pool, "prefill full size")
    assert st["cos"] >= 0.9999


def test_skewed_full_size(nv, weights, pool):
    g, _, st = _run(nv, W.SKEWED, weights, pool, "skewed full size")
    cnt = g["counts"]
    print("skewed histogram:", cnt.tolist())
    assert (cnt == 0).sum() >= 4, "skewed routing should leave at least 4 experts empty"
    assert st["cos"] >= 0.9999
