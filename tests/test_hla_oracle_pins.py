"""Pins of the HLA composition oracle (``oracle/hla.py``), CPU only.

The pages print no worked numbers for the query-conditioned composition, so
each pin is a special case the HLA note fixes, checked against oracle
functions that are pinned on their own (``tests/test_oracle_pins.py``):

* all gates 1: the native recurrence (HLA note, "Core method": w = 1 restores
  the native behaviour);
* all gates 0: every history chunk skipped, so each query sees its own chunk
  from a zero state (w = 0: the chunk is as if absent);
* two chunks: the queries of the second chunk are affine in the shared gate;
* three chunks: explicit composition of the chunk pairs from the C oracle's
  summaries, then the current chunk's prefix by the C recurrence;
* the inference threshold: gates below it act as 0, gates at it are kept
  (step 7).
A dropped (1 - w) I term, a gate applied to the wrong chunk, a reversed
history order or a missing current-chunk prefix each fails one of them.
"""
import numpy as np
import pytest

import oracle
from oracle import hla as hla_oracle
import workloads


def _inputs(T, dk, dv, r_ab, r_kv, decay="channel", seed=0, lead=(1, 2)):
    raw = workloads.generic_raw(lead[0], lead[1], T, dk, dv, r_ab, r_kv, "fp32", decay, seed=seed)
    return raw


def _run(raw, gates, chunk, theta=0.0):
    return hla_oracle.hla(raw["q"], raw["K"], raw["V"], raw["log_decay"], raw["A"], raw["B"], gates, chunk, theta)


def _gates(raw, chunk, value):
    lead = raw["q"].shape[:-2]
    T = raw["q"].shape[-2]
    return np.full(lead + (T, -(-T // chunk)), value, dtype=np.float64)


@pytest.mark.parametrize("T,chunk,r_ab,r_kv,decay", [(40, 8, 2, 1, "channel"), (37, 16, 1, 2, "scalar"),
                                                      (24, 5, 0, 1, "channel")])
def test_all_gates_one_is_native_recurrence(T, chunk, r_ab, r_kv, decay):
    raw = _inputs(T, 8, 6, r_ab, r_kv, decay, seed=T)
    out = _run(raw, _gates(raw, chunk, 1.0), chunk)
    ref, _ = oracle.generic(raw["q"], raw["K"], raw["V"], raw["log_decay"], raw["A"], raw["B"])
    assert np.abs(out - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


def test_all_gates_zero_is_chunk_local():
    T, chunk = 30, 8
    raw = _inputs(T, 8, 5, 2, 1, seed=3)
    out = _run(raw, _gates(raw, chunk, 0.0), chunk)
    ref = np.empty_like(out)
    for j in range(-(-T // chunk)):
        sl = slice(j * chunk, min(T, (j + 1) * chunk))
        part = {k: (None if v is None else v[:, :, sl]) for k, v in raw.items()}
        ref[:, :, sl], _ = oracle.generic(part["q"], part["K"], part["V"], part["log_decay"], part["A"], part["B"])
    assert np.abs(out - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


def test_two_chunks_affine_in_gate():
    T, chunk, w = 20, 10, 0.3
    raw = _inputs(T, 6, 4, 2, 1, seed=5)
    o0 = _run(raw, _gates(raw, chunk, 0.0), chunk)
    o1 = _run(raw, _gates(raw, chunk, 1.0), chunk)
    ow = _run(raw, _gates(raw, chunk, w), chunk)
    # the first chunk has no history: the gate does not reach it
    assert np.array_equal(ow[:, :, :chunk], o0[:, :, :chunk])
    mix = (1.0 - w) * o0 + w * o1
    assert np.abs(ow - mix).max() <= 1e-12 * np.abs(o1).max()


def test_three_chunks_explicit_composition():
    """Queries of chunk 2 with gates (w0, w1) on chunks 0 and 1:
    S = ((1 - w1) I + w1 A_1)(w0 B_0) + w1 B_1, then the chunk-2 prefix."""
    T, chunk, w0, w1 = 24, 8, 0.7, 0.25
    raw = _inputs(T, 6, 5, 2, 1, seed=9, lead=(1, 1))
    g = _gates(raw, chunk, 0.0)
    g[..., 0] = w0
    g[..., 1] = w1
    out = _run(raw, g, chunk)
    sA, sB = oracle.chunk_summaries(raw["K"], raw["V"], raw["log_decay"], raw["A"], raw["B"], chunk)
    I = np.eye(6)
    S = ((1 - w1) * I + w1 * sA[0, 0, 1]) @ (w0 * sB[0, 0, 0]) + w1 * sB[0, 0, 1]
    sl = slice(16, 24)
    part = {k: (None if v is None else v[:, :, sl]) for k, v in raw.items()}
    ref, _ = oracle.generic(part["q"], part["K"], part["V"], part["log_decay"], part["A"], part["B"],
                            initial_state=S[None, None])
    assert np.abs(out[:, :, sl] - ref).max() <= 1e-12 * np.abs(ref).max()
    # history applied in time order: swapping the two gates changes the result
    g2 = g.copy()
    g2[..., 0], g2[..., 1] = w1, w0
    assert np.abs(_run(raw, g2, chunk)[:, :, sl] - out[:, :, sl]).max() > 1e-6 * np.abs(ref).max()


def test_threshold_zeroes_small_gates():
    T, chunk, theta = 32, 8, 0.1
    raw = _inputs(T, 6, 4, 1, 1, seed=11)
    below = _run(raw, _gates(raw, chunk, 0.0999), chunk, theta)
    zero = _run(raw, _gates(raw, chunk, 0.0), chunk, theta)
    assert np.array_equal(below, zero)
    at = _run(raw, _gates(raw, chunk, 0.1), chunk, theta)
    kept = _run(raw, _gates(raw, chunk, 0.1), chunk, 0.0)
    assert np.array_equal(at, kept)
    assert np.abs(at - zero).max() > 0


def test_gates_generator_rate():
    g = workloads.hla_gates(1, 2, 512, 64, seed=0)
    assert g.shape == (1, 2, 512, 8) and g.dtype == np.float32
    assert 0.08 < float(np.mean(g >= 0.1)) < 0.15
    assert np.array_equal(g, workloads.hla_gates(1, 2, 512, 64, seed=0))
