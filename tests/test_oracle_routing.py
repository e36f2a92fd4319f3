"""Pins of the oracle's top-k softmax routing (CPU): closed forms, and scipy's
softmax with a stable argsort (library routines) on random logits."""
import numpy as np
from scipy.special import softmax

import oracle
import synth


def test_uniform_logits_tie_to_lower_ids():
    ids, w = oracle.topk_softmax(np.zeros((3, 64), np.float32), 8)
    assert (ids == np.arange(8)).all()
    assert (w == np.float32(1 / 64)).all()


def test_one_dominant_logit_and_closed_form():
    lg = np.zeros((1, 4), np.float32)
    lg[0, 2] = np.log(3.0)          # p = (1, 1, 3, 1) / 6
    ids, w = oracle.topk_softmax(lg, 4)
    assert ids.tolist() == [[2, 0, 1, 3]]
    np.testing.assert_allclose(w[0], np.float32([0.5, 1 / 6, 1 / 6, 1 / 6]), rtol=1e-7)


def test_against_scipy_softmax_and_stable_argsort():
    lg = synth.moe_logits(300, 64, seed=3)
    for k in (1, 8, 64):
        ids, w = oracle.topk_softmax(lg, k)
        p = softmax(lg.astype(np.float64), axis=1)
        ref = np.argsort(-p, axis=1, kind="stable")[:, :k]
        assert np.array_equal(ids, ref)
        np.testing.assert_allclose(w, np.take_along_axis(p, ref, axis=1).astype(np.float32), rtol=1e-6)
    # all experts: the weights sum to one
    ids, w = oracle.topk_softmax(lg, 64)
    np.testing.assert_allclose(w.astype(np.float64).sum(axis=1), 1.0, rtol=1e-6)


def test_same_routing_as_the_harness():
    ids0, w0 = synth.topk_routing(50, 64, 8, seed=7)
    ids, w = oracle.topk_softmax(synth.moe_logits(50, 64, seed=7), 8)
    # the harness ranks FP64 logits, the oracle their FP32 roundings: the
    # selections agree for these draws, the weights to FP32 rounding
    assert np.array_equal(ids, ids0)
    np.testing.assert_allclose(w, w0, rtol=1e-6)
