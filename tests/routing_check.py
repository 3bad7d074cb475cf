"""Validity of a top-k selection that differs from the oracle's by near-ties.

The router ranks experts by the biased score b = sigmoid(logit) + bias and
takes the k largest (page "vllm.models.deepseek_v41.amd.mono.runner",
MonoLayerWeights: the selection bias e_score_correction_bias).  Two experts
whose b differ by less than the arithmetic's error can come out in either
order, so where the GPU's picks differ from the oracle's the difference is
judged by the oracle's own scores: the picks must be distinct, ordered by b
(ties by index) up to `tol`, and no expert left out may beat a pick by more
than `tol`.  The picks that pass are near-ties; anything else is an error.
"""
from __future__ import annotations

import numpy as np

NEAR_TIE = 1e-6  # the margin below which two biased scores count as tied


def biased_scores(logits: np.ndarray, bias: np.ndarray) -> np.ndarray:
    """b = sigmoid(l) + bias in double, from the oracle's logits."""
    logits = np.asarray(logits, np.float64)
    return 1.0 / (1.0 + np.exp(-logits)) + np.asarray(bias, np.float64)


def check_picks(gpu_ids: np.ndarray, ref_ids: np.ndarray, logits: np.ndarray,
                bias: np.ndarray, tol: float = NEAR_TIE) -> list[int]:
    """Tokens whose picks differ from the oracle's as valid near-ties.

    Raises AssertionError when a token's picks are not a valid top-k of the
    oracle's biased scores within `tol`."""
    gpu_ids = np.asarray(gpu_ids)
    ref_ids = np.asarray(ref_ids)
    m, k = ref_ids.shape
    b = biased_scores(logits, bias)
    E = b.shape[1]
    ties = []
    for t in range(m):
        g = [int(e) for e in gpu_ids[t]]
        if g == [int(e) for e in ref_ids[t]]:
            continue
        assert all(0 <= e < E for e in g), f"token {t}: pick out of range {g}"
        assert len(set(g)) == k, f"token {t}: repeated pick {g}"
        bt = b[t]
        for j in range(k - 1):
            assert bt[g[j]] >= bt[g[j + 1]] - tol, (
                f"token {t}: pick {j} ({g[j]}, b={bt[g[j]]!r}) ranked above "
                f"pick {j + 1} ({g[j + 1]}, b={bt[g[j + 1]]!r}) beyond {tol}")
        rest = np.setdiff1d(np.arange(E), g)
        if rest.size:
            worst_in = min(bt[e] for e in g)
            best_out = bt[rest].max()
            assert worst_in >= best_out - tol, (
                f"token {t}: expert {int(rest[bt[rest].argmax()])} (b={best_out!r}) left out "
                f"while pick b={worst_in!r} was taken, beyond {tol}")
        ties.append(t)
    return ties


def weights_of(ids: np.ndarray, logits: np.ndarray, routed_scale: float) -> np.ndarray:
    """Routing weights of given picks from the oracle's logits: the picks'
    sigmoid scores renormalised to sum to one, times routed_scale."""
    s = 1.0 / (1.0 + np.exp(-np.asarray(logits, np.float64)))
    sel = np.take_along_axis(s, np.asarray(ids, np.int64), axis=1)
    return routed_scale * sel / sel.sum(axis=1, keepdims=True)
