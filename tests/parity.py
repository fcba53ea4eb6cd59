"""Comparison rules between the HIP path and the CPU oracle.

Routing: the set of selected experts must equal the oracle's, except for
tokens whose oracle logits have a gap below 1e-3 between the k-th and
(k+1)-th largest (two correct fp32 summation orders may choose differently
there); such a token's GPU selection must still lie within 1e-3 of the k-th
logit.  The order inside the selection (descending logit) must match too,
except that two selected experts whose oracle logits differ by less than 1e-3
may appear swapped: the same rule applied inside the selection.  Histogram,
offsets and permutation must equal the oracle's permutation of the GPU's own
ids, bit for bit.  Weights are compared per expert id (1e-5).

Output (bf16): |gpu - oracle| <= 2e-2 * rms(oracle) + ulp(oracle)/2 for every
element and sum|gpu - oracle| / sum|oracle| <= 5e-3, oracle in fp64.  The
half-ulp term is the rounding of the exact value to the bf16 output format
itself: without it the correctly rounded exact result would fail the max
gate wherever an output exceeds about 5x rms near the bottom of a binade.
"""
import json
import os

import numpy as np

import oracle

GAP = 1e-3
MAX_TOL = 2e-2
MEAN_TOL = 5e-3
WEIGHT_TOL = 1e-5


def bf16_to_f64(a) -> np.ndarray:
    a = np.asarray(a)
    return (a.astype(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check_routing(ids, weights, counts, offsets, slots, ref_logits, ref_ids, ref_w, E):
    """Returns the boolean mask of tokens whose selected set differs (all exempt)."""
    T, k = ref_ids.shape
    l = ref_logits.astype(np.float64)
    exempt = oracle.exempt_tokens(ref_logits, k, GAP)
    same_set = np.array([set(a) == set(b) for a, b in zip(ids.tolist(), ref_ids.tolist())], bool)
    bad = ~same_set & ~exempt
    assert not bad.any(), f"selected experts differ on non-exempt tokens {np.nonzero(bad)[0][:10]}"
    kth = -np.sort(-l, axis=1)[:, k - 1]
    for t in np.nonzero(~same_set)[0]:
        assert len(set(ids[t].tolist())) == k
        assert (l[t, ids[t]] >= kth[t] - GAP).all(), f"token {t}: selection outside the near-tie band"
    swapped = same_set & (ids != ref_ids).any(axis=1)
    for t in np.nonzero(swapped)[0]:
        j = np.nonzero(ids[t] != ref_ids[t])[0]
        gaps = np.abs(l[t, ids[t, j]] - l[t, ref_ids[t, j]])
        assert (gaps < GAP).all(), f"token {t}: order differs between logits {gaps.max():.2e} apart"
    for t in np.nonzero(same_set)[0]:
        a, b = np.argsort(ids[t]), np.argsort(ref_ids[t])
        np.testing.assert_allclose(weights[t, a], ref_w[t, b], rtol=0, atol=WEIGHT_TOL)
    c, o, s = oracle.permutation(ids, E)
    assert np.array_equal(counts, c), "expert counts differ"
    assert np.array_equal(offsets, o), "expert offsets differ"
    assert np.array_equal(slots, s), "sorted slots differ"
    return ~same_set


def bf16_half_ulp(v):
    """Half a bf16 ulp at |v| (0 at 0): bf16 keeps 8 significant bits."""
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(e - 8), 0.0)


def output_errors(got, ref):
    """(max over elements of (|err| - ulp/2) / rms, sum|err| / sum|ref|)."""
    err = np.abs(got - ref)
    rms = np.sqrt(np.mean(ref * ref))
    beyond = np.maximum(err - bf16_half_ulp(ref), 0.0)
    return beyond.max() / rms, err.sum() / np.abs(ref).sum()


def worst(got, ref, n=5):
    err = np.abs(got - ref)
    idx = np.argsort(err, axis=None)[::-1][:n]
    rows = [np.unravel_index(i, err.shape) for i in idx]
    return "; ".join(f"{tuple(int(v) for v in r)}: got {got[r]:.6g} ref {ref[r]:.6g}" for r in rows)


def _log_margin(label, mx, mean, raw_mx, max_tol, mean_tol):
    """Appends one JSON line per comparison to the file named by PARITY_LOG
    (unset: nothing is written), so the margins of a run can be tabulated."""
    path = os.environ.get("PARITY_LOG")
    if not path:
        return
    rec = {"case": label or os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0],
           "max_beyond_half_ulp_over_rms": float(mx), "max_raw_over_rms": float(raw_mx),
           "mean_rel": float(mean), "max_tol": max_tol, "mean_tol": mean_tol,
           "max_margin": float(mx / max_tol), "mean_margin": float(mean / mean_tol)}
    with open(path, "a") as f:
        f.write(json.dumps(rec) + "\n")


def check_output(got, ref, max_tol=MAX_TOL, mean_tol=MEAN_TOL, label=""):
    """Returns (max beyond half-ulp / rms, mean relative error, raw max / rms)."""
    mx, mean = output_errors(got, ref)
    raw = np.abs(got - ref).max() / max(np.sqrt(np.mean(ref * ref)), 1e-300)
    _log_margin(label, mx, mean, raw, max_tol, mean_tol)
    assert mx <= max_tol and mean <= mean_tol, (
        f"max (beyond half-ulp)/rms={mx:.3e} (<= {max_tol}), mean rel={mean:.3e} (<= {mean_tol}); "
        f"rms={np.sqrt(np.mean(ref * ref)):.4g}; worst: {worst(got, ref)}")
    return mx, mean, raw
