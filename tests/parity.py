"""Shared comparison rules of the GPU parity tests.

Logits: max-abs <= 2e-2 and relative L2 ||a-b|| / ||b|| <= 1e-3 over [V].
Tokens: identical streams, except that after the first step at which they
differ nothing is compared, and that step must have an oracle top-2 logit gap
below 2e-2 (a near-tie the rounding of either side may decide)."""
import sys

import numpy as np

LOGIT_MAX_ABS = 2e-2
LOGIT_REL_L2 = 1e-3
TIE_GAP = 2e-2


def logits_ok(gpu, ref, where=""):
    a = np.asarray(gpu, np.float64)
    b = np.asarray(ref, np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    d = float(np.abs(a - b).max())
    rel = float(np.linalg.norm(a - b) / np.linalg.norm(b))
    exact = float(np.mean(a == b))
    assert d <= LOGIT_MAX_ABS and rel <= LOGIT_REL_L2, \
        "%s: max-abs %.3e rel-L2 %.3e (exact %.4f)" % (where, d, rel, exact)
    return d, rel, exact


def tokens_ok(got, ref, gaps, where=""):
    """Returns the number of steps compared."""
    for t, (g, r) in enumerate(zip(got, ref)):
        if g != r:
            assert gaps[t] < TIE_GAP, "%s: token %d differs (%d vs %d), oracle gap %.3e" % (
                where, t, g, r, gaps[t])
            print("%s: streams part at step %d (oracle gap %.3e)" % (where, t, gaps[t]))
            sys.stdout.flush()
            return t
    assert len(got) == len(ref)
    return len(ref)
