"""Prioritized-replay source sampling: CPU reference.  Test infrastructure
only -- the product path never imports it.

Sources: "GPU IQL + HER Porting Plan", section "Current State" (the GPU PER
buffer samples by a prefix sum of the priorities and a search in it, with
no CPU-side binary search, and returns indices and importance-sampling
weights) and section "How HER Interacts with GPU PER" (``sample_indices``
draws only indices and IS weights, PER-weighted, for the HER sources).

Readings (the pages name the method, not its constants):
  * priorities are stored as they are sampled by (any exponent alpha already
    applied), so row i is drawn with probability p_i / sum(p);
  * draws are independent, with replacement, by inverse transform: u =
    U * total with U uniform in [0, 1), and the row is the first i whose
    inclusive prefix sum exceeds u (a searchsorted on the right side), so a
    row of priority 0 is never drawn;
  * U is 53 random bits of word 0 of Philox4x64-10 under the key (seed,
    PER_KEY1) at counter (draw, step, 0, 0), times 2^-53 -- the generator the
    HER donor draws use, with a key word of its own; u is capped just below
    the total (U * total can round up to it), so a row is always found;
  * importance weights are those of prioritized replay (Schaul et al., 2016):
    (N P(i))^-beta divided by the largest weight of the batch, which is
    (p_min / p_i)^beta with p_min the smallest priority among the batch's
    rows (N and the total cancel);
  * prefix sums are taken in binary64.
"""
import numpy as np

from . import philox

PER_KEY1 = 0x5045526472617773  # second key word of the sampling stream ("PERdraws")


def uniforms(n, seed, step):
    """U in [0, 1) for draws 0 .. n-1, as binary64."""
    rows = np.arange(n, dtype=np.uint64)
    w0, _, _, _ = philox.philox4x64((rows, np.uint64(step), 0, 0), (np.uint64(seed), np.uint64(PER_KEY1)))
    return (w0 >> np.uint64(11)).astype(np.float64) * 2.0 ** -53


def find_rows(prefix, u):
    """The first row whose inclusive prefix sum exceeds u, for each u (so a
    u equal to a prefix value takes the next row of positive priority, and a
    row of priority 0 is never found)."""
    return np.searchsorted(prefix, u, side="right")


def sample(priorities, n, seed, step, beta):
    """Returns (indices int64 [n], IS weights float64 [n], u [n], prefix [size])."""
    p = np.asarray(priorities, dtype=np.float64)
    prefix = np.cumsum(p)
    total = prefix[-1]
    u = np.minimum(uniforms(n, seed, step) * total, np.nextafter(total, -np.inf))
    idx = find_rows(prefix, u)
    pi = p[idx]
    w = (pi.min() / pi) ** beta
    return idx.astype(np.int64), w, u, prefix
