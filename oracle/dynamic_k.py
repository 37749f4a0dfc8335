"""Draft-length controller driven by the acceptance history.

TEST INFRASTRUCTURE ONLY (see ``oracle/spec_verify.py``): the reference the
library's native controller is checked against.

The rule, from page www.2kiu.com/news/5895634 §4.4 (the general policy is
also on page www.cf-1.com/news/5155685 §2.4: a long run of high acceptance
lengthens the draft, low acceptance shortens it):

* keep the acceptance statistics of the most recent ``window`` batches
  (100 on the page);
* when their acceptance rate is above ``raise_above`` (0.8), K grows by one;
  when it is below ``lower_below`` (0.6), K shrinks by one;
* K stays within [k_min, k_max] (2 and 10 on the page).

Readings where the page leaves the step open:

* The acceptance rate of a batch is accepted drafts / drafted tokens.  The
  window's rate is its accepted total over its drafted total.  A window
  only ever holds batches drafted at the current K (next point), so every
  batch in it drafted the same number of tokens unless some were dropped.
  This pooled rate then equals the plain mean of the per-batch rates.  It
  is taken from exact integer totals with one division, so every
  implementation decides alike.
* A decision needs a full window.  After K changes, the window starts empty.
  The rate depends on K (the later drafts of a longer run are accepted less
  often), so batches drafted at the old K say little about the new one.
  Without the restart, one crossing would walk K to its bound on stale
  data, one batch per step.
* Comparisons are strict, as the page's above/below.
* A batch that drafted nothing (a finished or failed sequence) is not
  observed.
* The initial K defaults to 5, the fixed value the same page suggests to
  start tuning from (§7).
"""
from __future__ import annotations


class DynamicK:
    """One controller; run one per sequence for per-sequence draft lengths."""

    def __init__(self, window: int = 100, raise_above: float = 0.8, lower_below: float = 0.6,
                 k_min: int = 2, k_max: int = 10, k_init: int = 5):
        if window < 1 or k_min < 0 or k_max < k_min or not (k_min <= k_init <= k_max):
            raise ValueError("need window >= 1 and 0 <= k_min <= k_init <= k_max")
        if not (0.0 <= lower_below <= raise_above <= 1.0):
            raise ValueError("need 0 <= lower_below <= raise_above <= 1")
        self.window = int(window)
        self.hi = float(raise_above)
        self.lo = float(lower_below)
        self.k_min = int(k_min)
        self.k_max = int(k_max)
        self.k = int(k_init)
        self.hist: list[tuple[int, int]] = []  # (accepted, drafted), oldest first

    def observe(self, accepted: int, drafted: int) -> int:
        """Record one batch and return the K to draft next."""
        accepted, drafted = int(accepted), int(drafted)
        if drafted < 0 or accepted < 0 or accepted > drafted:
            raise ValueError("need 0 <= accepted <= drafted")
        if drafted == 0:
            return self.k
        self.hist.append((accepted, drafted))
        if len(self.hist) > self.window:
            self.hist.pop(0)
        if len(self.hist) < self.window:
            return self.k
        acc = sum(a for a, _ in self.hist)
        dr = sum(d for _, d in self.hist)
        rate = float(acc) / float(dr)
        if rate > self.hi and self.k < self.k_max:
            self.k += 1
            self.hist = []
        elif rate < self.lo and self.k > self.k_min:
            self.k -= 1
            self.hist = []
        return self.k
