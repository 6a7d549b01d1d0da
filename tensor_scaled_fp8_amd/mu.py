"""Host-side policy for the gradient auto-scaling factor mu (g' = mu * g).

[FP8-LM reading note, "Proposed method", O1, Eq. 3] mu is changed
dynamically; the pages do not say how. This module takes the plainest
reading of "auto-scaling" used for loss scaling: mu is a power of two
(mu = 2^mu_log2, so scaling stays exact), lowered by one step whenever the
fraction of gradient elements clipped at the E5M2 maximum in a step exceeds
a threshold, and raised by one step after `window` consecutive steps below
it, within [lo, hi]. The clipped count comes from fp8_wgrad_fp8
(record field sat_count). Host logic only: no arithmetic of the FP8 path."""
from __future__ import annotations


class MuScaler:
    def __init__(self, mu_log2: int = 0, threshold: float = 1e-5, window: int = 100, lo: int = -16, hi: int = 16):
        if not lo <= mu_log2 <= hi:
            raise ValueError("mu_log2 outside [lo, hi]")
        if window < 1 or threshold < 0:
            raise ValueError("window must be >= 1 and threshold >= 0")
        self.mu_log2 = mu_log2
        self.threshold = threshold
        self.window = window
        self.lo, self.hi = lo, hi
        self.clean = 0

    def update(self, saturated: int, numel: int) -> int:
        """Record one step's clipped-element count; return the mu_log2 to use next."""
        if numel > 0 and saturated > self.threshold * numel:
            self.mu_log2 = max(self.lo, self.mu_log2 - 1)
            self.clean = 0
        else:
            self.clean += 1
            if self.clean >= self.window:
                self.mu_log2 = min(self.hi, self.mu_log2 + 1)
                self.clean = 0
        return self.mu_log2
