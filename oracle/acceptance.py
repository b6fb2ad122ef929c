"""Acceptance rule for one (batch, kv head) unit: an implementation's stop and
output against the oracle's ``UnitResult`` (test infrastructure only, like
the rest of this package).

  * The stop must equal the oracle's.  The one exception is a "margin-excused"
    unit: some stability check t <= max(stop, oracle stop) has a metric
    within a relative margin MARGIN of its threshold (``relative_margin``).
    There the fp32 accumulation of an implementation and the oracle's fp64
    can legitimately fall on opposite sides of the threshold (ART, Sec. 3.2,
    the stability tests).
  * The output is compared with the oracle's exact truncated attention at
    the implementation's own stop, O^(stop).  In detect-only mode, which
    attends to every block, it is compared with O^(T').  The bounds are
    relative L2 <= REL_L2 and max-abs <= MAX_ABS over the unit's query
    vectors.
With a test switched off (FLAG_NO_SCALE / FLAG_NO_DIR), only the remaining
test's margin can excuse a stop difference.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .art_oracle import FLAG_DETECT_ONLY, FLAG_NO_DIR, FLAG_NO_SCALE, UnitResult, relative_margin

REL_L2 = 1e-3
MAX_ABS = 4e-3
MARGIN = 1e-4


@dataclass
class UnitAgreement:
    stop_equal: bool
    excused: bool          # stops differ, within MARGIN of a threshold
    margin: float          # smallest relative margin over checks 1..max(stop)-1 (inf if not needed)
    stop_in_range: bool    # 1 <= stop <= T' (0 for an empty unit)
    rel_l2: float          # inf when the stop is out of range or the output is not finite
    max_abs: float

    @property
    def output_ok(self) -> bool:
        return self.stop_in_range and self.rel_l2 <= REL_L2 and self.max_abs <= MAX_ABS

    @property
    def ok(self) -> bool:
        return (self.stop_equal or self.excused) and self.output_ok


def unit_agreement(r: UnitResult, out_unit: np.ndarray, stop: int, eps_scale: float, eps_dir: float,
                   flags: int = 0) -> UnitAgreement:
    """Apply the rule to one unit: ``out_unit`` [query vectors, d] and ``stop``
    are the implementation's, ``r`` the oracle's result for the same unit."""
    sg, so = int(stop), int(r.stop)
    margin = np.inf
    if sg != so:
        hi = max(sg, so)
        if hi > 1:
            rs = relative_margin(r.d_scale[1:hi], eps_scale)
            rd = relative_margin(r.d_dir[1:hi], eps_dir)
            if flags & FLAG_NO_SCALE:
                rs = np.full_like(rs, np.inf)
            if flags & FLAG_NO_DIR:
                rd = np.full_like(rd, np.inf)
            both = np.minimum(rs, rd)
            if np.any(np.isfinite(both)):
                margin = float(np.nanmin(both))
    lo = 1 if r.num_traversal > 0 else 0
    in_range = lo <= sg <= r.num_traversal
    rel = mab = np.inf
    if in_range:
        t_out = r.num_traversal if (flags & FLAG_DETECT_ONLY) else sg
        ref = r.O[t_out - 1] if t_out > 0 else np.zeros_like(r.out)
        diff = np.asarray(out_unit, dtype=np.float64) - ref
        nrm = np.linalg.norm(ref)
        rel = float(np.linalg.norm(diff) / nrm if nrm > 0 else np.linalg.norm(diff))
        mab = float(np.abs(diff).max()) if diff.size else 0.0
        if not np.isfinite(rel) or not np.isfinite(mab):
            rel = mab = np.inf
    return UnitAgreement(stop_equal=sg == so, excused=sg != so and margin <= MARGIN, margin=margin,
                         stop_in_range=in_range, rel_l2=rel, max_abs=mab)
