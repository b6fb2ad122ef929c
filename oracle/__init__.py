"""fp64 CPU oracle for ART decode attention (test infrastructure only).

Imported only by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``; never by the library or its binding.
"""
from .art_oracle import (FLAG_DETECT_ONLY, FLAG_NO_DIR, FLAG_NO_SCALE, MODE_ART, MODE_FULL, ORDER_GIVEN,
                         ORDER_NATURAL, ORDER_RECENT_FIRST,
                         PROBE_STRIDE, UnitResult, art_decode, art_decode_rows, art_decode_workload, art_unit,
                         gather_unit, prefix_outputs, probe, relative_margin, stability_trace,
                         stop_index, threshold, traversal, widen)
from .select_oracle import (SELECT_ASCENDING, SELECT_IMPORTANCE, block_means, block_scores, keep_count,  # noqa: F401
                            mean_query, select_blocks, select_unit, select_workload)
