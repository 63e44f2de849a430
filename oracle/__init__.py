"""fp64 CPU oracle for the fused attention forward (test infrastructure only).

This package is the checker, not the product.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It shares no code with the HIP library or its Python binding and
imports neither.

Every function is the plain definition written out in numpy float64 (see
``oracle/attention.py`` for the passages each one follows).  Parity status:
every function here is pinned by a ``-m "not gpu"`` test against brute force,
closed forms or invariants; none is "parity unpinned".
"""

from .attention import (  # noqa: F401
    Bias,
    Mask,
    token_coords,
    table_relative_index,
    table_bias,
    relpos_rows,
    rel_pos_resized,
    e4m3_decode,
    dequantize_e4m3,
    relpos_bias,
    relpos_bias_gather,
    shift_region_labels,
    window_partition,
    window_reverse,
    shift_mask,
    attention_probs,
    attention_logsumexp,
    attention,
    attention_image,
    attention_image_logsumexp,
    attention_backward,
    attention_image_backward,
    run_workload,
    run_workload_logsumexp,
    run_workload_backward,
)
