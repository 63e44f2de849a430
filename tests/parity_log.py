"""Max-abs errors of the GPU parity checks against the fp64 oracle, one
record per compared case, kept for the end-of-run summary (conftest.py) and
written to gpurun_out/parity_errors.json."""

RECORDS = []
