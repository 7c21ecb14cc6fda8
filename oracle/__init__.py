"""Float64 CPU oracle for exact attention.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the package smoke check and
by the benchmark's ``cpu_baseline`` leg, never by the product path.  It shares no
code with the HIP library.
"""
from .attention import (dense_bwd, dense_fwd, dense_probs, loop_order_ledger,  # noqa: F401
                        online_fwd, online_fwd_kv_outer, sampled_bwd, transfer_ledger)
