"""Float64 CPU oracle for the fused Gaussian-mixture E-step (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package. The HIP library never calls it and shares no code with it.
"""
from .gmm_oracle import (  # noqa: F401
    LOG_2PI,
    EMPTY_REL,
    border_lists,
    component_scores,
    em,
    estep,
    estep_rows,
    kmeans,
    kmeans_assign,
    kmeans_update,
    log_gauss_diag,
    log_gauss_diag_expanded,
    mstep,
    responsibilities,
    row_logsumexp,
    top2,
)
