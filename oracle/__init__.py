"""fp64 CPU oracle for one Gaussian-mixture EM iteration.

Test infrastructure: only tests/, the smoke check and the benchmark's CPU
baseline leg import it.  It shares no code with soft_clustering_amd.
"""
from .gmm_oracle import (  # noqa: F401
    Params, Prepared, StepResult, NotPositiveDefinite, cholesky_lower,
    ridged_cholesky, prepare, forward_substitution, sq_mahalanobis, log_joint,
    log_normaliser, responsibilities, loglik, em_step, fit,
    DEFAULT_VAR_FLOOR, DEFAULT_RIDGE_REL, EMPTY_NK, LOG_2PI,
)
from .gmm_assign_fit import (  # noqa: F401
    splitmix64, sample_distinct, init_random_points, assign_topm, fit_tol,
)
