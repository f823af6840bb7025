"""CPU oracle for the per-frame decode step (test infrastructure only).

Only tests/, the smoke check and bench.py's cpu_baseline leg import this
package.  It never imports the HIP library or its binding.
"""
from .oracle import Oracle, build_oracle, load_library, model_struct  # noqa: F401
