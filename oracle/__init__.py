"""Float64 CPU oracle for Linformer attention.  Test infrastructure only: used by tests/, the
package smoke check and the benchmark's CPU-baseline leg, never by the product path."""
from .linformer_oracle import *  # noqa: F401,F403
