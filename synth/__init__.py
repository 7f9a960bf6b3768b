"""Seeded synthetic inputs (values, quantised caches, page tables) shared by the
oracle-side tests and the HIP path.  Holds no step of the DSA computation."""
from . import codecs, workloads  # noqa: F401
from .workloads import CONFIGS, Spec, Workload, make_workload, mark_absent  # noqa: F401
