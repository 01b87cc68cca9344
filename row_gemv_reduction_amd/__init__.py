"""MI355X-native row-parallel decode projections and ring-ordered reduction."""
from . import synth, workloads  # noqa: F401
