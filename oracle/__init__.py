"""CPU oracle (test infrastructure only): the plain float64 definition of the
paged KV-cache update and of ragged paged attention.  Only the tests, the
smoke check and the benchmark's CPU-baseline leg may import it."""
from . import rpa_oracle  # noqa: F401
