"""fp64 CPU oracle of the fast-weight scan: test infrastructure only (see fwmem_oracle)."""
from .fwmem_oracle import RULE_ADDITIVE, RULE_DELTA, phi, relerr, scan, step  # noqa: F401
