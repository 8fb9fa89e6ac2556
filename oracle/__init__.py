"""CPU oracle for MSA -- test infrastructure only (tests, smoke check and the
benchmark's CPU baseline); never imported by the library."""
from . import msa_oracle  # noqa: F401
