"""CPU oracle of one native-MTP speculative cycle (fp64).

TEST INFRASTRUCTURE: only the tests, the package smoke check and the bench's CPU
baseline may import it.  It shares no code with the HIP library.
"""
from . import mtp_oracle  # noqa: F401
