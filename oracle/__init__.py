"""CPU oracle for the Sketch&Walk hot path (fp64 NumPy).

Test infrastructure only: the tests, the smoke check and the bench's CPU
baseline leg may import it.  The HIP library never calls it and it imports
nothing from the HIP path.
"""
from .sws_oracle import *  # noqa: F401,F403
