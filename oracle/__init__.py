"""IF4 reference oracle -- TEST INFRASTRUCTURE ONLY.

Plain CPU statement of the IF4 path (see if4_oracle.h for the page
citations).  Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline
leg may import this package; the product path never does.
"""
from .oracle import *  # noqa: F401,F403
