"""CPU oracle for packed ternary weights (test infrastructure only; see tern_oracle)."""
from .tern_oracle import *  # noqa: F401,F403
from .tern_oracle import (FMT_2BIT, FMT_B3, OFF_NONE, OFF_ROW, OFF_GROUP,  # noqa: F401
                          PackError, CorruptError)
