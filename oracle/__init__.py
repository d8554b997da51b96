"""CPU oracle (test infrastructure only; see seed_oracle.py's header)."""
from .seed_oracle import *  # noqa: F401,F403
from .seed_oracle import (GDN, KDA, MAMBA2, RULES, compress, define_run, dense_run,  # noqa: F401
                          dense_state_bytes, dense_step, factored_run, reconstruct,
                          seed_step, shallow_state_bytes, sink_extract, state_from_dense,
                          trunc_svd, value_split)
