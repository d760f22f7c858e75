"""The oracle's chain runners (oracle/chains.py), under the name the tests use."""
from oracle.chains import (  # noqa: F401
    block_chain_full, block_params_of, chain_full, chain_masked_dy, chain_sampled, layouts, params_of)
