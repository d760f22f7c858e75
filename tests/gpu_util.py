"""Device-side runner for the GPU tests: re-exports the package's device helpers (which call
the library through its C ABI) and adds the tests' log helper. Nothing here computes any
part of the method."""
import sys

from shifted_window_attention_amd.device import (  # noqa: F401
    BLOCK_FIELDS, BlockOnDevice, ModuleOnDevice, from_dev, run_block_chain, run_chain, to_dev)


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()
