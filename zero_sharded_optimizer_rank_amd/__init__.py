"""One data-parallel rank's ZeRO step on its 1/N shard, native to MI355X (gfx950).

The step runs in hand-written HIP kernels behind the C ABI declared in
include/zero_shard.h (libzero_shard.so).  ``abi`` binds that ABI under the same
names; ``shard`` holds device buffers for one rank's shard and feeds them with
seeded synthetic inputs.
"""
from . import abi  # noqa: F401
