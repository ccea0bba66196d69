"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

Holds input drawing, the host block allocator, block-level relayouts and
byte accounting -- none of the attention arithmetic.  The oracle and the
HIP library both consume what this package produces; neither is imported
here.
"""

from .accounting import (ELEMENT_BYTES, copy_bytes, decode_bytes, kv_bytes,  # noqa: F401
                         prefill_bytes,
                         kv_bytes_per_token, row_bytes, write_bytes)
from .allocator import BlockManager, Sequence  # noqa: F401
from .batch import (PREFILL_WORKLOADS, WORKLOADS, Batch, Workload,  # noqa: F401
                    chunk_k_pool, contiguous_layout,
                    draw_lens, extract_sequences, host_view, make_batch,
                    permute_blocks, unshare)
