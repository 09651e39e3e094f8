"""Re-paging of 256-token pages into a 64-token scratch, reference.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed (sglang PR 39288, Root cause (2) and Modifications): the
pool keeps 256-token pages, the reader wants 64-token pages, and only the
source pages a step references are copied, each into four consecutive 64-token
pages of a scratch that was zero-filled when it was allocated:

  P1  for every listed p with 0 <= p < num_src_pages and k = 0..3, scratch
      page 4p + k takes the tokens 64k .. 64k + 63 of pool page p;
  P2  nothing else in the scratch changes (unlisted pages stay as they were:
      zero in a fresh scratch, so slot 0 is finite unless page 0 is copied).

With token rows stored contiguously, token t of pool page p (slot 256p + t)
lands at slot 64(4p + t // 64) + t % 64 = 256p + t of the scratch: the
re-paging keeps every slot number.
"""
from __future__ import annotations

import numpy as np


def split_pages_64(src_pool: np.ndarray, pages: np.ndarray, dst: np.ndarray, row_bytes: int) -> None:
    """src_pool uint8 [num_src_pages][>= 256 * row_bytes]; dst uint8
    [>= 4 * num_src_pages][>= 64 * row_bytes], updated in place."""
    q = 64 * row_bytes
    for p in np.asarray(pages, dtype=np.int64):
        if 0 <= p < src_pool.shape[0]:
            for k in range(4):
                dst[4 * p + k, :q] = src_pool[p, k * q:(k + 1) * q]
