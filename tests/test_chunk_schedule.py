"""Host logic of the whole-prompt chunked prefill (no GPU work): the chunk
schedule covers every query once, each chunk's keys end where its queries
end, and the compressed-key windows are appended exactly once, in order,
each by the chunk in which its last token arrives."""
import pytest

import oracle as O
from block_sparse_long_infllmv2_amd.pipeline import chunk_schedule
from block_sparse_long_infllmv2_amd.workloads import Params


@pytest.mark.parametrize("n,chunk,ks,s", [(131072, 8192, 32, 16), (2560, 512, 32, 16),
                                           (1000, 300, 32, 16), (40, 64, 32, 16),
                                           (5000, 777, 48, 8)])
def test_chunk_schedule_covers_queries_and_windows(n, chunk, ks, s):
    p = Params(kernel_size=ks, kernel_stride=s)
    sched = chunk_schedule(n, chunk, p)
    q_next, m_next = 0, 0
    for q0, q1, n_k, m0, m1 in sched:
        assert q0 == q_next and q1 > q0 and q1 - q0 <= chunk
        assert n_k == q1                         # keys up to the chunk's last query
        assert m0 == m_next and m1 >= m0
        # windows [m0, m1) end inside this chunk: last token m*s + ks - 1 in [q0, q1)
        for m in (m0, m1 - 1) if m1 > m0 else ():
            assert q0 <= m * s + ks - 1 < q1 or (q0 == 0 and m * s + ks - 1 < q1)
        q_next, m_next = q1, m1
    assert q_next == n
    assert m_next == O.num_windows(n, ks, s)
