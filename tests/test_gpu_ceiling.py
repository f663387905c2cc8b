"""Measured-ceiling helpers (include/hqmq_ceiling.h): they run on the GPU and
give figures in a plausible range for an MI355X; invalid arguments are
rejected on the host before anything is enqueued."""
import pytest
import torch

import kv_cache_quantization_hqmq_amd as K
from kv_cache_quantization_hqmq_amd import hqmq as B


def test_ceiling_arguments_rejected_on_host():
    for kind, nbytes in ((K.HQMQ_CEIL_COPY, 0), (K.HQMQ_CEIL_COPY, 24), (7, 1024)):
        with pytest.raises(K.HQMQError):
            B.hqmq_ceiling_stream(kind, None, None, nbytes, stream=0)
    with pytest.raises(K.HQMQError):
        B.hqmq_ceiling_compute(K.HQMQ_CEIL_FMA_F32, 0, None, stream=0)
    with pytest.raises(K.HQMQError):
        B.hqmq_ceiling_compute(9, 10, None, stream=0)


@pytest.mark.gpu
def test_ceilings_run_and_are_plausible():
    n = 256 << 20
    src = torch.ones(n // 2, dtype=torch.float16, device="cuda")
    dst = torch.zeros(n // 2, dtype=torch.float16, device="cuda")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for kind, moved, lo in ((K.HQMQ_CEIL_READ, n, 500), (K.HQMQ_CEIL_WRITE, n, 500),
                            (K.HQMQ_CEIL_COPY, 2 * n, 500)):
        B.hqmq_ceiling_stream(kind, src, dst, n)
        ev0.record()
        B.hqmq_ceiling_stream(kind, src, dst, n)
        ev1.record()
        torch.cuda.synchronize()
        gbps = moved / (ev0.elapsed_time(ev1) * 1e-3) / 1e9
        assert lo < gbps < 9000, (kind, gbps)
    # the copy wrote src's values
    assert torch.equal(dst, src)
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    for kind, iters, lo, hi in ((K.HQMQ_CEIL_FMA_F32, 2000, 5, 170), (K.HQMQ_CEIL_MFMA_F32, 1000, 20, 170),
                                (K.HQMQ_CEIL_MFMA_F16, 1000, 100, 2600)):
        B.hqmq_ceiling_compute(kind, iters, sink)
        ev0.record()
        fl = B.hqmq_ceiling_compute(kind, iters, sink)
        ev1.record()
        torch.cuda.synchronize()
        tf = fl / (ev0.elapsed_time(ev1) * 1e-3) / 1e12
        assert lo < tf < hi, (kind, tf)
