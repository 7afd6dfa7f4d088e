"""Full-size parity of the benchmark layer (W 4096x4096 fp16, 262144 fp16
tokens, 4-bit, group 128, block 128), in the launch configuration bench.py
times, checked on sampled outputs the oracle computes exactly."""
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(600)
def test_attention_projection_full_size():
    from workload_checks import run_job
    run_job("attn", 0)
