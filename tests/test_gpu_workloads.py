"""Full-size parity of every layer configuration, in the launch configuration
bench.py times, checked on sampled outputs the oracle computes exactly
(tests/workload_checks.py): the attention projection (4096x4096, 4-bit g128,
262144 tokens); the MLP pair at hidden size 4096 (up 11008x4096 and down
4096x11008, 3-bit per row, 262144 tokens); a 7B-shaped block over 65536 tokens
(q/k/v stacked on one Hessian, o, gate/up stacked on one Hessian, down; 4-bit
g128); a 175B-class FFN shard (fc1 49152x12288, fc2 12288x49152, 3-bit g128,
262144 tokens); and the attention projection end to end against the oracle's
own fp64 pipeline from X."""
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(600)
def test_attention_projection_full_size():
    from workload_checks import run_job
    run_job("attn", 0)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("job", [0, 1], ids=["up", "down"])
def test_mlp_pair(job):
    from workload_checks import run_job
    run_job("mlp", job)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("job", [0, 1, 2, 3], ids=["qkv", "o", "gate_up", "down"])
def test_7b_block(job):
    from workload_checks import run_job
    run_job("block7b", job)


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("job", [0, 1], ids=["fc1", "fc2"])
def test_175b_ffn_shard(job):
    from workload_checks import run_job
    run_job("ffn175b", job, sample_rows=1024 if job == 0 else 512, host_prepare_max_n=12288)


@pytest.mark.timeout(900)
def test_attention_projection_end_to_end_oracle():
    """The benchmark layer against the oracle's own fp64 pipeline from X
    (its own H, factor and sweep) on sampled rows."""
    import numpy as np
    import torch

    import oracle as O
    import post_weight_quantization_10_amd as pw
    import synth
    from parity import LOSS_RTOL, MIN_SAME, assert_codes, compare_codes, follow_check, say
    wl = synth.workloads()["attn"]
    job = wl.jobs[0]
    W = synth.stacked_weight(job, wl.seed, wl.wid)
    X = synth.x_full(job.x, wl.seed, wl.wid)
    m, n = W.shape
    say(f"[attn end-to-end] W {m}x{n} X {X.shape[0]}x{n}")
    res = pw.gptq_layer(torch.from_numpy(W).to("cuda:0"), torch.from_numpy(X).to("cuda:0"), job.bits, job.group,
                        job.block, job.damp)
    torch.cuda.synchronize()
    H = O.hessian([X[c:c + 2048] for c in range(0, X.shape[0], 2048)])
    Hd, lam = O.damp(H, job.damp)
    U, info = O.inverse_cholesky_upper(Hd)
    assert info == 0
    rows = np.sort(np.random.default_rng(99).choice(m, 1024, replace=False))
    ref = O.gptq_quantize(W[rows].astype(np.float64), U, job.bits, job.group, job.block)
    q = O.unpack_codes(res["qcodes"][rows].cpu().numpy().view(np.uint32), job.bits, n)
    s = res["scales"][rows].cpu().numpy()
    z = res["zeros"][rows].cpu().numpy()
    rep = compare_codes(q, s, z, ref, job.group)
    say(f"  identical {rep['same_frac']:.6f} diverged rows {rep['rows_diverged']}/{len(rows)}")
    assert_codes(rep, "attn end-to-end", min_same=MIN_SAME)
    follow_check(q, s, z, W[rows].astype(np.float64), U, job.bits, job.group, job.block, "attn end-to-end")
    Wr = W[rows].astype(np.float64)
    l_gpu = O.layer_loss(Wr, O.dequant_from(q, s, z, job.group), H)
    l_ref = O.layer_loss(Wr, ref["What"], H)
    assert abs(l_gpu - l_ref) <= LOSS_RTOL * l_ref
