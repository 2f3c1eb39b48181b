"""GPU parity of the batched-row weight-streaming GEMM (spec_mat_create /
spec_mat_mul): Y = X W^T for M = 1..128 activation rows (B sequences' K+1
verify rows), against numpy's fp64 product of the same bf16 weights.

The bound is the arithmetic's own: activations enter as bf16 high and low
parts (|x - hi - lo| <= 2^-17 |x|), bf16 x bf16 products are exact in fp32,
and fp32 accumulation of the K high-part and K low-part products (the wide
kernel sums both in one accumulator; the narrow one adds the two at the end)
plus the split-K sums adds at most (2K + 8) 2^-24 of sum |x w| -- so every
output must satisfy |y - ref| <= (2^-16 + (2K + 8) 2^-24) * sum_k |x_k w_nk|."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _case(N, K, Ms, seed):
    import speculative_decoding_02_amd as sd
    g = torch.Generator().manual_seed(seed)
    W = (torch.randn(N, K, generator=g) * 0.02).to(torch.bfloat16)
    Wd = W.cuda().contiguous()
    mat = sd.Mat(Wd)
    W64 = W.to(torch.float64).numpy()
    for M in Ms:
        X = torch.randn(M, K, generator=g, dtype=torch.float32)
        Y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        mat.mul(X.cuda(), Y)
        torch.cuda.synchronize()
        y = Y.cpu().numpy().astype(np.float64)
        X64 = X.numpy().astype(np.float64)
        ref = X64 @ W64.T
        bound = (2.0 ** -16 + (2 * K + 8) * 2.0 ** -24) * (np.abs(X64) @ np.abs(W64).T)
        err = np.abs(y - ref)
        assert np.all(np.isfinite(y)), M
        assert np.all(err <= bound), (M, float((err / bound).max()))


def test_rows_narrow():
    _case(512, 1024, [1, 5, 8, 9, 16, 31, 64, 100, 128], seed=1)


def test_rows_wide_two_blocks_per_workgroup():
    _case(12288, 512, [1, 7, 33, 128], seed=2)


def test_rows_wide_unsplit():
    # 192 column groups of 128: the wide kernel stores Y itself (no K split);
    # every row-tile count, with the last 16-row tile partly filled
    _case(24576, 256, [9, 17, 40, 100, 128], seed=3)


def test_rows_errors():
    import speculative_decoding_02_amd as sd
    W = torch.zeros(64, 64, dtype=torch.bfloat16, device="cuda")
    mat = sd.Mat(W)
    Y = torch.zeros(129, 64, device="cuda")
    for M in (0, 129):
        X = torch.zeros(max(M, 1), 64, device="cuda")
        with pytest.raises(sd.SpecError) as e:
            sd.spec_mat_mul(mat.handle, X[:M] if M else X[:0], Y)
        assert e.value.code == sd.SPEC_ERR_ARG
    with pytest.raises(sd.SpecError) as e:
        sd.spec_mat_create(torch.zeros(24, 64, dtype=torch.bfloat16, device="cuda"))
    assert e.value.code == sd.SPEC_ERR_ARG


def test_native_driver_gemm_sweep():
    """spec_run --gemm-rows drives spec_mat_mul natively (the process the
    counter profiles are taken on): one JSON line per (matrix, M) with a
    finite, positive time per launch."""
    import json
    import os
    import subprocess
    exe = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                       "speculative_decoding_02_amd", "spec_run")
    r = subprocess.run([exe, "--gemm-rows", "5,16,128", "--gemm-matrix", "qkv", "--rounds", "1"],
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr
    lines = [json.loads(l) for l in r.stdout.splitlines() if l.startswith("{")]
    assert [(d["matrix"], d["M"]) for d in lines] == [("8b qkv", 5), ("8b qkv", 16), ("8b qkv", 128)]
    for d in lines:
        assert (d["N"], d["K"]) == (6144, 4096) and d["launches"] > 0
        assert 0.0 < d["us_per_launch"] < 1e5
