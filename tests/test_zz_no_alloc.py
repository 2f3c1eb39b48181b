"""The allocation-free accept/reject entry point (spec_accept_reject_noalloc)
against spec_accept_reject: bit-identical tokens and n_acc on the same
inputs, over two calls in a row on one device, the second with a smaller
batch, vocabulary and K (so stale scratch contents from the first call are
present when the second runs), in sampling and greedy mode; both entry
points are called through the C ABI."""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _inputs(B, K, V, sigma, seed):
    T, D = synth.logit_pair(B, K, V, sigma, seed=seed)
    pos = np.arange(B, dtype=np.uint64) * 41 + 7
    d = np.stack([oracle.draft_sample_batch(D[:, i, :], synth.SEED_PHILOX, pos + i, 0)
                  for i in range(K)], 1).astype(np.int32)
    return T, D, d, pos


def _run(fn, T, D, d, pos, greedy):
    B, K1, V = T.shape
    Tt = torch.from_numpy(np.ascontiguousarray(T)).cuda()
    Dt = torch.from_numpy(np.ascontiguousarray(D)).cuda()
    dt = torch.from_numpy(np.ascontiguousarray(d)).cuda()
    pt = torch.from_numpy(pos.astype(np.int64)).cuda()
    out = torch.full((B, K1), -7, dtype=torch.int32, device="cuda")
    n = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    fn(Tt, Dt, dt, synth.SEED_PHILOX, pt, 0, greedy, out, n)
    torch.cuda.synchronize()
    return out.cpu().numpy(), n.cpu().numpy()


@pytest.mark.parametrize("greedy", [False, True])
def test_noalloc_matches_allocating_entry_point(greedy):
    import speculative_decoding_02_amd as sd
    cases = [(64, 8, 32000, 0.5, 11),   # the isolated-rule workload
             (5, 3, 1000, 2.0, 12)]     # then a smaller one over the same scratch
    for B, K, V, sigma, seed in cases:
        T, D, d, pos = _inputs(B, K, V, sigma, seed)
        o_ref, n_ref = _run(sd.spec_accept_reject, T, D, d, pos, greedy)
        o_new, n_new = _run(sd.spec_accept_reject_noalloc, T, D, d, pos, greedy)
        print(f"B={B} K={K} V={V} greedy={greedy}: n_acc {n_new.tolist()[:8]}...", flush=True)
        assert np.all(n_ref >= 0)
        np.testing.assert_array_equal(n_new, n_ref)
        np.testing.assert_array_equal(o_new, o_ref)


def test_noalloc_rejects_oversized_request():
    """A request beyond the fixed scratch is refused on the host before any
    device work, and a valid call afterwards still agrees."""
    import speculative_decoding_02_amd as sd
    B, K, V = 1 << 16, 63, 1024
    T = torch.zeros((1, 1, 1), device="cuda")  # never read: the size check comes first
    with pytest.raises(sd.SpecError) as e:
        sd.binding._check(sd.binding.lib().spec_accept_reject_noalloc(
            T.data_ptr(), T.data_ptr(), T.data_ptr(), B, K, V, 1, T.data_ptr(), 0, 0,
            T.data_ptr(), T.data_ptr(), None))
    assert e.value.code == sd.SPEC_ERR_CAPACITY
    T, D, d, pos = _inputs(3, 2, 512, 0.1, 13)
    o_ref, n_ref = _run(sd.spec_accept_reject, T, D, d, pos, False)
    o_new, n_new = _run(sd.spec_accept_reject_noalloc, T, D, d, pos, False)
    np.testing.assert_array_equal(n_new, n_ref)
    np.testing.assert_array_equal(o_new, o_ref)
