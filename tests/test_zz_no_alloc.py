"""GPU check of fa_bwd_noalloc, the backward entry point that allocates nothing:
its gradients must equal those of fa_bwd (the same kernels, with the row-sum
workspace in the library's static array instead of a caller buffer) bit for
bit, on two calls in a row, the second smaller than the first, so that the
second call runs over what the first left in the shared workspace."""
import pytest
import torch

import synthetic
from tests import gpu_checks as G

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _inputs(B, H, N, d, seed, causal):
    import exact_tiled_attention_18_amd as fa
    q, k, v = (x.to(DEV) for x in synthetic.draw_qkv(B, H, N, d, seed=seed, dtype="bf16"))
    do = synthetic.draw_qkv(B, H, N, d, seed=seed + 1, dtype="bf16")[0].to(DEV)
    o, lse = fa.fa_fwd(q, k, v, causal=causal)
    return q, k, v, o, do, lse


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_noalloc_matches_fa_bwd_twice(fa, causal, d):
    for (B, H, N), seed in (((2, 8, 1000), 71), ((1, 2, 300), 73)):
        G.log(f"case bwd_noalloc B{B} H{H} N{N} d{d} causal={causal}")
        q, k, v, o, do, lse = _inputs(B, H, N, d, seed, causal)
        ref = fa.fa_bwd(q, k, v, o, do, lse, causal=causal)
        got = fa.fa_bwd_noalloc(q, k, v, o, do, lse, causal=causal)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(a, b), name


def test_noalloc_full_size_then_small(fa):
    """The largest bench workload's backward shape (B1 H32 N16384 d128 causal, 2^19 rows
    of the 2^22-row workspace), then a small one."""
    for (B, H, N, d), seed in (((1, 32, 16384, 128), 81), ((1, 1, 129, 128), 83)):
        G.log(f"case bwd_noalloc B{B} H{H} N{N} d{d} causal")
        q, k, v, o, do, lse = _inputs(B, H, N, d, seed, True)
        ref = fa.fa_bwd(q, k, v, o, do, lse, causal=True)
        got = fa.fa_bwd_noalloc(q, k, v, o, do, lse, causal=True)
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(got, ref))
        del q, k, v, o, do, lse, ref, got


def test_noalloc_rejects_problems_beyond_the_workspace(fa):
    n = fa.FA_BWD_NOALLOC_MAX_ROWS // 2 + 1
    q = torch.zeros((1, 2, n, 64), dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros((1, 2, n), dtype=torch.float32, device=DEV)
    with pytest.raises(fa.FAError) as e:
        fa.fa_bwd_noalloc(q, q, q, q, q, lse)
    assert e.value.status == fa.FA_ERR_SCRATCH
