"""The allocation-free attention call against the regular one: the same kernels serve both, so
the outputs must be identical bit for bit.  Two calls in a row, the second on a smaller
problem, the first with the repair epilogue."""

import numpy as np
import pytest
import torch

from synthetic import make_custom

from gpu_common import dev, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bsa():
    import block_sparse_attention_antidiagonal_amd as m

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def _case(bsa, seed, S, Hq, Hkv, D):
    wl = make_custom(seed, B=1, Hq=Hq, Hkv=Hkv, S=S, D=D, dtype="bf16")
    lay = bsa.cluster_layout(torch.from_numpy(wl.labels).cuda(), wl.C)
    q, k, v = dev(wl.q, "bf16"), dev(wl.k, "bf16"), dev(wl.v, "bf16")
    kv = bsa.kv_pack(k, v, lay)
    mask = bsa.mask_from_keep(torch.from_numpy(wl.mask).cuda())
    return wl, lay, q, kv, mask


def test_noalloc_matches_workspace_call(bsa):
    assert bsa._lib.load().bsa_sparse_attention_static_scratch_bytes() == 48 << 20
    # first call: larger problem, with the repair epilogue
    say("noalloc call 1")
    wl, lay, q, kv, mask = _case(bsa, 501, 3000, 4, 2, 128)
    rng = np.random.default_rng(0)
    A = torch.from_numpy((rng.standard_normal((1, 4, 128, 128)) * 0.2).astype(np.float32)).cuda()
    c = torch.from_numpy((rng.standard_normal((1, 4, 128)) * 0.1).astype(np.float32)).cuda()
    want = bsa.block_sparse_attention(q, kv, lay, mask, True, wl.scale, A=A, c=c)
    got = torch.empty_like(q)
    bsa.block_sparse_attention_noalloc(q, kv, lay, mask, got, True, wl.scale, A=A, c=c)
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    # second call: a smaller problem (other shapes and cluster counts), hard drop, with lse
    say("noalloc call 2")
    wl2, lay2, q2, kv2, mask2 = _case(bsa, 502, 700, 2, 1, 64)
    want2, lse_want = bsa.block_sparse_attention(q2, kv2, lay2, mask2, False, wl2.scale, return_lse=True)
    got2 = torch.empty_like(q2)
    lse = torch.empty(1, 2, 700, dtype=torch.float32, device=q2.device)
    bsa.block_sparse_attention_noalloc(q2, kv2, lay2, mask2, got2, False, wl2.scale, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(got2, want2)
    assert torch.equal(lse, lse_want)
