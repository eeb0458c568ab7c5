"""gptk_attn_bwd_noalloc (the allocation-free attention backward, whose rowsum(dO*O)
scratch is the library's own device array) against gptk_attn_bwd (the same kernels fed
a caller-owned scratch) on the same inputs, two calls in a row, the second smaller:
the results must be identical bit for bit.  The over-size request is refused before
anything runs."""
import numpy as np
import pytest
import torch

from gpt_pretraining_step_train_amd import binding as B
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    torch.cuda.set_device(0)


def _inputs(Bn, T, H, Hkv, hd, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    qkv = torch.randn(Bn * T, (H + 2 * Hkv) * hd, device="cuda", generator=g).bfloat16()
    dO = torch.randn(Bn * T, H * hd, device="cuda", generator=g).bfloat16()
    return qkv, dO


# (B, T, H, Hkv, hd, window): the d24 attention shape at batch 4, then a smaller ragged
# grouped-query case with a sliding window
CASES = [(4, 2048, 12, 12, 128, 0), (2, 300, 6, 2, 64, 100)]


def test_noalloc_attention_backward_matches_the_workspace_entry_point():
    for Bn, T, H, Hkv, hd, win in CASES:
        say("attention backward without allocation", (Bn, T, H, Hkv, hd, win))
        qkv, dO = _inputs(Bn, T, H, Hkv, hd, Bn * T + H)
        o = torch.empty(Bn * T, H * hd, device="cuda", dtype=torch.bfloat16)
        lse = torch.empty(Bn * H * T, device="cuda")
        B.attn_fwd(B.GPT_BF16, qkv, o, lse, Bn, T, H, hd, win, n_kv=Hkv)
        D = torch.empty(Bn * H * T, device="cuda")
        ref = torch.empty_like(qkv)
        B.attn_bwd(B.GPT_BF16, qkv, o, dO, lse, D, ref, Bn, T, H, hd, win, n_kv=Hkv)
        got = torch.full_like(qkv, float("nan"))
        B.attn_bwd_noalloc(B.GPT_BF16, qkv, o, dO, lse, got, Bn, T, H, hd, win, n_kv=Hkv)
        torch.cuda.synchronize()
        r, gt = ref.view(torch.int16).cpu().numpy(), got.view(torch.int16).cpu().numpy()
        np.testing.assert_array_equal(gt, r)
        assert np.isfinite(got.float().cpu().numpy()).all()


def test_noalloc_refuses_more_than_its_scratch():
    x = torch.empty(8, device="cuda")
    rc = B.lib().gptk_attn_bwd_noalloc(B.GPT_BF16, B._ptr(x), B._ptr(x), B._ptr(x), B._ptr(x), B._ptr(x),
                                       64, 2048, 16, 16, 128, 0, B._stream())
    assert rc == 1  # 64 * 16 * 2048 > 2^20 entries
