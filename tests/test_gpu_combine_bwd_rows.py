"""Combine backward past one pass of its grid.

For rows of 512 or more 16-byte chunks (d >= 4096 in bf16) the combine
backward runs one workgroup per (token, slot) row for up to 2^20 rows and
steps the same workgroups over the rows after that. T = 131073 tokens at
d = 4096 with k = 8 gives 1,048,640 logical rows: token 131072's eight rows
are taken in the second pass, token 131071's are the last of the first.
Sampled tokens from both passes are compared with the fp64 oracle of the
combine backward (the return to source order of Support combined expert and
data parallelism in TrainerRank, Desired behavior).

Inputs are seeded draws on the device (torch's generator, not this library);
row_of_slot is a random permutation of the T*k rows, which is all the kernel
assumes of it. Bars derived from the arithmetic:
  dy[row] = bf16(w * dout) from an fp32 product: per element within 2^-8 of
  the fp64 value (one bf16 rounding, 2^-9, plus the fp32 product's 2^-24);
  dtopk_w: an fp32 dot product of 4096 terms in any order is within
  (n - 1) 2^-24 sum|dout_i y_i| < 2^-12 sum|dout_i y_i| of the exact sum.
"""
import numpy as np
import pytest

import oracle
from tests.parity_util import to_host64

pytestmark = pytest.mark.gpu

T, D, K, E = 131073, 4096, 8, 64


def test_combine_bwd_second_pass_rows():
    import torch
    import token_dispatch_grouped_amd as moe
    from token_dispatch_grouped_amd import _lib as L

    R = T * K
    g = torch.Generator(device="cuda")
    g.manual_seed(20260)
    dout = torch.randn(T, D, generator=g, device="cuda", dtype=torch.bfloat16)
    y = torch.randn(R, D, generator=g, device="cuda", dtype=torch.bfloat16)
    topk_w = torch.rand(T, K, generator=g, device="cuda", dtype=torch.float32)
    ros = torch.randperm(R, generator=g, device="cuda", dtype=torch.int64).to(torch.int32).view(T, K).contiguous()
    dy = torch.full((R, D), float("nan"), device="cuda", dtype=torch.bfloat16)
    dtw = torch.full((T, K), float("nan"), device="cuda", dtype=torch.float32)
    shape = L.make_shape(T, D, E, K, 64, moe.MOE_DTYPE_BF16)
    print(f"combine_bwd rows: T={T} d={D} k={K}", flush=True)
    moe.moe_unpermute_combine_bwd(shape, dout, y, topk_w, ros, dy, dtw)
    torch.cuda.synchronize()

    sample = np.array([0, 1, 7, 8, 12345, 65536, 131064, 131071, 131072])
    idx = torch.from_numpy(sample).cuda()
    rows = ros[idx].long()                                  # [S, K]
    dout_s = to_host64(dout[idx])
    y_s = to_host64(y[rows.view(-1)])                       # slot order
    w_s = topk_w[idx].double().cpu().numpy()
    local = np.arange(len(sample) * K, dtype=np.int32).reshape(len(sample), K)
    dy_ref, dw_ref = oracle.unpermute_combine_bwd(dout_s, y_s, w_s, local)

    dy_gpu = to_host64(dy[rows.view(-1)])
    assert np.all(np.isfinite(dy_gpu)), "a sampled dy row was not written"
    assert np.all(np.abs(dy_gpu - dy_ref) <= 2.0 ** -8 * np.abs(dy_ref)), "dy outside one bf16 rounding"

    dw_gpu = dtw[idx].double().cpu().numpy()
    bound = 2.0 ** -12 * np.einsum("sd,skd->sk", np.abs(dout_s), np.abs(y_s.reshape(len(sample), K, D)))
    assert np.all(np.abs(dw_gpu - dw_ref) <= bound), "dtopk_w outside the fp32 summation bound"

    # every row of the second pass and of the last first-pass token is written
    tail = ros[torch.tensor([131071, 131072], device="cuda")].long().view(-1)
    assert torch.isfinite(dy[tail].float()).all().item()
    assert torch.isfinite(dtw).all().item(), "some dtopk_w entry was not written"
