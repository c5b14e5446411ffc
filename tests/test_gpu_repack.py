"""Repack kernels vs the oracle's row maps: bit exact for any row size."""
import numpy as np
import pytest
import torch

import shared_prompt_exact_amd as dk
from oracle import repack

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N,P,R,row_shape,dtype", [
    (4, 64, 32, (2, 64), torch.bfloat16),     # 256-byte rows, 128-bit path
    (3, 17, 5, (3,), torch.int32),           # 12-byte rows, 32-bit path
    (5, 9, 7, (7,), torch.uint8),            # odd row size, byte path
    (2, 0, 11, (4, 8), torch.float32),       # no prompt
    (3, 13, 0, (1,), torch.int64),           # no response
    (32, 811, 97, (8, 128), torch.bfloat16),  # many rows of 2 KiB
])
def test_gather_scatter_bit_exact(N, P, R, row_shape, dtype):
    print(f"repack N={N} P={P} R={R} row={row_shape} {dtype}", flush=True)
    g = torch.Generator().manual_seed(N * 1000 + P)
    rows_rep = N * (P + R)
    raw = torch.randint(0, 256, (rows_rep,) + row_shape + (torch.tensor([], dtype=dtype).element_size(),),
                        generator=g, dtype=torch.uint8)
    rep_host = raw.view(dtype).reshape((rows_rep,) + row_shape)
    rep = rep_host.cuda()
    packed = dk.dualkv_repack(rep, N, P, R, dk.DUALKV_GATHER)
    back = dk.dualkv_repack(packed, N, P, R, dk.DUALKV_SCATTER)
    torch.cuda.synchronize()
    exp_packed = repack.gather(rep_host.view(torch.uint8).numpy(), N, P, R)
    assert np.array_equal(packed.cpu().view(torch.uint8).numpy(), exp_packed)
    exp_back = repack.scatter(exp_packed, N, P, R)
    assert np.array_equal(back.cpu().view(torch.uint8).numpy(), exp_back)
