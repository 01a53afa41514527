"""The no-allocation variant of the Flat bucket search (sa_bucket_select_noalloc, scratch in a static device
array) against the workspace variant (sa_bucket_select) through the C ABI: the index lists, counts and chosen
buckets must agree bit-exactly, on two calls in a row of which the second is smaller (the array keeps the first
call's keys, which the second must not see), and once more at the largest size the array admits."""
import numpy as np
import pytest
import torch

import long_context_sparse_sa_amd as sa
from long_context_sparse_sa_amd import _lib

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _case(seed, L, nb, B, d=128):
    g = torch.Generator(device="cpu").manual_seed(seed)
    centres = torch.randn((nb, d), generator=g)
    assign = torch.randint(0, nb, (L,), generator=g, dtype=torch.int64)
    k = (centres[assign] + 0.3 * torch.randn((L, d), generator=g)).to(torch.bfloat16).to(DEV)
    q = torch.randn((B, d), generator=g).to(torch.bfloat16).to(DEV)
    reps, offsets, members = sa.sa_bucket_build(k, assign.to(torch.int32).to(DEV), nb)
    return q, reps, offsets, members


def _compare(seed, L, nb, B, top_b, n_sink, n_window, cap):
    q, reps, offsets, members = _case(seed, L, nb, B)
    t = torch.tensor([L - 1 - 37 * b for b in range(B)], dtype=torch.int32, device=DEV)
    ref = sa.sa_bucket_select(q, reps, offsets, members, L, top_b, n_sink, n_window, cap=cap, t=t,
                              return_buckets=True)
    # outputs prefilled with garbage: every entry must be written
    out = (torch.full((B, cap), 12345, dtype=torch.int32, device=DEV),
           torch.full((B,), 777, dtype=torch.int32, device=DEV),
           torch.full((B, top_b), -5, dtype=torch.int32, device=DEV))
    got = sa.sa_bucket_select_noalloc(q, reps, offsets, members, L, top_b, n_sink, n_window, t=t,
                                      return_buckets=True, out=out)
    torch.cuda.synchronize()
    for a, b in zip(got, ref):
        np.testing.assert_array_equal(a.cpu().numpy(), b.cpu().numpy())
    assert int(got[1].min().item()) > 0


def test_two_calls_second_smaller():
    _compare(0, L=1 << 18, nb=16384, B=8, top_b=32, n_sink=4, n_window=128, cap=8192)
    _compare(1, L=50_000, nb=1000, B=3, top_b=7, n_sink=2, n_window=16, cap=4096)


def test_largest_admitted_size_and_rejection():
    max_keys = _lib.load().sa_bucket_select_noalloc_max_keys()
    assert max_keys == 1 << 21
    nb = 1 << 17
    B = max_keys // nb  # 16 queries x 131072 buckets fill the array exactly
    _compare(2, L=1 << 20, nb=nb, B=B, top_b=16, n_sink=4, n_window=64, cap=2048)
    q, reps, offsets, members = _case(3, 1 << 18, nb, B + 1)
    with pytest.raises(sa.SAError) as e:
        sa.sa_bucket_select_noalloc(q, reps, offsets, members, 1 << 18, 16, cap=2048)
    assert e.value.status == 5  # SA_ERR_WORKSPACE: nothing launched
