"""kda_fwd_chunked_noalloc (the prefill on the library's built-in device scratch) against
kda_fwd_chunked with a caller workspace, through the C ABI.

The two run the same kernels on the same inputs, so o and the final state must agree bit
for bit (well inside the parity bound). Two calls in a row, the second smaller than the
first, check that nothing left in the shared scratch by one call changes the next one's
results; a call too large for the scratch must be rejected with KDA_ERROR_WORKSPACE.
"""
import dataclasses

import numpy as np
import pytest
import torch

import gated_delta_rule_channel_amd as kda
from gated_delta_rule_channel_amd import inputs as I
from tests.parity_util import check

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _args(x):
    t = [a.to(DEV) for a in (x.q, x.k, x.v, x.g, x.beta)]
    h0 = None if x.h0 is None else x.h0.to(DEV)
    cu = None if x.cu_seqlens is None else x.cu_seqlens.to(DEV)
    return t, h0, cu


def _both(x):
    t, h0, cu = _args(x)
    B, T, H, Dk = t[0].shape
    Dv = t[2].shape[-1]
    N = B if cu is None else cu.numel() - 1
    nan = float("nan")
    o_ref = torch.full((B, T, H, Dv), nan, device=DEV)
    h_ref = torch.full((N, H, Dk, Dv), nan, device=DEV)
    o_na = torch.full((B, T, H, Dv), nan, device=DEV)
    h_na = torch.full((N, H, Dk, Dv), nan, device=DEV)
    kda.fwd_chunked(*t, scale=x.scale, initial_state=h0, cu_seqlens=cu, out=o_ref,
                    final_state=h_ref)
    kda.fwd_chunked_noalloc(*t, scale=x.scale, initial_state=h0, cu_seqlens=cu, out=o_na,
                            final_state=h_na)
    torch.cuda.synchronize()
    return (o_ref.cpu().numpy(), h_ref.cpu().numpy()), (o_na.cpu().numpy(), h_na.cpu().numpy())


def _same(ref, got, dtype):
    (o_ref, h_ref), (o, h) = ref, got
    check("o (no-alloc vs workspace)", o, o_ref, dtype)
    check("ht (no-alloc vs workspace)", h, h_ref, dtype)
    np.testing.assert_array_equal(o, o_ref)
    np.testing.assert_array_equal(h, h_ref)


def test_noalloc_matches_workspace_call_twice_second_smaller():
    # first call: 16 heads x 16 chunks of the main workload's generators (about 25 MB of
    # scratch); second: packed sequences with an initial state, fp32, far smaller
    w1 = dataclasses.replace(I.WORKLOADS[2], T=1000, H=16)
    x1 = I.prefill_inputs(w1)
    print("[no-alloc] call 1: B1 T1000 H16 d128 bf16", flush=True)
    ref, got = _both(x1)
    _same(ref, got, "bf16")
    w2 = dataclasses.replace(I.WORKLOADS[4], dtype="f32", Dk=64, Dv=32, h0=True)
    x2 = I.prefill_inputs(w2, heads=[0, 1, 2], lengths=[70, 0, 129, 5])
    print("[no-alloc] call 2: packed 4 sequences, H3 d64/32 f32, h0", flush=True)
    ref, got = _both(x2)
    _same(ref, got, "f32")


def test_noalloc_rejects_a_call_beyond_the_scratch():
    B, T, H, D = 1, 8192, 64, 128
    need = kda.workspace_size(B, T, H, D, D, B, False, kda.KDA_DTYPE_BF16)
    assert need > kda.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, T, H, D), dtype=torch.bfloat16, device=DEV)
    g = torch.zeros((B, T, H, D), dtype=torch.float32, device=DEV)
    beta = torch.zeros((B, T, H), dtype=torch.bfloat16, device=DEV)
    print("[no-alloc] oversize call is rejected", flush=True)
    with pytest.raises(kda.KDAError) as ei:
        kda.fwd_chunked_noalloc(q, q, q, g, beta)
    assert ei.value.status == kda.KDA_ERROR_WORKSPACE
