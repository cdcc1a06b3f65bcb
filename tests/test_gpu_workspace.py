"""Every workspace byte the state pass reads is written by the prep kernel of the same call.

The workspace is caller memory with no defined contents, and some regions of a block are
deliberately left unwritten (the all-zero second A_qk column half of token tiles 0 and 1).
Each case runs the same call on a workspace of zero bytes and on one of 0xFF bytes (NaN
as bfloat16 and as float32) and requires bitwise equal, finite results: on the bf16 d = 128
prep kernel in its KDA, raw-projection and Gated DeltaNet-2 modes, on the general prep
kernel (float32 input, head sizes below 128, Gated DeltaNet), and on packed input with an
initial state.
"""
import dataclasses

import numpy as np
import pytest
import torch

import gated_delta_rule_channel_amd as kda
from gated_delta_rule_channel_amd import inputs as I

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _same_on_poisoned_workspace(name, call, nbytes):
    print(f"[workspace] {name}: {nbytes} bytes", flush=True)
    outs = []
    for fill in (0x00, 0xFF):
        ws = torch.full((nbytes,), fill, dtype=torch.uint8, device=DEV)
        o, ht = call(ws)
        torch.cuda.synchronize()
        outs.append((o.float().cpu().numpy(), ht.cpu().numpy()))
    (o0, h0), (o1, h1) = outs
    assert np.all(np.isfinite(o0)) and np.all(np.isfinite(h0))
    np.testing.assert_array_equal(o1, o0)
    np.testing.assert_array_equal(h1, h0)


def _dev(*ts):
    return [t.to(DEV) for t in ts]


def _code(x):
    return kda.KDA_DTYPE_BF16 if x.q.dtype == torch.bfloat16 else kda.KDA_DTYPE_F32


@pytest.mark.parametrize("wid,dtype,T,H,D", [
    (2, "bf16", 300, 3, 128),      # the bf16 d = 128 prep kernel, ragged last chunk
    (1, "bf16", 150, 2, 64),       # the general prep kernel, bf16
    (1, "f32", 200, 2, 64),        # the general prep kernel, float32
])
def test_kda_fixed_length(wid, dtype, T, H, D):
    w = dataclasses.replace(I.WORKLOADS[wid], T=T, H=H, Dk=D, Dv=D, dtype=dtype)
    x = I.prefill_inputs(w)
    q, k, v, g, b = _dev(x.q, x.k, x.v, x.g, x.beta)
    B = q.shape[0]
    n = kda.workspace_size(B, T, H, D, D, B, False, _code(x))
    _same_on_poisoned_workspace(
        f"KDA B{B} T{T} H{H} d{D} {dtype}",
        lambda ws: kda.fwd_chunked(q, k, v, g, b, scale=x.scale, workspace=ws), n)


def test_kda_packed_with_initial_state():
    w = dataclasses.replace(I.WORKLOADS[4], h0=True)
    lengths = [70, 0, 129, 5]
    x = I.prefill_inputs(w, heads=[0, 1, 2], lengths=lengths)
    q, k, v, g, b, h0, cu = _dev(x.q, x.k, x.v, x.g, x.beta, x.h0, x.cu_seqlens)
    n = kda.workspace_size(1, q.shape[1], 3, 128, 128, len(lengths), True, _code(x))
    _same_on_poisoned_workspace(
        "KDA packed 4 sequences H3 d128 bf16, h0",
        lambda ws: kda.fwd_chunked(q, k, v, g, b, scale=x.scale, initial_state=h0,
                                   cu_seqlens=cu, workspace=ws), n)


def test_gated_deltanet():
    w = dataclasses.replace(I.WORKLOADS[2], T=300, H=3)
    x = I.gdn_prefill_inputs(w)
    q, k, v, g, b = _dev(x.q, x.k, x.v, x.g, x.beta)
    n = kda.workspace_size(1, 300, 3, 128, 128, 1, False, _code(x))
    _same_on_poisoned_workspace(
        "Gated DeltaNet T300 H3 d128 bf16",
        lambda ws: kda.gdn_fwd_chunked(q, k, v, g, b, scale=x.scale, workspace=ws), n)


def test_gated_deltanet_2():
    w = dataclasses.replace(I.WORKLOADS[2], T=300, H=3)
    x, eb, ew = I.gdn2_prefill_inputs(w)
    q, k, v, g, eb, ew = _dev(x.q, x.k, x.v, x.g, eb, ew)
    n = kda.workspace_size(1, 300, 3, 128, 128, 1, False, _code(x))
    _same_on_poisoned_workspace(
        "Gated DeltaNet-2 T300 H3 d128 bf16",
        lambda ws: kda.gdn2_fwd_chunked(q, k, v, g, eb, ew, scale=x.scale, workspace=ws), n)


def test_raw_projections():
    B, T, H, D = 1, 300, 3, 128
    rng = np.random.default_rng(17)
    mk = lambda *shape, s=1.0: torch.from_numpy(s * rng.standard_normal(shape)).to(torch.bfloat16)
    q, k, v, a = mk(B, T, H, D, s=2.0), mk(B, T, H, D, s=0.5), mk(B, T, H, D), mk(B, T, H, D, s=3.0)
    b = mk(B, T, H, s=2.0)
    q, k, v, a, b = _dev(q, k, v, a, b)
    n = kda.workspace_size(B, T, H, D, D, B, False, kda.KDA_DTYPE_BF16)
    _same_on_poisoned_workspace(
        "raw projections T300 H3 d128 bf16",
        lambda ws: kda.fwd_chunked_raw(q, k, v, a, b, scale=D ** -0.5, workspace=ws), n)
