"""Gated DeltaNet (scalar gate) on the GPU, through the C ABI, against the float64 oracle.

Both outputs o and final states ht are compared element by element on the
same seeded inputs the oracle receives, with the bounds of the KDA tests.
"""
import dataclasses

import numpy as np
import pytest
import torch

import gated_delta_rule_channel_amd as kda
from gated_delta_rule_channel_amd import inputs as I
from oracle import native
from tests.parity_util import check

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _gpu(x: I.PrefillInputs, scale=None, out_dtype=None):
    q, k, v, g, b = (t.to(DEV) for t in (x.q, x.k, x.v, x.g, x.beta))
    cu = None if x.cu_seqlens is None else x.cu_seqlens.to(DEV)
    h0 = None if x.h0 is None else x.h0.to(DEV)
    o, ht = kda.gdn_fwd_chunked(q, k, v, g, b, scale=x.scale if scale is None else scale,
                                initial_state=h0, cu_seqlens=cu, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), ht.cpu().numpy()


def _compare(x, dtype, scale=None):
    s = x.scale if scale is None else scale
    o_ref, ht_ref = native.gdn_prefill(x.q, x.k, x.v, x.g, x.beta, scale=s, h0=x.h0,
                                       cu_seqlens=None if x.cu_seqlens is None
                                       else x.cu_seqlens.numpy())
    o, ht = _gpu(x, scale=scale)
    check("o", o, o_ref, dtype)
    check("ht", ht, ht_ref, dtype)
    return o, ht


@pytest.mark.parametrize("wid", [0, 1])
def test_gdn_small_workloads_f32(wid):
    w = I.WORKLOADS[wid]
    print(f"[gdn] {w.name}", flush=True)
    _compare(I.gdn_prefill_inputs(w), "f32")


def test_gdn_main_size_full():
    """B1 T8192 H64 d128 bf16 with a scalar gate: every head against the oracle."""
    w = I.WORKLOADS[2]
    print(f"[gdn] {w.name}", flush=True)
    _compare(I.gdn_prefill_inputs(w), w.dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gdn_varlen_edges(dtype):
    """Packed sequences with empty, one-token, exact-chunk and ragged lengths, with h0."""
    w = dataclasses.replace(I.WORKLOADS[4], H=3, Dk=64, Dv=32, dtype=dtype, h0=True)
    x = I.gdn_prefill_inputs(w, lengths=[0, 1, 64, 130, 0, 63, 200])
    print(f"[gdn] varlen edges {dtype}", flush=True)
    _, ht = _compare(x, dtype, scale=0.8)
    np.testing.assert_array_equal(ht[0], x.h0[0].numpy())
    np.testing.assert_array_equal(ht[4], x.h0[4].numpy())


@pytest.mark.parametrize("B,T,H,Dk,Dv,dtype", [(2, 77, 2, 16, 128, "f32"), (1, 250, 3, 128, 16, "bf16"),
                                               (3, 129, 1, 32, 64, "bf16"), (1, 1, 2, 64, 64, "f32")])
def test_gdn_ragged_shapes(B, T, H, Dk, Dv, dtype):
    w = dataclasses.replace(I.WORKLOADS[1], B=B, T=T, H=H, Dk=Dk, Dv=Dv, dtype=dtype)
    print(f"[gdn] B{B} T{T} H{H} {Dk}x{Dv} {dtype}", flush=True)
    _compare(I.gdn_prefill_inputs(w), dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gdn_steep_gate_pairwise_path(dtype):
    """Scalar log-decays of -30 .. -80 on some tokens push their 16-token blocks past the
    factorisation bound (the pairwise path); g = 0 on others."""
    w = dataclasses.replace(I.WORKLOADS[1], B=1, T=192, H=2, Dk=64, Dv=64, dtype=dtype)
    x = I.gdn_prefill_inputs(w)
    g = x.g.clone()
    rng = np.random.default_rng(4321)
    idx = rng.choice(192, size=12, replace=False)
    g[0, idx, :] = torch.from_numpy(-rng.uniform(30.0, 80.0, size=(12, 2))).float()
    g[0, 100:110, :] = 0.0
    x.g = g
    print(f"[gdn] steep gate {dtype}", flush=True)
    _compare(x, dtype)


def test_gdn_equals_kda_with_repeated_gate():
    """The scalar-gate path and the per-channel path agree when g is repeated over the
    channels (the two read the gate differently and share everything after it)."""
    w = dataclasses.replace(I.WORKLOADS[2], T=700, H=4)
    x = I.gdn_prefill_inputs(w)
    print("[gdn] vs kda with repeated gate", flush=True)
    q, k, v, g, b = (t.to(DEV) for t in (x.q, x.k, x.v, x.g, x.beta))
    o1, h1 = kda.gdn_fwd_chunked(q, k, v, g, b)
    gk = g[..., None].expand(*g.shape, q.shape[-1]).contiguous()
    o2, h2 = kda.fwd_chunked(q, k, v, gk, b)
    torch.cuda.synchronize()
    check("o gdn vs kda", o1.cpu().numpy(), o2.cpu().numpy(), "f32")
    check("ht gdn vs kda", h1.cpu().numpy(), h2.cpu().numpy(), "f32")


def test_gdn_bf16_output_is_rounded_fp32_output():
    w = dataclasses.replace(I.WORKLOADS[2], T=300, H=3)
    x = I.gdn_prefill_inputs(w)
    print("[gdn] bf16 output", flush=True)
    o32, h32 = _gpu(x)
    o16, h16 = _gpu(x, out_dtype=torch.bfloat16)
    np.testing.assert_array_equal(o16, torch.from_numpy(o32).to(torch.bfloat16).float().numpy())
    np.testing.assert_array_equal(h16, h32)


# --- decode ----------------------------------------------------------------------------------
def _decode(x: I.DecodeInputs, scale=1.0):
    q, k, v, g, b = (t.to(DEV) for t in (x.q, x.k, x.v, x.g, x.beta))
    st = x.state.to(DEV)
    o = kda.gdn_decode_step(q, k, v, g, b, st, scale=scale)
    torch.cuda.synchronize()
    return o.cpu().numpy(), st.cpu().numpy()


def test_gdn_decode_full_size():
    """256 requests x 64 heads x 128 x 128 fp32 states, scalar gate per (request, head)."""
    w = I.WORKLOADS[3]
    print(f"[gdn] decode {w.name}", flush=True)
    x = I.gdn_decode_inputs(w)
    o_ref, S_ref = native.gdn_decode(x.q, x.k, x.v, x.g, x.beta, x.state)
    o, S = _decode(x)
    check("o", o, o_ref, w.dtype)
    check("state", S, S_ref, w.dtype)


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 128), (128, 16), (64, 64)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gdn_decode_shapes(dk, dv, dtype):
    w = dataclasses.replace(I.WORKLOADS[3], Dk=dk, Dv=dv, dtype=dtype, H=3, N=5)
    print(f"[gdn] decode dk={dk} dv={dv} {dtype}", flush=True)
    x = I.gdn_decode_inputs(w)
    o_ref, S_ref = native.gdn_decode(x.q, x.k, x.v, x.g, x.beta, x.state, scale=0.6)
    o, S = _decode(x, scale=0.6)
    check("o", o, o_ref, dtype)
    check("state", S, S_ref, dtype)


def test_gdn_decode_steps_equal_prefill():
    """T decode steps against a carried state equal one prefill over the same tokens."""
    x = I.gdn_prefill_inputs(I.WORKLOADS[1], heads=[0, 1], T=70)
    print("[gdn] decode steps vs prefill", flush=True)
    o_pf, ht_pf = kda.gdn_fwd_chunked(*(t.to(DEV) for t in (x.q, x.k, x.v, x.g, x.beta)),
                                      initial_state=x.h0.to(DEV))
    st = x.h0.to(DEV).clone()
    outs = []
    for t in range(x.q.shape[1]):
        sl = lambda a: a[:, t].contiguous().to(DEV)
        outs.append(kda.gdn_decode_step(sl(x.q), sl(x.k), sl(x.v), sl(x.g), sl(x.beta), st))
    torch.cuda.synchronize()
    o_dec = torch.stack(outs, dim=1).cpu().numpy()
    check("o(decode) vs o(prefill)", o_dec, o_pf.cpu().numpy(), "f32")
    check("state(decode) vs ht(prefill)", st.cpu().numpy(), ht_pf.cpu().numpy(), "f32")
