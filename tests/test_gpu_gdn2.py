"""Gated DeltaNet-2 (erase gate b, write gate w) on the GPU, through the C ABI, against the
float64 oracle.

Both outputs o and final states ht are compared element by element on the same seeded
inputs the oracle receives, with the bounds of the KDA tests.
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


def _gpu(x: I.PrefillInputs, b, w, scale=None, out_dtype=None):
    q, k, v, g, eb, ew = (t.to(DEV) for t in (x.q, x.k, x.v, x.g, b, w))
    cu = None if x.cu_seqlens is None else x.cu_seqlens.to(DEV)
    h0 = None if x.h0 is None else x.h0.to(DEV)
    o, ht = kda.gdn2_fwd_chunked(q, k, v, g, eb, ew, scale=x.scale if scale is None else scale,
                                 initial_state=h0, cu_seqlens=cu, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), ht.cpu().numpy()


def _compare(x, b, w, dtype, scale=None):
    s = x.scale if scale is None else scale
    o_ref, ht_ref = native.gdn2_prefill(x.q, x.k, x.v, x.g, b, w, scale=s, h0=x.h0,
                                        cu_seqlens=None if x.cu_seqlens is None
                                        else x.cu_seqlens.numpy())
    o, ht = _gpu(x, b, w, scale=scale)
    check("o", o, o_ref, dtype)
    check("ht", ht, ht_ref, dtype)
    return o, ht


@pytest.mark.parametrize("wid", [0, 1])
def test_gdn2_small_workloads_f32(wid):
    w_ = I.WORKLOADS[wid]
    print(f"[gdn2] {w_.name}", flush=True)
    _compare(*I.gdn2_prefill_inputs(w_), "f32")


def test_gdn2_main_size_full():
    """B1 T8192 H64 d128 bf16 with erase and write gates: every head against the oracle."""
    w_ = I.WORKLOADS[2]
    print(f"[gdn2] {w_.name}", flush=True)
    _compare(*I.gdn2_prefill_inputs(w_), w_.dtype)


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 64), ("bf16", 128)])
def test_gdn2_varlen_edges(dtype, d):
    """Packed sequences with empty, one-token, exact-chunk and ragged lengths, with h0."""
    w_ = dataclasses.replace(I.WORKLOADS[4], H=3, Dk=d, Dv=d // 2 if d == 64 else d,
                             dtype=dtype, h0=True)
    x, b, w = I.gdn2_prefill_inputs(w_, lengths=[0, 1, 64, 130, 0, 63, 200])
    print(f"[gdn2] varlen edges {dtype} d{d}", flush=True)
    _, ht = _compare(x, b, w, dtype, scale=0.8)
    np.testing.assert_array_equal(ht[0], x.h0[0].numpy())
    np.testing.assert_array_equal(ht[4], x.h0[4].numpy())


@pytest.mark.parametrize("B,T,H,Dk,Dv,dtype", [(2, 77, 2, 16, 128, "f32"), (1, 250, 3, 128, 16, "bf16"),
                                               (3, 129, 1, 32, 64, "bf16"), (1, 1, 2, 64, 64, "f32"),
                                               (2, 100, 3, 128, 128, "bf16")])
def test_gdn2_ragged_shapes(B, T, H, Dk, Dv, dtype):
    w_ = dataclasses.replace(I.WORKLOADS[1], B=B, T=T, H=H, Dk=Dk, Dv=Dv, dtype=dtype)
    print(f"[gdn2] B{B} T{T} H{H} {Dk}x{Dv} {dtype}", flush=True)
    _compare(*I.gdn2_prefill_inputs(w_), dtype)


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 64), ("bf16", 128)])
def test_gdn2_steep_decay_pairwise_path(dtype, d):
    """Log-decays of -30 .. -80 in some channels send blocks through the pairwise path,
    where the erase gate enters the exact pair sums."""
    w_ = dataclasses.replace(I.WORKLOADS[1], B=1, T=192, H=2, Dk=d, Dv=d, dtype=dtype)
    x, b, w = I.gdn2_prefill_inputs(w_)
    g = x.g.clone()
    rng = np.random.default_rng(2468)
    g[..., :5] = torch.from_numpy(-rng.uniform(30.0, 80.0, size=(1, 192, 2, 5))).float()
    x.g = g
    print(f"[gdn2] steep decay {dtype}", flush=True)
    _compare(x, b, w, dtype)


def test_gdn2_zero_erase_unit_write():
    """b = 0, w = 1: nothing is erased, every value is added at its key (gated linear
    attention)."""
    w_ = dataclasses.replace(I.WORKLOADS[1], B=1, T=200, H=2)
    x, b, w = I.gdn2_prefill_inputs(w_)
    print("[gdn2] b = 0, w = 1", flush=True)
    _compare(x, torch.zeros_like(b), torch.ones_like(w), "f32")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gdn2_collapses_to_kda_on_the_gpu(dtype):
    """b = beta 1 and w = beta 1 reproduce the KDA path (the two form W and U through
    different roundings, so they agree to float32 accuracy, not bit for bit)."""
    w_ = dataclasses.replace(I.WORKLOADS[2], T=700, H=4, dtype=dtype)
    x = I.prefill_inputs(w_)
    print(f"[gdn2] vs kda, {dtype}", flush=True)
    q, k, v, g, beta = (t.to(DEV) for t in (x.q, x.k, x.v, x.g, x.beta))
    eb = beta[..., None].expand(*beta.shape, q.shape[-1]).contiguous()
    ew = beta[..., None].expand(*beta.shape, v.shape[-1]).contiguous()
    o1, h1 = kda.gdn2_fwd_chunked(q, k, v, g, eb, ew)
    o2, h2 = kda.fwd_chunked(q, k, v, g, beta)
    torch.cuda.synchronize()
    check("o gdn2 vs kda", o1.cpu().numpy(), o2.cpu().numpy(), "f32")
    check("ht gdn2 vs kda", h1.cpu().numpy(), h2.cpu().numpy(), "f32")


# --- decode ----------------------------------------------------------------------------------
def _decode(x: I.DecodeInputs, b, w, scale=1.0):
    q, k, v, g, eb, ew = (t.to(DEV) for t in (x.q, x.k, x.v, x.g, b, w))
    st = x.state.to(DEV)
    o = kda.gdn2_decode_step(q, k, v, g, eb, ew, st, scale=scale)
    torch.cuda.synchronize()
    return o.cpu().numpy(), st.cpu().numpy()


def test_gdn2_decode_full_size():
    """256 requests x 64 heads x 128 x 128 fp32 states with erase and write gates."""
    w_ = I.WORKLOADS[3]
    print(f"[gdn2] decode {w_.name}", flush=True)
    x, b, w = I.gdn2_decode_inputs(w_)
    o_ref, S_ref = native.gdn2_decode(x.q, x.k, x.v, x.g, b, w, x.state)
    o, S = _decode(x, b, w)
    check("o", o, o_ref, w_.dtype)
    check("state", S, S_ref, w_.dtype)


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 128), (128, 16), (64, 64)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gdn2_decode_shapes(dk, dv, dtype):
    w_ = dataclasses.replace(I.WORKLOADS[3], Dk=dk, Dv=dv, dtype=dtype, H=3, N=5)
    print(f"[gdn2] decode dk={dk} dv={dv} {dtype}", flush=True)
    x, b, w = I.gdn2_decode_inputs(w_)
    o_ref, S_ref = native.gdn2_decode(x.q, x.k, x.v, x.g, b, w, x.state, scale=0.6)
    o, S = _decode(x, b, w, scale=0.6)
    check("o", o, o_ref, dtype)
    check("state", S, S_ref, dtype)


def test_gdn2_decode_steps_equal_prefill():
    """T decode steps against a carried state equal one prefill over the same tokens."""
    x, b, w = I.gdn2_prefill_inputs(I.WORKLOADS[1], heads=[0, 1], T=70)
    print("[gdn2] decode steps vs prefill", flush=True)
    o_pf, ht_pf = kda.gdn2_fwd_chunked(*(t.to(DEV) for t in (x.q, x.k, x.v, x.g, b, w)),
                                       initial_state=x.h0.to(DEV))
    st = x.h0.to(DEV).clone()
    outs = []
    for t in range(x.q.shape[1]):
        sl = lambda a: a[:, t].contiguous().to(DEV)
        outs.append(kda.gdn2_decode_step(sl(x.q), sl(x.k), sl(x.v), sl(x.g), sl(b), sl(w), st))
    torch.cuda.synchronize()
    o_dec = torch.stack(outs, dim=1).cpu().numpy()
    check("o(decode) vs o(prefill)", o_dec, o_pf.cpu().numpy(), "f32")
    check("state(decode) vs ht(prefill)", st.cpu().numpy(), ht_pf.cpu().numpy(), "f32")
