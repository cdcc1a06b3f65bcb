"""Chunked-prefill parity on the GPU (through the C ABI) against the float64 oracle.

Every case compares both the outputs o and the final states ht, element by
element, on the same seeded inputs the oracle receives.
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


def _gpu(x: I.PrefillInputs, scale=None, h0=None, alias=False, output_final_state=True):
    q, k, v, g, b = (t.to(DEV) for t in (x.q, x.k, x.v, x.g, x.beta))
    cu = None if x.cu_seqlens is None else x.cu_seqlens.to(DEV)
    init = (x.h0 if h0 is None else h0)
    init = None if init is None else init.to(DEV)
    fs = init if (alias and init is not None) else None
    o, ht = kda.fwd_chunked(q, k, v, g, b, scale=x.scale if scale is None else scale,
                            initial_state=init, cu_seqlens=cu, final_state=fs,
                            output_final_state=output_final_state)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), None if ht is None else ht.cpu().numpy()


def _ref(x: I.PrefillInputs, scale=None, h0=None):
    return native.prefill(x.q, x.k, x.v, x.g, x.beta, scale=x.scale if scale is None else scale,
                          h0=x.h0 if h0 is None else h0,
                          cu_seqlens=None if x.cu_seqlens is None else x.cu_seqlens.numpy())


def _compare(x, dtype, **kw):
    o_ref, ht_ref = _ref(x, **{k: v for k, v in kw.items() if k in ("scale", "h0")})
    o, ht = _gpu(x, **kw)
    fo = check("o", o, o_ref, dtype)
    fs = check("ht", ht, ht_ref, dtype)
    return fo, fs


@pytest.mark.parametrize("wid", [0, 1])
def test_small_workloads_f32(wid):
    w = I.WORKLOADS[wid]
    print(f"[prefill] {w.name}", flush=True)
    _compare(I.prefill_inputs(w), w.dtype)


def test_main_prefill_full():
    """B1 T8192 H64 d128 bf16: every head against the oracle."""
    w = I.WORKLOADS[2]
    print(f"[prefill] {w.name}", flush=True)
    _compare(I.prefill_inputs(w), w.dtype)


def test_batched_full_heads_with_ragged_tail():
    """B2 T4100 H64 d128 bf16, the main workload's generators and launch shape with two
    sequences of a partial last chunk: every head against the oracle."""
    w = dataclasses.replace(I.WORKLOADS[2], B=2, T=4100)
    print(f"[prefill] {w.name} B2 T4100", flush=True)
    _compare(I.prefill_inputs(w), w.dtype)


def test_varlen_long_context_full():
    """8 packed sequences (lengths ~U[1024, 32768]) with near-0 and near-1 decay channels.

    The GPU runs every head at full size; the oracle checks four sampled heads
    (heads are independent, so the sampled heads' inputs are the same draws)."""
    w = I.WORKLOADS[4]
    print(f"[prefill] {w.name}", flush=True)
    x = I.prefill_inputs(w)
    o, ht = _gpu(x)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(ht))
    sample = [0, 21, 42, 63]
    xs = I.prefill_inputs(w, heads=sample)
    o_ref, ht_ref = _ref(xs)
    check("o[sampled heads]", o[:, :, sample], o_ref, w.dtype)
    check("ht[sampled heads]", ht[:, sample], ht_ref, w.dtype)


CASES = [
    # (B, T, H, Dk, Dv, dtype)
    (1, 1, 2, 64, 64, "f32"),
    (3, 63, 2, 32, 64, "f32"),
    (2, 65, 3, 64, 128, "f32"),
    (1, 130, 2, 128, 32, "f32"),
    (2, 200, 2, 16, 16, "f32"),
    (1, 257, 2, 128, 128, "f32"),
    (2, 100, 2, 128, 128, "bf16"),
    (1, 300, 3, 64, 16, "bf16"),
    (3, 77, 2, 16, 128, "bf16"),
    (3, 77, 2, 16, 128, "f32"),
    (1, 90, 2, 16, 64, "bf16"),
    (2, 64, 2, 32, 32, "bf16"),
]


@pytest.mark.parametrize("B,T,H,Dk,Dv,dtype", CASES)
def test_ragged_shapes(B, T, H, Dk, Dv, dtype):
    w = dataclasses.replace(I.WORKLOADS[1], B=B, T=T, H=H, Dk=Dk, Dv=Dv, dtype=dtype,
                            g_factor=True)
    print(f"[prefill] B{B} T{T} H{H} dk{Dk} dv{Dv} {dtype}", flush=True)
    _compare(I.prefill_inputs(w), dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_varlen_edges(dtype):
    """Zero-length, single-token, exact-chunk and ragged sequences, with an initial state."""
    w = dataclasses.replace(I.WORKLOADS[4], dtype=dtype, Dk=64, Dv=64, h0=True)
    x = I.prefill_inputs(w, heads=[1, 2, 3], lengths=[0, 1, 64, 65, 200, 0, 129])
    print(f"[prefill] varlen edges {dtype}", flush=True)
    o_ref, ht_ref = _ref(x)
    o, ht = _gpu(x)
    check("o", o, o_ref, dtype)
    check("ht", ht, ht_ref, dtype)
    # an empty sequence hands its initial state through unchanged
    np.testing.assert_array_equal(ht[0], x.h0[0].numpy())
    np.testing.assert_array_equal(ht[5], x.h0[5].numpy())


def test_alias_initial_and_final_state():
    w = I.WORKLOADS[1]
    x = I.prefill_inputs(w, heads=[0, 1], T=150)
    print("[prefill] h0 == ht", flush=True)
    o_ref, ht_ref = _ref(x)
    o, ht = _gpu(x, alias=True)
    check("o", o, o_ref, "f32")
    check("ht (aliased)", ht, ht_ref, "f32")


def test_scale_and_no_final_state():
    w = I.WORKLOADS[1]
    x = I.prefill_inputs(w, heads=[2], T=96)
    print("[prefill] scale 0.5, no ht", flush=True)
    o_ref, _ = _ref(x, scale=0.5)
    o, ht = _gpu(x, scale=0.5, output_final_state=False)
    assert ht is None
    check("o", o, o_ref, "f32")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_steep_decay_pairwise_path(dtype):
    """Log-decays of -30 .. -80 per token in some channels push the 16-token blocks past the
    factorisation bound, so those blocks take the pairwise path; near-zero decays as well."""
    w = dataclasses.replace(I.WORKLOADS[1], B=1, T=192, H=2, Dk=64, Dv=64, dtype=dtype)
    x = I.prefill_inputs(w)
    g = x.g.clone()
    rng = np.random.default_rng(1234)
    steep = torch.from_numpy(-rng.uniform(30.0, 80.0, size=(1, 192, 2, 5))).float()
    g[..., :5] = steep
    g[..., 5:9] = 0.0
    x.g = g
    print(f"[prefill] steep decay {dtype}", flush=True)
    _compare(x, dtype)


def _mild_decay(x, seed):
    rng = np.random.default_rng(seed)
    return torch.from_numpy(-rng.uniform(0.0, 0.02, size=tuple(x.g.shape))).float()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gate_closed_beta_is_pure_decay(dtype):
    """beta = 0 writes nothing: the state only decays, S_t = diag(exp(g_t)) S_(t-1), and
    o_t = scale q_t^T diag(exp(G_t)) h0 with G_t the running sum of g. Checked against that
    closed form as well as the oracle, over three chunks and a ragged tail."""
    w = dataclasses.replace(I.WORKLOADS[1], B=1, T=200, H=2, Dk=64, Dv=64, dtype=dtype)
    x = I.prefill_inputs(w)
    x.g = _mild_decay(x, 77)
    x.beta = torch.zeros_like(x.beta)
    print(f"[prefill] beta = 0 {dtype}", flush=True)
    fo, fs = _compare(x, dtype)
    o, ht = _gpu(x)
    G = np.cumsum(x.g.double().numpy(), axis=1)                        # [1, T, H, Dk]
    h0 = x.h0.double().numpy()[0]                                      # [H, Dk, Dv]
    q = x.q.double().numpy()[0]                                        # [T, H, Dk]
    o_cf = x.scale * np.einsum("thi,hij->thj", q * np.exp(G[0]), h0)[None]
    ht_cf = (np.exp(G[0, -1])[:, :, None] * h0)[None]
    check("o (closed form)", o, o_cf, dtype)
    check("ht (closed form)", ht, ht_cf, dtype)


def test_no_decay_unit_beta_stores_last_pair():
    """g = 0, beta = 1 is the plain delta rule: with a unit-norm key the write overwrites the
    value stored along k, so k_T^T S_T = v_T for the last token of every head."""
    w = dataclasses.replace(I.WORKLOADS[1], B=1, T=200, H=3, Dk=64, Dv=64)
    x = I.prefill_inputs(w)
    x.g = torch.zeros_like(x.g)
    x.beta = torch.ones_like(x.beta)
    print("[prefill] g = 0, beta = 1", flush=True)
    _compare(x, "f32")
    _, ht = _gpu(x)
    k_last = x.k.double().numpy()[0, -1]                               # [H, Dk]
    got = np.einsum("hi,hij->hj", k_last, ht[0].astype(np.float64))
    check("k_T^T S_T vs v_T", got, x.v.double().numpy()[0, -1], "f32")


def test_resume_split_equals_one_pass():
    """[0, T1) then [T1, T) with ht -> h0 equals one pass; T1 is not a chunk multiple."""
    w = I.WORKLOADS[1]
    x = I.prefill_inputs(w, heads=[0, 3], T=400)
    T1 = 150
    print("[prefill] resume split", flush=True)
    o_ref, ht_ref = _ref(x)

    def part(sl, h0):
        y = dataclasses.replace(x, q=x.q[:, sl].contiguous(), k=x.k[:, sl].contiguous(),
                                v=x.v[:, sl].contiguous(), g=x.g[:, sl].contiguous(),
                                beta=x.beta[:, sl].contiguous(), h0=h0)
        return _gpu(y)

    oa, ha = part(slice(0, T1), x.h0)
    ob, hb = part(slice(T1, None), torch.from_numpy(ha))
    check("o", np.concatenate([oa, ob], axis=1), o_ref, "f32")
    check("ht", hb, ht_ref, "f32")


def test_deterministic_bitwise():
    w = I.WORKLOADS[2]
    x = I.prefill_inputs(w, heads=list(range(8)))
    print("[prefill] determinism", flush=True)
    o1, h1 = _gpu(x)
    o2, h2 = _gpu(x)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(h1, h2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bf16_output_is_rounded_fp32_output(dtype):
    """A bfloat16 o is the float32 o rounded to nearest even, element for element."""
    w = dataclasses.replace(I.WORKLOADS[2], T=300, H=3, dtype=dtype)
    x = I.prefill_inputs(w)
    print(f"[prefill] bf16 output {dtype}", flush=True)
    q, k, v, g, b = (t.to(DEV) for t in (x.q, x.k, x.v, x.g, x.beta))
    o32, h32 = kda.fwd_chunked(q, k, v, g, b)
    o16, h16 = kda.fwd_chunked(q, k, v, g, b, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert o16.dtype == torch.bfloat16
    assert torch.equal(o16, o32.to(torch.bfloat16))
    assert torch.equal(h16, h32)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_nan_in_one_head_stays_in_that_head(dtype):
    """Heads are independent recurrences: a NaN in one head's inputs (a value, a gate and a
    query element at different tokens) must leave every other head's o and final state
    equal to the oracle's, and must not hide that head's own corruption."""
    w = dataclasses.replace(I.WORKLOADS[2], T=300, H=8, dtype=dtype)
    x = I.prefill_inputs(w)
    bad = 3
    x.v[0, 100, bad, 5] = float("nan")
    x.g[0, 150, bad, 7] = float("nan")
    x.q[0, 220, bad, 9] = float("nan")
    print(f"[prefill] NaN in head {bad} {dtype}", flush=True)
    o_ref, ht_ref = _ref(x)
    o, ht = _gpu(x)
    keep = [h for h in range(w.H) if h != bad]
    check("o (other heads)", o[:, :, keep], o_ref[:, :, keep], dtype)
    check("ht (other heads)", ht[:, keep], ht_ref[:, keep], dtype)
    assert not np.all(np.isfinite(o[:, 100:, bad])), "the NaN head shows no corruption"
    assert not np.all(np.isfinite(ht[:, bad]))


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128)])
def test_out_of_range_cu_seqlens_are_clamped(dtype, d):
    """A cu_seqlens that breaks its documented precondition (a negative start, an end past
    the tokens) is clamped to [0, T] on the device: the call stays inside its buffers and
    gives exactly the result of the clamped offsets."""
    w = dataclasses.replace(I.WORKLOADS[4], dtype=dtype, Dk=d, Dv=d, h0=True)
    x = I.prefill_inputs(w, heads=[0, 1], lengths=[50, 70])             # 120 tokens
    dev = torch.device("cuda:0")
    args = [t.to(dev) for t in (x.q, x.k, x.v, x.g, x.beta)]
    print(f"[prefill] clamped cu_seqlens {dtype} d{d}", flush=True)
    good = torch.tensor([0, 50, 120], dtype=torch.int32, device=dev)
    bad = torch.tensor([-5, 50, 200], dtype=torch.int32, device=dev)
    o1, h1 = kda.fwd_chunked(*args, initial_state=x.h0.to(dev), cu_seqlens=good)
    o2, h2 = kda.fwd_chunked(*args, initial_state=x.h0.to(dev), cu_seqlens=bad)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
