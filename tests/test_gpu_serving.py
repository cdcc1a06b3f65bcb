"""Serving-state operations on the GPU: multi-token decode against a slot-indexed state pool
with per-token snapshots, and state copies for forks and rollbacks, through the C ABI.

Outputs and states are compared with the float64 oracle's decode step applied token by
token; copies are compared bit for bit.
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


def _tokens(w, N, T, heads=None):
    """Decode-workload draws for N requests x T tokens, laid out [N, T, H, D]."""
    x = I.decode_inputs(w, heads=heads, N=N * T, with_state=False)
    r = lambda a: a.view(N, T, *a.shape[1:]).contiguous()
    return r(x.q), r(x.k), r(x.v), r(x.g), r(x.beta)


def _pool(w, P, H, seed):
    rng = np.random.default_rng(seed)
    return torch.from_numpy(0.1 * rng.standard_normal((P, H, w.Dk, w.Dv))).float()


def _oracle_steps(q, k, v, g, beta, S0, scale=1.0, keep_all=True):
    """The oracle's decode step applied to tokens 0 .. T-1 in order: o [N,T,H,Dv] and the
    state after every token [N,T,H,Dk,Dv] (only the last one, [N,1,...], if not keep_all)."""
    N, T = q.shape[:2]
    S = S0.double().numpy()
    outs, snaps = [], []
    for t in range(T):
        o, S = native.decode(q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t], S, scale=scale)
        outs.append(o)
        if keep_all or t == T - 1:
            snaps.append(S)
    return np.stack(outs, axis=1), np.stack(snaps, axis=1)


@pytest.mark.parametrize("dk,dv,dtype,T", [(128, 128, "bf16", 4), (64, 32, "f32", 4),
                                           (16, 128, "bf16", 4), (128, 16, "f32", 4),
                                           (128, 128, "bf16", 11), (32, 64, "f32", 17),
                                           (16, 16, "bf16", 9)])
def test_decode_multi_slots_and_snapshots(dk, dv, dtype, T):
    """Token counts past one staged group of 8 (11, 17) and a ragged last group."""
    w = dataclasses.replace(I.WORKLOADS[3], Dk=dk, Dv=dv, dtype=dtype, H=3)
    N, P = 5, 9
    print(f"[serving] decode_multi dk={dk} dv={dv} {dtype} T={T}", flush=True)
    q, k, v, g, beta = _tokens(w, N, T)
    pool = _pool(w, P, 3, 11)
    slots = torch.tensor([7, 2, 0, 5, 3], dtype=torch.int32)
    o_ref, snap_ref = _oracle_steps(q, k, v, g, beta, pool[slots.long()], scale=0.9)
    pd = pool.to(DEV)
    snaps = torch.empty((N, T, 3, dk, dv), device=DEV)
    o = kda.decode_multi(*(t.to(DEV) for t in (q, k, v, g, beta)), pd, slots=slots.to(DEV),
                         snapshots=snaps, scale=0.9)
    torch.cuda.synchronize()
    check("o", o.cpu().numpy(), o_ref, dtype)
    check("snapshots", snaps.cpu().numpy(), snap_ref, dtype)
    after = pd.cpu()
    check("pool slots", after[slots.long()].numpy(), snap_ref[:, -1], dtype)
    untouched = [i for i in range(P) if i not in slots.tolist()]
    assert torch.equal(after[untouched], pool[untouched])


def test_decode_multi_full_size_speculative_verify():
    """256 requests x 4 drafted tokens x 64 heads x 128 x 128 against a pool of 320 slots."""
    w = I.WORKLOADS[3]
    N, T, P = 256, 4, 320
    print("[serving] decode_multi N256 T4 H64", flush=True)
    q, k, v, g, beta = _tokens(w, N, T)
    pool = _pool(w, P, 64, 12)
    slots = torch.from_numpy(np.random.default_rng(13).permutation(P)[:N].astype(np.int32))
    o_ref, snap_ref = _oracle_steps(q, k, v, g, beta, pool[slots.long()], keep_all=False)
    pd = pool.to(DEV)
    o = kda.decode_multi(*(t.to(DEV) for t in (q, k, v, g, beta)), pd, slots=slots.to(DEV))
    torch.cuda.synchronize()
    check("o", o.cpu().numpy(), o_ref, "bf16")
    check("pool slots", pd.cpu()[slots.long()].numpy(), snap_ref[:, -1], "bf16")


def test_decode_multi_one_token_equals_decode_step():
    w = I.WORKLOADS[3]
    x = I.decode_inputs(w, heads=list(range(8)), N=16)
    print("[serving] T = 1 vs decode_step", flush=True)
    a = [t.to(DEV) for t in (x.q, x.k, x.v, x.g, x.beta)]
    s1, s2 = x.state.to(DEV), x.state.to(DEV)
    o1 = kda.decode_step(*a, s1)
    o2 = kda.decode_multi(*(t[:, None].contiguous() for t in a), s2)
    torch.cuda.synchronize()
    check("o", o2[:, 0].cpu().numpy(), o1.cpu().numpy(), "f32")
    check("state", s2.cpu().numpy(), s1.cpu().numpy(), "f32")


def test_decode_multi_equals_prefill():
    """T tokens of decode_multi equal a prefill of the same T tokens from the same state."""
    x = I.prefill_inputs(I.WORKLOADS[1], heads=[0, 1, 2], T=70)
    print("[serving] decode_multi vs prefill", flush=True)
    a = [t.to(DEV) for t in (x.q, x.k, x.v, x.g, x.beta)]
    o_pf, ht = kda.fwd_chunked(*a, initial_state=x.h0.to(DEV))
    pool = x.h0.to(DEV).clone()
    o_md = kda.decode_multi(*a, pool)
    torch.cuda.synchronize()
    check("o", o_md.cpu().numpy(), o_pf.cpu().numpy(), "f32")
    check("state", pool.cpu().numpy(), ht.cpu().numpy(), "f32")


def test_rollback_restores_the_accepted_prefix():
    """Verify T = 5 drafted tokens with snapshots, accept m of them per request, restore the
    snapshot of token m - 1 into the slot: bit for bit the state that decoding only the m
    accepted tokens leaves, and the outputs of those tokens match too."""
    w = I.WORKLOADS[3]
    N, T, P, H = 6, 5, 10, 4
    print("[serving] rollback", flush=True)
    q, k, v, g, beta = _tokens(w, N, T, heads=list(range(H)))
    pool0 = _pool(w, P, H, 14).to(DEV)
    slots = torch.tensor([9, 1, 4, 6, 0, 3], dtype=torch.int32, device=DEV)
    accepted = [1, 5, 3, 2, 4, 1]
    a = [t.to(DEV) for t in (q, k, v, g, beta)]
    pool = pool0.clone()
    snaps = torch.empty((N, T, H, w.Dk, w.Dv), device=DEV)
    o_all = kda.decode_multi(*a, pool, slots=slots, snapshots=snaps)
    src = torch.tensor([n * T + m - 1 for n, m in enumerate(accepted)], dtype=torch.int32,
                       device=DEV)
    kda.state_copy(pool, slots, snaps.view(N * T, H, w.Dk, w.Dv), src)
    torch.cuda.synchronize()
    for n, m in enumerate(accepted):
        ref_pool = pool0.clone()
        sl = slots[n:n + 1]
        # fresh copies: a view of request n starts off the 16-byte alignment the ABI asks for
        o_m = kda.decode_multi(*(t[n:n + 1, :m].clone() for t in a), ref_pool, slots=sl.clone())
        torch.cuda.synchronize()
        assert torch.equal(pool[slots[n].item()], ref_pool[slots[n].item()]), n
        assert torch.equal(o_all[n, :m], o_m[0]), n


def test_state_copy_forks_and_skips_out_of_range():
    w = I.WORKLOADS[3]
    P, H = 12, 3
    print("[serving] state_copy", flush=True)
    pool = _pool(dataclasses.replace(w, Dk=64, Dv=128), P, H, 15).to(DEV)
    before = pool.clone()
    src = torch.tensor([0, 3, 5, 2], dtype=torch.int32, device=DEV)
    dst = torch.tensor([7, 8, 99, 11], dtype=torch.int32, device=DEV)    # 99: out of range
    kda.state_copy(pool, dst, pool, src)
    torch.cuda.synchronize()
    assert torch.equal(pool[7], before[0])
    assert torch.equal(pool[8], before[3])
    assert torch.equal(pool[11], before[2])
    keep = [i for i in range(P) if i not in (7, 8, 11)]
    assert torch.equal(pool[keep], before[keep])


def test_decode_multi_skips_out_of_range_slot():
    w = dataclasses.replace(I.WORKLOADS[3], H=2)
    N, T, P = 3, 2, 4
    print("[serving] decode_multi out-of-range slot", flush=True)
    q, k, v, g, beta = _tokens(w, N, T)
    pool = _pool(w, P, 2, 16).to(DEV)
    before = pool.clone()
    slots = torch.tensor([1, 4, 2], dtype=torch.int32, device=DEV)   # request 1: slot 4 >= P
    o = torch.full((N, T, 2, w.Dv), 7.0, device=DEV)
    kda.decode_multi(*(t.to(DEV) for t in (q, k, v, g, beta)), pool, slots=slots, out=o)
    torch.cuda.synchronize()
    assert torch.all(o[1] == 7.0)
    assert torch.equal(pool[[0, 3]], before[[0, 3]])
    assert not torch.equal(pool[1], before[1]) and not torch.equal(pool[2], before[2])
