"""The C ABI library on a host without a GPU: it loads, exports every symbol the
header declares, sizes workspaces, and rejects invalid arguments before any
device work (no compute call is made here)."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_channel_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kda.LIB_PATH):
        from gated_delta_rule_channel_amd import build
        build.build()
    return kda.load_library()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert _declared() == sorted(kda.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError):
        kda.load_library(str(tmp_path / "nope.so"))


def test_status_strings(lib):
    assert kda.status_string(0) == "KDA_SUCCESS"
    assert kda.status_string(1) == "KDA_ERROR_INVALID_VALUE"
    assert kda.status_string(3) == "KDA_ERROR_WORKSPACE"
    assert kda.status_string(99).startswith("KDA_ERROR")


def test_workspace_size(lib):
    # chunk slots: B * ceil(T/64) fixed-length, floor(T/64) + N packed
    # per (chunk, head): W, Qd, KdT at 2.5 bytes per element and A_qk, U at 3 for bf16 input,
    # everything at 4 for fp32 input; exp(G_end) in fp32
    slots = 128
    header = ((slots * 16 + 255) // 256) * 256 + 256
    for dtype, nb, eb in ((kda.KDA_DTYPE_BF16, 2.5, 3), (kda.KDA_DTYPE_F32, 4, 4)):
        per_block = int(nb * 3 * 64 * 128 + eb * (64 * 128 + 64 * 64)) + 128 * 4
        n = kda.workspace_size(1, 8192, 64, 128, 128, 1, False, dtype)
        assert n == header + slots * 64 * ((per_block + 255) // 256 * 256)
    n2 = kda.workspace_size(1, 105872, 64, 128, 128, 8, True, kda.KDA_DTYPE_BF16)
    assert n2 > kda.workspace_size(1, 105872 - 64 * 8, 64, 128, 128, 8, True, kda.KDA_DTYPE_BF16)
    with pytest.raises(kda.KDAError):
        kda.workspace_size(1, 64, 1, 48, 64, 1, False, kda.KDA_DTYPE_F32)
    with pytest.raises(kda.KDAError):
        kda.workspace_size(2, 64, 1, 64, 64, 2, True, kda.KDA_DTYPE_F32)   # packed needs B == 1
    with pytest.raises(kda.KDAError):
        kda.workspace_size(1, 0, 1, 64, 64, 1, False, kda.KDA_DTYPE_F32)


FAKE = 0x10000  # never dereferenced: every call below fails host validation first


def _fwd(lib, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, scale=1.0, h0=None, ht=None, o=FAKE,
             cu=None, N=1, B=1, T=64, H=1, Dk=64, Dv=64, dtype=0, odtype=0, ws=None, wsb=0,
             stream=None)
    a.update(over)
    return lib.kda_fwd_chunked(a["q"], a["k"], a["v"], a["g"], a["beta"], a["scale"], a["h0"],
                               a["ht"], a["o"], a["cu"], a["N"], a["B"], a["T"], a["H"],
                               a["Dk"], a["Dv"], a["dtype"], a["odtype"], a["ws"], a["wsb"],
                               a["stream"])


def test_prefill_validation(lib):
    E = kda.KDA_ERROR_INVALID_VALUE
    assert _fwd(lib, q=None) == E
    assert _fwd(lib, o=None) == E
    assert _fwd(lib, Dk=48) == E
    assert _fwd(lib, Dv=256) == E
    assert _fwd(lib, T=0) == E
    assert _fwd(lib, H=-1) == E
    assert _fwd(lib, dtype=7) == E
    assert _fwd(lib, odtype=5) == E
    assert _fwd(lib, cu=FAKE, B=2, N=2) == E             # packed input requires B == 1
    assert _fwd(lib, cu=FAKE, N=0) == E
    assert _fwd(lib, k=FAKE + 4) == E                    # misaligned
    assert _fwd(lib, ht=FAKE + 8) == E
    assert _fwd(lib) == kda.KDA_ERROR_WORKSPACE          # no workspace
    assert _fwd(lib, ws=FAKE, wsb=10) == kda.KDA_ERROR_WORKSPACE
    assert _fwd(lib, ws=FAKE + 16, wsb=1 << 40) == kda.KDA_ERROR_WORKSPACE   # not 256-aligned


def test_decode_validation(lib):
    E = kda.KDA_ERROR_INVALID_VALUE
    f = lambda **o: lib.kda_decode_step(o.get("q", FAKE), FAKE, FAKE, FAKE, FAKE, 1.0,
                                        o.get("state", FAKE), FAKE, o.get("N", 4), 2,
                                        o.get("Dk", 64), o.get("Dv", 64), o.get("dtype", 1),
                                        o.get("odtype", 0), None)
    assert f(q=None) == E
    assert f(state=None) == E
    assert f(N=0) == E
    assert f(Dk=24) == E
    assert f(Dv=512) == E
    assert f(dtype=2) == E
    assert f(odtype=3) == E
    assert f(state=FAKE + 4) == E


def test_binding_rejects_mismatched_arguments():
    """The binding checks shapes and dtypes on the host before anything reaches the
    library (a wrong shape would otherwise make a kernel read past a buffer)."""
    import torch
    kda = pytest.importorskip("gated_delta_rule_channel_amd")
    B, T, H, D = 1, 64, 2, 16
    q = torch.zeros(B, T, H, D, dtype=torch.bfloat16)
    g = torch.zeros(B, T, H, D)
    beta = torch.zeros(B, T, H, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="v has shape"):
        kda.fwd_chunked(q, q, torch.zeros(B, T + 1, H, D, dtype=torch.bfloat16), g, beta)
    with pytest.raises(TypeError, match="share one dtype"):
        kda.fwd_chunked(q, q, torch.zeros(B, T, H, D), g, beta)
    with pytest.raises(ValueError, match="beta has shape"):
        kda.fwd_chunked(q, q, q, g, torch.zeros(B, T, H + 1, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="initial_state has shape"):
        kda.fwd_chunked(q, q, q, g, beta, initial_state=torch.zeros(B, H, D, D + 1))
    with pytest.raises(ValueError, match="contiguous GPU"):
        kda.fwd_chunked(q, q, q, g, beta)                     # well formed, but on the CPU
    N = 3
    qd = torch.zeros(N, H, D)
    st = torch.zeros(N, H, D, D)
    with pytest.raises(ValueError, match="state has shape"):
        kda.decode_step(qd, qd, qd, qd, torch.zeros(N, H), torch.zeros(N, H, D, 2 * D))
    with pytest.raises(ValueError, match="g has shape"):
        kda.decode_step(qd, qd, qd, torch.zeros(N, H, D + 16), torch.zeros(N, H), st)
    with pytest.raises(ValueError, match="contiguous GPU"):
        kda.decode_step(qd, qd, qd, qd, torch.zeros(N, H), st)


def test_binding_gdn_takes_one_gate_per_token():
    """The Gated DeltaNet calls take g [B,T,H] (prefill) and [N,H] (decode) and refuse the
    per-channel shape; the KDA calls refuse the scalar one."""
    import torch
    kda = pytest.importorskip("gated_delta_rule_channel_amd")
    B, T, H, D = 1, 64, 2, 16
    q = torch.zeros(B, T, H, D)
    beta = torch.zeros(B, T, H)
    with pytest.raises(ValueError, match="g has shape"):
        kda.gdn_fwd_chunked(q, q, q, torch.zeros(B, T, H, D), beta)
    with pytest.raises(ValueError, match="g has shape"):
        kda.fwd_chunked(q, q, q, torch.zeros(B, T, H), beta)
    with pytest.raises(ValueError, match="contiguous GPU"):
        kda.gdn_fwd_chunked(q, q, q, torch.zeros(B, T, H), beta)    # well formed, on the CPU
    N = 3
    qd = torch.zeros(N, H, D)
    st = torch.zeros(N, H, D, D)
    with pytest.raises(ValueError, match="g has shape"):
        kda.gdn_decode_step(qd, qd, qd, qd, torch.zeros(N, H), st)
    with pytest.raises(ValueError, match="contiguous GPU"):
        kda.gdn_decode_step(qd, qd, qd, torch.zeros(N, H), torch.zeros(N, H), st)


def test_gdn_entry_points_validate_like_kda(lib):
    """The scalar-gate entry points run the same host checks before any launch."""
    E = kda.KDA_ERROR_INVALID_VALUE
    g = lambda **o: lib.kda_gdn_fwd_chunked(
        o.get("q", FAKE), FAKE, FAKE, o.get("g", FAKE), FAKE, 1.0, None, None, FAKE, None, 1, 1,
        64, 1, o.get("Dk", 64), 64, 0, 0, o.get("ws", None), o.get("wsb", 0), None)
    assert g(q=None) == E
    assert g(g=None) == E
    assert g(Dk=48) == E
    assert g(g=FAKE + 4) == E
    assert g() == kda.KDA_ERROR_WORKSPACE
    d = lambda **o: lib.kda_gdn_decode_step(FAKE, FAKE, FAKE, o.get("g", FAKE), FAKE, 1.0, FAKE,
                                            FAKE, o.get("N", 4), 2, 64, 64, 1, 0, None)
    assert d(g=None) == E
    assert d(N=0) == E
    assert d(g=FAKE + 8) == E


def test_serving_entry_points_validate(lib):
    """Host checks of the serving-state calls (nothing reaches the device)."""
    E = kda.KDA_ERROR_INVALID_VALUE
    m = lambda **o: lib.kda_decode_multi(
        o.get("q", FAKE), FAKE, FAKE, FAKE, FAKE, 1.0, o.get("pool", FAKE), o.get("P", 4),
        o.get("slots", None), o.get("snap", None), FAKE, o.get("N", 4), o.get("T", 2), 2,
        o.get("Dk", 64), 64, 1, 0, None)
    assert m(q=None) == E
    assert m(pool=None) == E
    assert m(T=0) == E
    assert m(P=3) == E                        # no slot table: one state per request needed
    assert m(Dk=40) == E
    assert m(snap=FAKE + 8) == E              # misaligned snapshots
    assert m(slots=FAKE + 2, P=8) == E        # misaligned slot table
    c = lambda **o: lib.kda_state_copy(o.get("dst", FAKE), 4, o.get("ds", FAKE), FAKE, 4, FAKE,
                                       o.get("pairs", 2), 2, 64, o.get("Dv", 64), None)
    assert c(pairs=0, dst=None) == kda.KDA_SUCCESS      # nothing to copy
    assert c(dst=None) == E
    assert c(pairs=-1) == E
    assert c(Dv=24) == E
    assert c(ds=FAKE + 2) == E
    assert c(pairs=70000) == kda.KDA_ERROR_NOT_SUPPORTED


def test_binding_serving_shapes():
    import torch
    kda_ = pytest.importorskip("gated_delta_rule_channel_amd")
    N, T, H, D = 2, 3, 2, 16
    q = torch.zeros(N, T, H, D)
    beta = torch.zeros(N, T, H)
    pool = torch.zeros(4, H, D, D)
    with pytest.raises(ValueError, match="beta has shape"):
        kda_.decode_multi(q, q, q, q, torch.zeros(N, T), pool)
    with pytest.raises(ValueError, match="pool has shape"):
        kda_.decode_multi(q, q, q, q, beta, torch.zeros(4, H, D, 2 * D))
    with pytest.raises(TypeError, match="slots must be int32"):
        kda_.decode_multi(q, q, q, q, beta, pool, slots=torch.zeros(N, dtype=torch.int64))
    with pytest.raises(ValueError, match="one state per request"):
        kda_.decode_multi(q, q, q, q, beta, torch.zeros(1, H, D, D))
    with pytest.raises(ValueError, match="contiguous GPU"):
        kda_.decode_multi(q, q, q, q, beta, pool)
    s = torch.zeros(3, dtype=torch.int32)
    with pytest.raises(ValueError, match="same H, Dk, Dv"):
        kda_.state_copy(pool, s, torch.zeros(4, H, D, 2 * D), s)
    with pytest.raises(ValueError, match="one length"):
        kda_.state_copy(pool, s, pool, torch.zeros(2, dtype=torch.int32))


def test_prepare_inputs_validates(lib):
    E = kda.KDA_ERROR_INVALID_VALUE
    p = lambda **o: lib.kda_prepare_inputs(
        o.get("q", FAKE), FAKE, FAKE, o.get("b", FAKE), 1.0, FAKE, FAKE, o.get("g", FAKE),
        o.get("bo", FAKE), o.get("tokens", 8), o.get("H", 2), o.get("Dk", 64), o.get("dt", 1),
        None)
    assert p(q=None) == E
    assert p(g=None) == E
    assert p(tokens=0) == E
    assert p(Dk=48) == E
    assert p(dt=3) == E
    assert p(g=FAKE + 4) == E                 # g_out not 16-byte aligned
    assert p(bo=FAKE + 1) == E                # beta_out not element-aligned
    assert p(tokens=1 << 34) == kda.KDA_ERROR_NOT_SUPPORTED
