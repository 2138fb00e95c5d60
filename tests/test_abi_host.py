"""The C ABI on a host without a GPU: the library loads, exports every symbol
include/rlk.h declares, and rejects bad arguments on the host before anything
is launched. No call here passes validation (no compute runs without a GPU)."""
import ctypes
import math
import os
import re

import pytest

from grpo_loss_rlk_amd import _native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
P = ctypes.c_void_p
FAKE = P(0x100000)          # a 256-aligned address that is never dereferenced
WS = P(0x200000)


@pytest.fixture(scope="module")
def L():
    return _native.lib()


def _declared():
    src = open(os.path.join(ROOT, "include", "rlk.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"\b(rlk_[a-z0-9_]+)\s*\(", src))


def test_exports_every_declared_symbol(L):
    declared = _declared()
    assert declared == set(_native.SIGNATURES), declared ^ set(_native.SIGNATURES)
    for name in declared:
        assert hasattr(L, name), name


def test_version_and_status_text(L):
    assert L.rlk_abi_version() == 2
    assert L.rlk_status_str(0) == b"ok"
    assert b"workspace" in L.rlk_status_str(3)


def _logits_call(L, **kw):
    a = dict(logits=FAKE, dtype=1, n=4, V=1000, stride=1000, targets=FAKE, T=0.7, p=0.95,
             t_row=None, p_row=None, top_k=0, k_row=None, lpf=FAKE, lpt=FAKE, ht=FAKE, hf=None,
             ns=None, th=None, fl=None, ws=WS, ws_bytes=1 << 20)
    a.update(kw)
    return L.rlk_logprob_from_logits(a["logits"], a["dtype"], a["n"], a["V"], a["stride"],
                                     a["targets"], a["T"], a["p"], a["t_row"], a["p_row"],
                                     a["top_k"], a["k_row"], a["lpf"], a["lpt"], a["ht"], a["hf"],
                                     a["ns"],
                                     a["th"], a["fl"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(top_k=-1), _native.RLK_EINVAL),
    (dict(top_k=5, ws=None), _native.RLK_EWORKSPACE),    # top-k is opt-in: accepted
    (dict(k_row=P(0x100002)), _native.RLK_EINVAL),      # per-row top-k not 4-byte aligned
    (dict(T=0.0), _native.RLK_EINVAL),
    (dict(T=-1.0), _native.RLK_EINVAL),
    (dict(T=math.nan), _native.RLK_EINVAL),
    (dict(T=math.inf), _native.RLK_EINVAL),
    (dict(p=0.0), _native.RLK_EINVAL),
    (dict(p=1.0000001), _native.RLK_EINVAL),
    (dict(p=math.nan), _native.RLK_EINVAL),
    (dict(dtype=7), _native.RLK_EINVAL),
    (dict(V=0), _native.RLK_EINVAL),
    (dict(V=(1 << 24) + 1, stride=(1 << 24) + 1), _native.RLK_EINVAL),
    (dict(stride=999), _native.RLK_EINVAL),
    (dict(n=-1), _native.RLK_EINVAL),
    (dict(logits=None), _native.RLK_EINVAL),
    (dict(targets=None), _native.RLK_EINVAL),
    (dict(lpt=None), _native.RLK_EINVAL),
    (dict(logits=P(0x100001)), _native.RLK_EINVAL),
    (dict(targets=P(0x100004)), _native.RLK_EINVAL),
    (dict(ws=None), _native.RLK_EWORKSPACE),
    (dict(ws=P(0x200010)), _native.RLK_EWORKSPACE),
    (dict(ws_bytes=0), _native.RLK_EWORKSPACE),
])
def test_logits_validation(L, kw, status):
    assert _logits_call(L, **kw) == status
    assert len(L.rlk_last_error()) > 0


def _noalloc_call(L, **kw):
    a = dict(logits=FAKE, dtype=1, n=4, V=1000, stride=1000, targets=FAKE, T=0.7, p=0.95,
             t_row=None, p_row=None, top_k=0, k_row=None, lpf=FAKE, lpt=FAKE, ht=FAKE)
    a.update(kw)
    return L.rlk_logprob_from_logits_noalloc(a["logits"], a["dtype"], a["n"], a["V"], a["stride"],
                                             a["targets"], a["T"], a["p"], a["t_row"],
                                             a["p_row"], a["top_k"], a["k_row"], a["lpf"],
                                             a["lpt"], a["ht"],
                                             None, None, None, None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(n=(1 << 20) + 1), _native.RLK_EINVAL),      # beyond the static scratch
    (dict(n=1 << 40), _native.RLK_EINVAL),
    (dict(top_k=-5), _native.RLK_EINVAL),
    (dict(T=0.0), _native.RLK_EINVAL),
    (dict(stride=999), _native.RLK_EINVAL),
    (dict(lpt=None), _native.RLK_EINVAL),
    (dict(n=-1), _native.RLK_EINVAL),
])
def test_noalloc_validation(L, kw, status):
    """The no-allocation entry point checks its arguments (and its row limit)
    on the host before it touches the GPU."""
    assert _noalloc_call(L, **kw) == status
    assert len(L.rlk_last_error()) > 0
    if kw.get("n", 0) > (1 << 20):
        assert b"no-allocation limit" in L.rlk_last_error()


def test_noalloc_empty_batch_is_a_noop(L):
    assert _noalloc_call(L, n=0, logits=None, targets=None) == 0


def test_logits_empty_batch_is_a_noop(L):
    assert _logits_call(L, n=0, logits=None, targets=None, ws=None) == 0


def test_workspace_queries(L):
    assert L.rlk_logprob_from_logits_workspace_size(4096, 151936, 1) >= 4096
    assert L.rlk_grpo_token_loss_workspace_size(1000, 32) > 0


def _grpo(L, **kw):
    prm = _native.GrpoParams(ctypes.sizeof(_native.GrpoParams), 2.0, 0.2, 0.28, 0.01, 1e-6, 1, 1,
                             0, 0, 0, 0, 0, 0.3, 0.5, 2.0)
    for k, v in kw.pop("prm", {}).items():
        setattr(prm, k, v)
    # cu_seqlens is a device array: its values are checked by the kernels, so
    # the host checks only its pointer and the sizes passed by value
    a = dict(lp_new=FAKE, lp_old=FAKE, lp_ref=FAKE, cu=FAKE, n=2, T=5, rewards=FAKE, adv=None,
             G=2, params=ctypes.byref(prm), loss=FAKE, grad=FAKE, status=None, ws=WS,
             ws_bytes=1 << 20)
    a.update(kw)
    return L.rlk_grpo_token_loss(a["lp_new"], a["lp_old"], a["lp_ref"], a["cu"], a["n"], a["T"],
                                 a["rewards"], a["adv"], a["G"], a["params"], a["loss"],
                                 a["grad"], None, None, None, None, a["status"], a["ws"],
                                 a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(params=None), _native.RLK_EINVAL),
    (dict(prm=dict(struct_size=4)), _native.RLK_EINVAL),
    (dict(prm=dict(tis_cap=0.0)), _native.RLK_EINVAL),
    (dict(prm=dict(eps_low=1.0)), _native.RLK_EINVAL),
    (dict(prm=dict(eps_high=-0.1)), _native.RLK_EINVAL),
    (dict(prm=dict(kl_coef=-1.0)), _native.RLK_EINVAL),
    (dict(prm=dict(std_ddof=2)), _native.RLK_EINVAL),
    (dict(T=-1), _native.RLK_EINVAL),
    (dict(T=(1 << 40) + 1), _native.RLK_EINVAL),
    (dict(n=0), _native.RLK_EINVAL),
    (dict(cu=None), _native.RLK_EINVAL),
    (dict(cu=P(0x100004)), _native.RLK_EINVAL),          # not 8-byte aligned
    (dict(status=P(0x100002)), _native.RLK_EINVAL),      # not 4-byte aligned
    (dict(adv=FAKE), _native.RLK_EINVAL),
    (dict(rewards=None), _native.RLK_EINVAL),
    (dict(G=3), _native.RLK_EINVAL),
    (dict(G=1), _native.RLK_EINVAL),
    (dict(lp_ref=None), _native.RLK_EINVAL),
    (dict(grad=None), _native.RLK_EINVAL),
    (dict(loss=None), _native.RLK_EINVAL),
    (dict(ws_bytes=8), _native.RLK_EWORKSPACE),
    # the first params layout (32 bytes) is accepted: defaults for the rest
    (dict(prm=dict(struct_size=32, ipo_eps=-1.0), ws_bytes=8), _native.RLK_EWORKSPACE),
    (dict(prm=dict(struct_size=31)), _native.RLK_EINVAL),
    (dict(prm=dict(loss_type=5)), _native.RLK_EINVAL),
    (dict(prm=dict(loss_type=-1)), _native.RLK_EINVAL),
    (dict(prm=dict(correction=2)), _native.RLK_EINVAL),
    (dict(prm=dict(aggregation=2)), _native.RLK_EINVAL),
    (dict(prm=dict(filter_zero_adv=2)), _native.RLK_EINVAL),
    (dict(prm=dict(baseline=2)), _native.RLK_EINVAL),
    (dict(prm=dict(ipo_eps=0.0)), _native.RLK_EINVAL),
    (dict(prm=dict(icepop_lo=0.0)), _native.RLK_EINVAL),
    (dict(prm=dict(icepop_lo=2.0, icepop_hi=1.0)), _native.RLK_EINVAL),
    (dict(prm=dict(aggregation=1), rewards=None, adv=FAKE, G=3), _native.RLK_EINVAL),
])
def test_grpo_validation(L, kw, status):
    assert _grpo(L, **kw) == status
    assert len(L.rlk_last_error()) > 0


def _fused(L, **kw):
    a = dict(h=FAKE, w=FAKE, n=4, H=128, V=1000, hs=128, wsd=128, targets=FAKE, T=1.0, p=1.0,
             top_k=0, lp=FAKE, ent=FAKE, saved=FAKE, ns=None, fl=None, ws=WS, ws_bytes=1 << 30)
    a.update(kw)
    return L.rlk_logprob_fused_linear(a["h"], a["w"], a["n"], a["H"], a["V"], a["hs"], a["wsd"],
                                      a["targets"], a["T"], a["p"], a["top_k"], a["lp"],
                                      a["ent"], a["saved"], a["ns"], a["fl"], a["ws"],
                                      a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(top_k=-3), _native.RLK_EINVAL),
    (dict(T=0.0), _native.RLK_EINVAL),
    (dict(p=1.5), _native.RLK_EINVAL),
    (dict(H=100, hs=128, wsd=128), _native.RLK_EINVAL),
    (dict(H=0, hs=128, wsd=128), _native.RLK_EINVAL),
    (dict(hs=120), _native.RLK_EINVAL),
    (dict(hs=132), _native.RLK_EINVAL),
    (dict(wsd=1 << 23), _native.RLK_EINVAL),
    (dict(V=0), _native.RLK_EINVAL),
    (dict(n=1 << 23), _native.RLK_EINVAL),
    (dict(h=None), _native.RLK_EINVAL),
    (dict(w=P(0x100008)), _native.RLK_EINVAL),
    (dict(lp=None), _native.RLK_EINVAL),
    (dict(ws=None), _native.RLK_EWORKSPACE),
    (dict(ws_bytes=16), _native.RLK_EWORKSPACE),
    (dict(p=0.9, ws_bytes=1 << 12), _native.RLK_EWORKSPACE),
])
def test_fused_validation(L, kw, status):
    assert _fused(L, **kw) == status
    assert len(L.rlk_last_error()) > 0


def _fused_bwd(L, **kw):
    a = dict(h=FAKE, w=FAKE, n=4, H=128, V=1000, hs=128, wsd=128, targets=FAKE, saved=FAKE,
             glp=FAKE, gh=None, T=1.0, p=1.0, top_k=0, dh=FAKE, dw=FAKE, ws=WS, ws_bytes=1 << 30)
    a.update(kw)
    return L.rlk_logprob_fused_linear_bwd(a["h"], a["w"], a["n"], a["H"], a["V"], a["hs"],
                                          a["wsd"], a["targets"], a["saved"], a["glp"], a["gh"],
                                          a["T"], a["p"], a["top_k"], a["dh"], a["dw"], a["ws"],
                                          a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(p=0.0), _native.RLK_EINVAL),
    (dict(top_k=-1), _native.RLK_EINVAL),
    (dict(T=math.inf), _native.RLK_EINVAL),
    (dict(H=96, hs=128, wsd=128), _native.RLK_EINVAL),
    (dict(V=1 << 23), _native.RLK_EINVAL),
    (dict(dw=None), _native.RLK_EINVAL),
    (dict(dh=None), _native.RLK_EINVAL),
    (dict(saved=None), _native.RLK_EINVAL),
    (dict(dw=P(0x100002)), _native.RLK_EINVAL),
    (dict(ws=None), _native.RLK_EWORKSPACE),
    (dict(ws_bytes=1 << 10), _native.RLK_EWORKSPACE),
])
def test_fused_bwd_validation(L, kw, status):
    assert _fused_bwd(L, **kw) == status
    assert len(L.rlk_last_error()) > 0


def test_fused_workspace_queries(L):
    # top-p < 1 stores a block of fp32 logits: 4096 rows x V (padded to 64) x 4 bytes
    assert L.rlk_logprob_fused_linear_workspace_size(8192, 4096, 151936, 0.95, 0) >= 4096 * 151936 * 4
    assert L.rlk_logprob_fused_linear_workspace_size(8192, 4096, 151936, 1.0, 0) < 4096 * 151936
    # top-k needs the stored logits at any top-p
    assert L.rlk_logprob_fused_linear_workspace_size(8192, 4096, 151936, 1.0, 50) >= 4096 * 151936 * 4
    # backward: W^T and h^T in bf16 plus two bf16 copies of one 32768-row chunk of G
    need = 2 * 4096 * 151936 + 2 * 4096 * 8192 + 2 * 2 * 8192 * 32768
    assert L.rlk_logprob_fused_linear_bwd_workspace_size(8192, 4096, 151936, 1.0) >= need


def _support(L, **kw):
    a = dict(logits=FAKE, dtype=1, n=4, V=1000, stride=1000, targets=FAKE, T=1.0, off=FAKE,
             ids=FAKE, nnz=10, p=0.0, k=0, lp=FAKE, ent=FAKE, fl=None, ws=WS, ws_bytes=1 << 30)
    a.update(kw)
    return L.rlk_logprob_from_support(a["logits"], a["dtype"], a["n"], a["V"], a["stride"],
                                      a["targets"], a["T"], a["off"], a["ids"], a["nnz"], a["p"],
                                      a["k"], a["lp"], a["ent"], a["fl"], a["ws"], a["ws_bytes"],
                                      None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), _native.RLK_EINVAL),
    (dict(T=0.0), _native.RLK_EINVAL),
    (dict(T=math.inf), _native.RLK_EINVAL),
    (dict(p=1.5), _native.RLK_EINVAL),
    (dict(p=-0.25), _native.RLK_EINVAL),
    (dict(p=math.nan), _native.RLK_EINVAL),
    (dict(n=-1), _native.RLK_EINVAL),
    (dict(n=1 << 31), _native.RLK_EINVAL),
    (dict(V=0), _native.RLK_EINVAL),
    (dict(stride=999), _native.RLK_EINVAL),
    (dict(nnz=-1), _native.RLK_EINVAL),
    (dict(off=None), _native.RLK_EINVAL),
    (dict(ids=None), _native.RLK_EINVAL),
    (dict(lp=None), _native.RLK_EINVAL),
    (dict(ent=None), _native.RLK_EINVAL),
    (dict(logits=P(0x100001)), _native.RLK_EINVAL),
    (dict(off=P(0x100004)), _native.RLK_EINVAL),
    (dict(p=0.9, ws=None), _native.RLK_EWORKSPACE),
    (dict(p=0.9, ws_bytes=16), _native.RLK_EWORKSPACE),
    (dict(p=0.9, k=-1), _native.RLK_EINVAL),
    (dict(k=5), _native.RLK_EINVAL),                     # a top-k check needs check_top_p
    (dict(p=0.9, k=5, ws=None), _native.RLK_EWORKSPACE),
])
def test_support_validation(L, kw, status):
    assert _support(L, **kw) == status
    assert len(L.rlk_last_error()) > 0


def test_support_empty_batch_and_workspace(L):
    assert _support(L, n=0, logits=None, targets=None, off=None, ids=None, lp=None,
                    ent=None) == _native.RLK_OK
    assert L.rlk_logprob_from_support_workspace_size(4096, 151936, 1, 0.0) == 0
    need = L.rlk_logprob_from_support_workspace_size(4096, 151936, 1, 0.95)
    assert need >= 4096 * (5 * 4 + 1) + L.rlk_logprob_from_logits_workspace_size(4096, 151936, 1)


def _sample(L, **kw):
    a = dict(logits=FAKE, dtype=1, n=4, V=1000, stride=1000, T=1.0, p=0.9, k=0, t_row=None,
             p_row=None, k_row=None, seed=1, off=0, keys=None, out=FAKE, lp=None, ent=None,
             ns=None, fl=None, ws=WS, ws_bytes=1 << 30)
    a.update(kw)
    return L.rlk_sample_top_p(a["logits"], a["dtype"], a["n"], a["V"], a["stride"], a["T"],
                              a["p"], a["k"], a["t_row"], a["p_row"], a["k_row"], a["seed"],
                              a["off"], a["keys"], a["out"], a["lp"], a["ent"], a["ns"], a["fl"],
                              a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=3), _native.RLK_EINVAL),
    (dict(T=0.0), _native.RLK_EINVAL),
    (dict(T=math.nan), _native.RLK_EINVAL),
    (dict(p=0.0), _native.RLK_EINVAL),
    (dict(p=1.01), _native.RLK_EINVAL),
    (dict(n=-2), _native.RLK_EINVAL),
    (dict(V=0), _native.RLK_EINVAL),
    (dict(V=(1 << 24) + 1, stride=(1 << 24) + 1), _native.RLK_EINVAL),
    (dict(stride=10), _native.RLK_EINVAL),
    (dict(out=None), _native.RLK_EINVAL),
    (dict(logits=None), _native.RLK_EINVAL),
    (dict(out=P(0x100004)), _native.RLK_EINVAL),
    (dict(keys=P(0x100004)), _native.RLK_EINVAL),
    (dict(ws=None), _native.RLK_EWORKSPACE),
    (dict(ws_bytes=8), _native.RLK_EWORKSPACE),
    (dict(k=-2), _native.RLK_EINVAL),
    (dict(k=40, ws=None), _native.RLK_EWORKSPACE),      # top-k is opt-in: accepted
    (dict(t_row=P(0x100002)), _native.RLK_EINVAL),
    (dict(p_row=P(0x100001)), _native.RLK_EINVAL),
    (dict(k_row=P(0x100003)), _native.RLK_EINVAL),
])
def test_sample_validation(L, kw, status):
    assert _sample(L, **kw) == status
    assert len(L.rlk_last_error()) > 0


def test_sample_empty_batch_and_workspace(L):
    assert _sample(L, n=0, logits=None, out=None) == _native.RLK_OK
    need = L.rlk_sample_top_p_workspace_size(4096, 151936, 1)
    assert need >= 4096 * (8 + 4 * 4 + 1) + L.rlk_logprob_from_logits_workspace_size(4096, 151936, 1)
