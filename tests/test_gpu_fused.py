"""GPU parity of rlk_logprob_fused_linear against the fp64 oracle (logits
h . W^T formed in fp64 from the same bf16 operands), plus bitwise determinism
and batch invariance. Tolerance (bf16 inputs, fp32 accumulate): |d lp| <= 2e-3,
|d H| <= 1e-3 |H| with a 1e-5 floor."""
import numpy as np
import pytest
import torch

import synth
import grpo_loss_rlk_amd as rlk
from oracle import fused as OF
from oracle import logprob as OL

from gpu_util import DEV, assert_close_rows, bf16_to_device, bits_equal, host

pytestmark = pytest.mark.gpu

LP_TOL, H_RTOL, H_ATOL = 2e-3, 1e-3, 1e-5


def _inputs(name, N, H=None, V=None, seed_rows=None):
    kw = {"N": N}
    if H is not None:
        kw["H"] = H
    if V is not None:
        kw["V"] = V
    w = synth.workload(name, **kw)
    hb = synth.hidden_rows(w, range(w.N))
    wb = synth.weight_rows(w, range(w.V))
    y = synth.uniform_targets(w, w.N)
    return w, hb, wb, y


def _run(hb, wb, y, T, p=1.0):
    h = bf16_to_device(hb)
    W = bf16_to_device(wb)
    print(f"  rlk_logprob_fused_linear N={h.shape[0]} H={h.shape[1]} V={W.shape[0]} T={T}", flush=True)
    out = rlk.logprob_fused_linear(h, W, torch.as_tensor(y), T, p)
    torch.cuda.synchronize()
    return out


def _check(out, hb, wb, y, T, rows=None):
    rows = np.arange(hb.shape[0]) if rows is None else np.asarray(rows)
    h64 = OL.widen_bf16(hb[rows])
    w64 = OL.widen_bf16(wb)
    o = OF.forward(h64, w64, y[rows], OL.f32(T), 1.0)
    assert_close_rows(host(out["logprob"])[rows], o.lp_trunc, LP_TOL, what="logprob")
    assert_close_rows(host(out["entropy"])[rows], o.h_trunc, H_ATOL, H_RTOL, what="entropy")
    assert np.all(host(out["nucleus_size"])[rows] == hb.shape[0] * 0 + wb.shape[0])
    sv = host(out["saved"])[rows]
    # saved: log Z of z/T and E_q[z/T]
    z = OF.logits(h64, w64) / OL.f32(T)
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    logZ = (m[:, 0] + np.log(e.sum(axis=1)))
    Eq = (e * z).sum(axis=1) / e.sum(axis=1)
    np.testing.assert_allclose(sv[:, 0], logZ, rtol=1e-5, atol=1e-4)
    np.testing.assert_allclose(sv[:, 1], Eq, rtol=1e-5, atol=1e-4)
    return o


@pytest.mark.parametrize("N,H,V,T", [(300, 256, 1000, 1.0), (77, 128, 515, 0.7),
                                     (513, 512, 2049, 1.8), (5, 64, 7, 1.0),
                                     (5, 64, 1, 1.0), (9, 64, 2, 0.7)])
def test_ragged_small_shapes(N, H, V, T):
    w, hb, wb, y = _inputs("fused", N, H, V)
    out = _run(hb, wb, y, T)
    _check(out, hb, wb, y, T)


def test_qwen_head_sampled_rows():
    """Qwen3-8B head shape (H=4096, V=151936) on 700 tokens; 16 rows checked."""
    w, hb, wb, y = _inputs("fused", 700)
    out = _run(hb, wb, y, 1.0)
    rows = np.random.default_rng(0).choice(w.N, 16, replace=False)
    o = _check(out, hb, wb, y, 1.0, rows)
    # sanity magnitude: H ~ log V - sigma^2/2 with sigma = 0.02 * sqrt(4096) = 1.28
    assert 10.5 < float(np.mean(o.h_trunc)) < 11.5


def test_bad_target_and_bitwise_batch_invariance():
    w, hb, wb, y = _inputs("fused", 300, 256, 1000)
    y = y.copy()
    y[3] = -1
    y[4] = w.V
    h = bf16_to_device(hb)
    W = bf16_to_device(wb)
    yt = torch.as_tensor(y)
    ref = rlk.logprob_fused_linear(h, W, yt, 0.7)
    f = host(ref["flags"])
    assert f[3] & rlk.FLAG_BAD_TARGET and f[4] & rlk.FLAG_BAD_TARGET
    assert np.isnan(host(ref["logprob"])[3])
    again = rlk.logprob_fused_linear(h, W, yt, 0.7)
    for k in ("logprob", "entropy", "saved"):
        assert bits_equal(ref[k], again[k]), k
    for split in (1, 37, 256):
        parts = [rlk.logprob_fused_linear(h[i:i + split].contiguous(), W, yt[i:i + split], 0.7)
                 for i in range(0, w.N, split)]
        for k in ("logprob", "entropy", "saved"):
            assert bits_equal(ref[k], torch.cat([p_[k] for p_ in parts])), (k, split)
    perm = torch.from_numpy(np.random.default_rng(1).permutation(w.N))
    pr = rlk.logprob_fused_linear(h[perm.to(DEV)].contiguous(), W, yt[perm], 0.7)
    for k in ("logprob", "entropy", "saved"):
        assert bits_equal(ref[k][perm.to(DEV)], pr[k]), k


def test_qwen_head_full_size_sampled_rows():
    """The full Qwen3-8B head launch the benchmark times (hidden [8192, 4096],
    W [151936, 4096], T=1, p=1); 8 rows checked against the oracle one by one
    (each row's logits formed in fp64)."""
    w = synth.workload("fused")
    hb = synth.hidden_rows(w, range(w.N))
    wb = synth.weight_rows(w, range(w.V))
    y = synth.uniform_targets(w, w.N)
    out = _run(hb, wb, y, w.temperature)
    rows = np.random.default_rng(3).choice(w.N, 8, replace=False)
    W64 = OL.widen_bf16(wb)
    z = OL.widen_bf16(hb[rows]) @ W64.T
    o = OL.logprob_from_logits(z, y[rows], OL.f32(w.temperature), 1.0)
    assert_close_rows(host(out["logprob"])[rows], o.lp_trunc, LP_TOL, what="logprob")
    assert_close_rows(host(out["entropy"])[rows], o.h_trunc, H_ATOL, H_RTOL, what="entropy")
    assert np.all(np.isfinite(host(out["logprob"])))



@pytest.mark.parametrize("p", [1.0, 0.9])
def test_nonfinite_hidden_rows_are_flagged(p):
    """A NaN or an infinity in a hidden row makes that token's logits
    non-finite: its outputs are NaN with the non-finite flag, at top-p 1 and
    below; every other row is bitwise the clean run's. Also a whole W tile of
    NaN (256 vocabulary rows) flags every row."""
    w, hb, wb, y = _inputs("fused", 300, 256, 1000)
    h = bf16_to_device(hb)
    W = bf16_to_device(wb)
    yt = torch.as_tensor(y)
    clean = rlk.logprob_fused_linear(h, W, yt, 0.7, p)
    hbad = hb.copy()
    hbad[5, 17] = 0x7fc0          # NaN
    hbad[9, 3] = 0x7f80           # +inf
    hbad[11, 200] = 0xff80        # -inf
    out = rlk.logprob_fused_linear(bf16_to_device(hbad), W, yt, 0.7, p)
    torch.cuda.synchronize()
    fl = host(out["flags"])
    bad = np.zeros(w.N, bool)
    bad[[5, 9, 11]] = True
    assert np.all(fl[bad] & rlk.FLAG_NONFINITE), fl[bad]
    assert np.all(np.isnan(host(out["logprob"])[bad]))
    assert np.all(np.isnan(host(out["entropy"])[bad]))
    assert not np.any(fl[~bad] & rlk.FLAG_NONFINITE)
    good = torch.from_numpy(np.flatnonzero(~bad)).to(DEV)
    for k in ("logprob", "entropy"):
        assert bits_equal(clean[k][good], out[k][good]), k
    wbad = wb.copy()
    wbad[256:512, :] = 0x7fc0     # the second vocabulary tile entirely NaN
    out = rlk.logprob_fused_linear(h, bf16_to_device(wbad), yt, 0.7, p)
    torch.cuda.synchronize()
    assert np.all(host(out["flags"]) & rlk.FLAG_NONFINITE)
    assert np.all(np.isnan(host(out["logprob"])))


def test_zero_rows():
    """N = 0: empty outputs from the forward; the backward writes dW = 0."""
    H, V = 64, 3001
    w = synth.workload("fused", N=1, H=H, V=V)
    W = bf16_to_device(synth.weight_rows(w, range(V)))
    h = torch.empty(0, H, device=DEV, dtype=torch.bfloat16)
    y = torch.empty(0, device=DEV, dtype=torch.int64)
    for p in (1.0, 0.9):
        print(f"  rlk_logprob_fused_linear N=0 H={H} V={V} p={p}", flush=True)
        out = rlk.logprob_fused_linear(h, W, y, 0.7, p)
        torch.cuda.synchronize()
        assert out["logprob"].numel() == 0 and out["entropy"].numel() == 0
        g = torch.empty(0, device=DEV, dtype=torch.float32)
        print(f"  rlk_logprob_fused_linear_bwd N=0 H={H} V={V} p={p}", flush=True)
        dh, dw = rlk.logprob_fused_linear_bwd(h, W, y, out["saved"], g, g, 0.7, p)
        torch.cuda.synchronize()
        assert dh.numel() == 0 and dw.shape == (V, H)
        assert torch.count_nonzero(dw).item() == 0

