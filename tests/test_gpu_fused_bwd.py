"""GPU parity of rlk_logprob_fused_linear_bwd against the fp64 oracle, at
top-p = 1 and through the top-p cut (nucleus held fixed).

The GPU forward supplies `saved` to the GPU backward; the oracle recomputes
everything from the same bf16 inputs. Tolerance (bf16 G and bf16 dh, fp32
accumulation): normwise relative ||d||_F / ||ref||_F <= 5e-3 for dh and dW,
and <= 1e-2 for every single row of dh and every single vocabulary row of dW
(relative to the larger of the row's norm and 1e-3 of the rms row norm; the
expected per-row error is about 1e-3, the bf16 rounding of G). dh rows are
bitwise independent of how the rows are batched (fixed vocabulary chunks,
fixed summation order); dW sums over all rows and is checked for run-to-run
determinism.
"""
import numpy as np
import pytest
import torch

import synth
import grpo_loss_rlk_amd as rlk
from oracle import fused as OF
from oracle import logprob as OL
from oracle import sampling as OS

from gpu_util import DEV, assert_close_rows, bf16_to_device, bits_equal, host

pytestmark = pytest.mark.gpu

NORM_TOL, ROW_TOL = 5e-3, 1e-2


def _inputs(name, N, H=None, V=None):
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


def _upstream(N, seed):
    r = np.random.default_rng(seed)
    g_lp = (r.standard_normal(N) / N).astype(np.float32)
    g_h = (r.standard_normal(N) / N).astype(np.float32)
    return g_lp, g_h


def _gpu_bwd(h, W, yt, g_lp, g_h, T, p=1.0):
    print(f"  rlk fused fwd+bwd N={h.shape[0]} H={h.shape[1]} V={W.shape[0]} T={T} p={p}",
          flush=True)
    fwd = rlk.logprob_fused_linear(h, W, yt, T, p)
    dh, dw = rlk.logprob_fused_linear_bwd(h, W, yt, fwd["saved"], torch.as_tensor(g_lp).to(DEV),
                                          torch.as_tensor(g_h).to(DEV), T, p)
    torch.cuda.synchronize()
    return dh, dw


def _rel(got, want):
    return np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300)


def _rows_ok(got, want, what, floor_rms=None):
    """Every row of ``got`` within ROW_TOL of ``want`` relative to the larger
    of the row's norm and 1e-3 of the rms row norm (a row whose exact value
    vanishes -- a one-token nucleus: q = 1 and d = E_q d -- keeps fp32
    rounding of q around 1). ``floor_rms``: the rms row norm to use when
    ``want`` holds only a sample of the rows."""
    ref_rows = np.linalg.norm(want, axis=1)
    rms = np.sqrt(np.mean(ref_rows ** 2)) if floor_rms is None else floor_rms
    floor = 1e-3 * rms + 1e-300
    rows = np.linalg.norm(got - want, axis=1) / np.maximum(ref_rows, floor)
    assert np.all(rows <= ROW_TOL), (what, np.flatnonzero(rows > ROW_TOL)[:8], rows.max())


def _check(dh, dw, hb, wb, y, g_lp, g_h, T, p=1.0):
    dh_ref, dw_ref = OF.backward(OL.widen_bf16(hb), OL.widen_bf16(wb), y, g_lp.astype(np.float64),
                                 g_h.astype(np.float64), OL.f32(T), OL.f32(p))
    dh_got = host(dh.float()).astype(np.float64)
    dw_got = host(dw).astype(np.float64)
    assert _rel(dh_got, dh_ref) <= NORM_TOL, ("dh", _rel(dh_got, dh_ref))
    assert _rel(dw_got, dw_ref) <= NORM_TOL, ("dW", _rel(dw_got, dw_ref))
    _rows_ok(dh_got, dh_ref, "dh rows")
    # every vocabulary row of dW: the last partial vocabulary tile, the
    # 32768-row chunk seams of a large V and rows no target names included
    _rows_ok(dw_got, dw_ref, "dW rows")


@pytest.mark.parametrize("N,H,V,T", [(300, 256, 1000, 1.0), (77, 128, 515, 0.7),
                                     (513, 512, 2049, 1.8), (5, 64, 7, 1.0),
                                     (96, 64, 70001, 1.0)])
def test_bwd_ragged_shapes(N, H, V, T):
    """Ragged tiles in every dimension; V = 70001 spans three vocabulary chunks."""
    w, hb, wb, y = _inputs("fused", N, H, V)
    y = y.copy()
    if N > 4:
        y[3] = -1          # no valid target: only the entropy term
    g_lp, g_h = _upstream(N, N + V)
    dh, dw = _gpu_bwd(bf16_to_device(hb), bf16_to_device(wb), torch.as_tensor(y), g_lp, g_h, T)
    _check(dh, dw, hb, wb, y, g_lp, g_h, T)


def test_bwd_llama_loss_form_small():
    """Llama-3-70B loss form on a small shape: g_lp = -1/N, g_H = -0.001/N."""
    w, hb, wb, y = _inputs("llama70b", 257, 128, 3001)
    N = w.N
    g_lp = np.full(N, -1.0 / N, dtype=np.float32)
    g_h = np.full(N, -0.001 / N, dtype=np.float32)
    dh, dw = _gpu_bwd(bf16_to_device(hb), bf16_to_device(wb), torch.as_tensor(y), g_lp, g_h, 1.0)
    _check(dh, dw, hb, wb, y, g_lp, g_h, 1.0)


def test_bwd_determinism_and_dh_batch_invariance():
    w, hb, wb, y = _inputs("fused", 300, 128, 40000)
    h, W, yt = bf16_to_device(hb), bf16_to_device(wb), torch.as_tensor(y)
    g_lp, g_h = _upstream(w.N, 7)
    dh, dw = _gpu_bwd(h, W, yt, g_lp, g_h, 0.9)
    dh2, dw2 = _gpu_bwd(h, W, yt, g_lp, g_h, 0.9)
    assert bits_equal(dh, dh2) and bits_equal(dw, dw2)
    for split in (1, 150, 299):
        a, b = slice(0, split), slice(split, w.N)
        dha, _ = _gpu_bwd(h[a].contiguous(), W, yt[a], g_lp[a], g_h[a], 0.9)
        dhb, _ = _gpu_bwd(h[b].contiguous(), W, yt[b], g_lp[b], g_h[b], 0.9)
        assert bits_equal(dh, torch.cat([dha, dhb])), split


def _top_p_inputs(N, H, V, T, p, sigma):
    """Peaked rows (logit sd about sqrt(H) sigma), Gumbel-max targets inside the
    nucleus, one target outside it and one out of range; the upstream
    gradients of rows the oracle flags as within 1e-6 of the top-p boundary
    are zeroed on both sides (either nucleus is valid there)."""
    w = synth.workload("grpo", N=N, H=H, V=V, sigma=sigma, temperature=T, top_p=p)
    hb = synth.hidden_rows(w, range(N))
    wb = synth.weight_rows(w, range(V))
    z64 = OF.logits(OL.widen_bf16(hb), OL.widen_bf16(wb))
    Tf, pf = OL.f32(T), OL.f32(p)
    y = np.array([OS.gumbel_max_target(z64[i], Tf, pf, synth.gumbel_uniforms(w, i, V))
                  for i in range(N)], dtype=np.int64)
    y[1] = int(np.argmin(z64[1]))      # almost surely outside the nucleus
    y[2] = -1                          # out of range: entropy term only
    o = OL.logprob_from_logits(z64, y, Tf, pf)
    assert o.flags[1] & OL.FLAG_OUTSIDE
    g_lp, g_h = _upstream(N, N + V + 1)
    bnd = (o.flags & OL.FLAG_BOUNDARY) != 0
    g_lp[bnd] = 0.0
    g_h[bnd] = 0.0
    return hb, wb, y, g_lp, g_h, bnd.mean()


@pytest.mark.parametrize("N,H,V,T,p,sigma", [(300, 256, 1000, 0.7, 0.95, 0.15),
                                             (77, 128, 515, 1.3, 0.5, 0.2),
                                             (257, 64, 5003, 0.7, 0.9, 0.3),
                                             (96, 64, 70001, 0.7, 0.9, 0.3)])
def test_bwd_top_p_shapes(N, H, V, T, p, sigma):
    """Backward through the top-p cut (the nucleus of the GPU forward, held
    fixed), ragged tiles; V = 70001 spans three vocabulary chunks."""
    hb, wb, y, g_lp, g_h, frac_bnd = _top_p_inputs(N, H, V, T, p, sigma)
    assert frac_bnd < 0.05, frac_bnd       # the comparison covers most rows
    dh, dw = _gpu_bwd(bf16_to_device(hb), bf16_to_device(wb), torch.as_tensor(y), g_lp, g_h,
                      T, p)
    _check(dh, dw, hb, wb, y, g_lp, g_h, T, p)


def test_bwd_top_p_determinism_and_dh_batch_invariance():
    hb, wb, y, g_lp, g_h, _ = _top_p_inputs(300, 128, 40000, 0.7, 0.95, 0.2)
    h, W, yt = bf16_to_device(hb), bf16_to_device(wb), torch.as_tensor(y)
    dh, dw = _gpu_bwd(h, W, yt, g_lp, g_h, 0.7, 0.95)
    dh2, dw2 = _gpu_bwd(h, W, yt, g_lp, g_h, 0.7, 0.95)
    assert bits_equal(dh, dh2) and bits_equal(dw, dw2)
    for split in (1, 150):
        a, b = slice(0, split), slice(split, len(y))
        dha, _ = _gpu_bwd(h[a].contiguous(), W, yt[a], g_lp[a], g_h[a], 0.7, 0.95)
        dhb, _ = _gpu_bwd(h[b].contiguous(), W, yt[b], g_lp[b], g_h[b], 0.7, 0.95)
        assert bits_equal(dh, torch.cat([dha, dhb])), split


def _oracle_dh_row(h_row64, W64, y, g_lp, g_h, T, p=1.0):
    """fp64 dh row of one token: the oracle's G row from the full fp64 logit row."""
    z = (W64 @ h_row64)[None, :]
    G = OF.grad_logits(z, np.array([y]), np.array([g_lp]), np.array([g_h]), T, p)[0]
    return G @ W64


def _seam_rows(V, chunk=32768, tile=256):
    """Vocabulary rows at every chunk seam, the first and last rows and the
    first row of the last (possibly partial) tile."""
    rows = {0, 1, V - 1, V - 2, (V - 1) // tile * tile}
    for c in range(chunk, V, chunk):
        rows |= {c - 1, c}
    return np.array(sorted(r for r in rows if 0 <= r < V))


def test_bwd_llama_width_sampled():
    """Llama-3-70B head width (H = 8192, V = 128256: four vocabulary chunks)
    on 1024 tokens, the loss form -mean lp - 0.001 mean H: the forward's lp
    and H of every token, and sampled rows of dh and of dW (every chunk seam,
    the ends, every target row sampled and random rows) against the oracle
    computed from the full fp64 logits."""
    w = synth.workload("llama70b", N=1024)
    hb = synth.hidden_rows(w, range(w.N))
    wb = synth.weight_rows(w, range(w.V))
    y = synth.uniform_targets(w, w.N)
    N, V = w.N, w.V
    g_lp = np.full(N, -1.0 / N, dtype=np.float32)
    g_h = np.full(N, -0.001 / N, dtype=np.float32)
    h, W, yt = bf16_to_device(hb), bf16_to_device(wb), torch.as_tensor(y)
    print(f"  rlk fused fwd+bwd N={N} H={w.H} V={V}", flush=True)
    fwd = rlk.logprob_fused_linear(h, W, yt, 1.0, 1.0)
    dh, dw = rlk.logprob_fused_linear_bwd(h, W, yt, fwd["saved"], torch.as_tensor(g_lp).to(DEV),
                                          torch.as_tensor(g_h).to(DEV), 1.0, 1.0)
    torch.cuda.synchronize()
    h64, W64 = OL.widen_bf16(hb), OL.widen_bf16(wb)
    z = OF.logits(h64, W64)
    o = OL.logprob_from_logits(z, y, 1.0, 1.0)
    assert_close_rows(host(fwd["logprob"]), o.lp_trunc, 2e-3, what="logprob")
    assert_close_rows(host(fwd["entropy"]), o.h_trunc, 1e-5, 1e-3, what="entropy")
    G = OF.grad_logits(z, y, g_lp.astype(np.float64), g_h.astype(np.float64), 1.0, 1.0)
    del z
    rng = np.random.default_rng(2)
    vs = np.unique(np.concatenate([_seam_rows(V), y[:16], rng.choice(V, 48, replace=False)]))
    ns = np.unique(np.concatenate([[0, 1, N - 1], rng.choice(N, 13, replace=False)]))
    # the floor of the per-row checks: the rms row norm of all of dW, from
    # ||G^T h||_F^2 = sum(G * (h h^T) G) without forming the [V, H] product
    dw_rms = np.sqrt(np.sum(G * ((h64 @ h64.T) @ G)) / V)
    _rows_ok(host(dw[vs]).astype(np.float64), G[:, vs].T @ h64, "dW rows", dw_rms)
    dh_ref = G[ns] @ W64
    _rows_ok(host(dh[ns].float()).astype(np.float64), dh_ref, "dh rows")


def test_bwd_llama70b_full_size_sampled():
    """Full Llama-3-70B head (16384 x 8192 . 128256 x 8192): the forward's lp
    and H on 8 rows, two dh rows against the oracle computed row by row, and
    the zero-sum property of dW rows (rows of G sum to zero, so
    sum_v dW[v, :] = 0 up to rounding). Sampled dW rows need every token's
    logits and are checked at this width on 1024 tokens (above)."""
    w = synth.workload("llama70b")
    hb = synth.hidden_rows(w, range(w.N))
    wb = synth.weight_rows(w, range(w.V))
    y = synth.uniform_targets(w, w.N)
    N = w.N
    g_lp = np.full(N, -1.0 / N, dtype=np.float32)
    g_h = np.full(N, -0.001 / N, dtype=np.float32)
    h, W, yt = bf16_to_device(hb), bf16_to_device(wb), torch.as_tensor(y)
    print(f"  rlk fused fwd+bwd N={N} H={w.H} V={w.V}", flush=True)
    fwd = rlk.logprob_fused_linear(h, W, yt, 1.0, 1.0)
    dh, dw = rlk.logprob_fused_linear_bwd(h, W, yt, fwd["saved"], torch.as_tensor(g_lp).to(DEV),
                                          torch.as_tensor(g_h).to(DEV), 1.0, 1.0)
    torch.cuda.synchronize()
    colsum = host(torch.sum(dw, dim=0, dtype=torch.float64))
    assert np.abs(colsum).max() <= 3e-4, np.abs(colsum).max()
    W64 = OL.widen_bf16(wb)
    rows = np.array([0, 1, 4097, 8191, 8192, 12345, N - 2, N - 1])
    o = OL.logprob_from_logits(OL.widen_bf16(hb[rows]) @ W64.T, y[rows], 1.0, 1.0)
    assert_close_rows(host(fwd["logprob"])[rows], o.lp_trunc, 2e-3, what="logprob")
    assert_close_rows(host(fwd["entropy"])[rows], o.h_trunc, 1e-5, 1e-3, what="entropy")
    for n in (0, N - 1):
        want = _oracle_dh_row(OL.widen_bf16(hb[n]), W64, int(y[n]), -1.0 / N, -0.001 / N, 1.0)
        got = host(dh[n].float()).astype(np.float64)
        assert _rel(got, want) <= ROW_TOL, (n, _rel(got, want))


def test_bwd_grpo_full_size_sampled():
    """Config-4 LM-head backward at full size (T_tot ~ 110k packed tokens,
    H=4096, V=151936, T=0.7, p=0.95) through the GPU forward's nucleus, with
    upstream g_lp ~ N(0,1)/T_tot and no entropy term (the GRPO loss has none):
    three dh rows (Gumbel-max targets from the nucleus) against the oracle row
    by row, and the zero-sum property of dW columns (each row of G sums to
    zero over the nucleus)."""
    w = synth.workload("grpo")
    cu = synth.cu_seqlens(synth.response_lengths(w))
    T_tot = int(cu[-1])
    wb = synth.weight_rows(w, range(w.V))
    hb = synth.hidden_rows(w, range(T_tot))
    rows = np.array([0, T_tot // 2, T_tot - 1])
    W64 = OL.widen_bf16(wb)
    z64 = OL.widen_bf16(hb[rows]) @ W64.T
    Tf, pf = OL.f32(w.temperature), OL.f32(w.top_p)
    y = synth.uniform_targets(w, T_tot)
    y[rows] = [OS.gumbel_max_target(z64[i], Tf, pf, synth.gumbel_uniforms(w, int(r), w.V))
               for i, r in enumerate(rows)]
    g_lp = (np.random.default_rng(11).standard_normal(T_tot) / T_tot).astype(np.float32)
    h, W, yt = bf16_to_device(hb), bf16_to_device(wb), torch.as_tensor(y)
    print(f"  rlk fused fwd+bwd T_tot={T_tot} p={w.top_p}", flush=True)
    fwd = rlk.logprob_fused_linear(h, W, yt, w.temperature, w.top_p)
    dh, dw = rlk.logprob_fused_linear_bwd(h, W, yt, fwd["saved"], torch.as_tensor(g_lp).to(DEV),
                                          None, w.temperature, w.top_p)
    torch.cuda.synchronize()
    colsum = host(torch.sum(dw, dim=0, dtype=torch.float64))
    assert np.abs(colsum).max() <= 3e-4, np.abs(colsum).max()
    for i, n in enumerate(rows):
        want = _oracle_dh_row(OL.widen_bf16(hb[n]), W64, int(y[n]), float(g_lp[n]), 0.0, Tf, pf)
        got = host(dh[n].float()).astype(np.float64)
        assert _rel(got, want) <= ROW_TOL, (n, _rel(got, want))


def test_bwd_grad_hidden_only_2_byte_aligned():
    """grad_hidden needs only 2-byte alignment: the dh epilogue writes four
    bf16 values as one 8-byte store when the output is 8-byte aligned and as
    four 2-byte stores otherwise. Through the C ABI with grad_hidden at an
    offset of 2 bytes (one and several vocabulary chunks, so the first,
    middle and last dh modes all store), dh must equal the aligned call's
    bitwise, and dW too."""
    from grpo_loss_rlk_amd import _native
    L = _native.lib()
    for N, H, V in [(300, 128, 5000), (197, 64, 70001)]:
        w, hb, wb, y = _inputs("fused", N, H, V)
        h, W = bf16_to_device(hb), bf16_to_device(wb)
        yt = torch.as_tensor(y).to(DEV)
        g_lp, g_h = _upstream(N, 11)
        glp, gh = torch.as_tensor(g_lp).to(DEV), torch.as_tensor(g_h).to(DEV)
        fwd = rlk.logprob_fused_linear(h, W, yt, 0.7, 0.95)
        dh_ref, dw_ref = rlk.logprob_fused_linear_bwd(h, W, yt, fwd["saved"], glp, gh, 0.7, 0.95)
        buf = torch.full((N * H + 4,), float("nan"), device=DEV, dtype=torch.bfloat16)
        dw = torch.empty(V, H, device=DEV, dtype=torch.float32)
        ws_n = L.rlk_logprob_fused_linear_bwd_workspace_size(N, H, V, 0.95)
        ws = torch.empty(ws_n, device=DEV, dtype=torch.uint8)
        print(f"  rlk bwd with grad_hidden at +2 bytes N={N} H={H} V={V}", flush=True)
        st = L.rlk_logprob_fused_linear_bwd(
            h.data_ptr(), W.data_ptr(), N, H, V, h.stride(0), W.stride(0), yt.data_ptr(),
            fwd["saved"].data_ptr(), glp.data_ptr(), gh.data_ptr(), 0.7, 0.95, 0,
            buf.data_ptr() + 2, dw.data_ptr(), ws.data_ptr(), ws_n,
            torch.cuda.current_stream().cuda_stream)
        assert st == _native.RLK_OK, L.rlk_last_error()
        torch.cuda.synchronize()
        dh = buf[1:1 + N * H].view(N, H)
        assert bits_equal(dh, dh_ref)
        assert bits_equal(dw, dw_ref)
        # nothing written outside [ptr, ptr + 2 N H)
        assert torch.isnan(buf[0].float()) and torch.isnan(buf[1 + N * H:].float()).all()


@pytest.mark.parametrize("p", [1.0, 0.9])
def test_maximum_rows(p):
    """N = 2^23 - 1 tokens, the most the fused path accepts: 513 logits
    blocks at top-p, and in the backward rows of h^T and G^T 2^23 + 64
    elements long, at the edge of the tile GEMM's 32-bit copy offsets. The
    upstream gradients are zero except on 64 sampled rows (block seams and
    the last row among them), so the oracle's dW is the sum over those rows
    alone; the forward and dh are compared there, and dh of every other row
    must be exactly 0."""
    N, H, V, T = (1 << 23) - 1, 64, 7, 0.7
    r = np.random.default_rng(123)
    hb = synth.bf16_bits_from_f32(r.standard_normal((N, H), dtype=np.float32)).reshape(N, H)
    wb = synth.bf16_bits_from_f32(r.standard_normal((V, H), dtype=np.float32)
                                  * np.float32(0.2)).reshape(V, H)
    y = r.integers(0, V, N)
    rows = np.unique(np.concatenate([[0, 16383, 16384, N - 16384, N - 1],
                                     r.choice(N, 59, replace=False)]))
    g_lp = np.zeros(N, np.float32)
    g_h = np.zeros(N, np.float32)
    g_lp[rows] = (r.standard_normal(len(rows)) / len(rows)).astype(np.float32)
    g_h[rows] = (r.standard_normal(len(rows)) / len(rows)).astype(np.float32)
    h, W, yt = bf16_to_device(hb), bf16_to_device(wb), torch.as_tensor(y).to(DEV)
    print(f"  rlk fused fwd+bwd N={N} H={H} V={V} T={T} p={p}", flush=True)
    fwd = rlk.logprob_fused_linear(h, W, yt, T, p)
    dh, dw = rlk.logprob_fused_linear_bwd(h, W, yt, fwd["saved"], torch.as_tensor(g_lp).to(DEV),
                                          torch.as_tensor(g_h).to(DEV), T, p)
    torch.cuda.synchronize()
    h64, w64 = OL.widen_bf16(hb[rows]), OL.widen_bf16(wb)
    o = OF.forward(h64, w64, y[rows], OL.f32(T), OL.f32(p))
    ok = (o.flags & OL.FLAG_BOUNDARY) == 0
    lp = host(fwd["logprob"])[rows]
    assert_close_rows(lp[ok], o.lp_trunc[ok], 2e-3, what="logprob")
    assert_close_rows(host(fwd["entropy"])[rows][ok], o.h_trunc[ok], 1e-5, 1e-3, what="entropy")
    lp_all = fwd["logprob"]
    assert bool(torch.all((lp_all <= 0) | torch.isneginf(lp_all)))
    dh_ref, dw_ref = OF.backward(h64, w64, y[rows], g_lp[rows].astype(np.float64),
                                 g_h[rows].astype(np.float64), OL.f32(T), OL.f32(p))
    idx = torch.as_tensor(rows).to(DEV)
    dh_rows = host(dh.index_select(0, idx).float()).astype(np.float64)
    assert _rel(dh_rows, dh_ref) <= NORM_TOL, ("dh", _rel(dh_rows, dh_ref))
    _rows_ok(dh_rows, dh_ref, "dh rows")
    others = torch.ones(N, dtype=torch.bool, device=DEV)
    others[idx] = False
    assert int(torch.count_nonzero(dh[others])) == 0
    dw_got = host(dw).astype(np.float64)
    assert _rel(dw_got, dw_ref) <= NORM_TOL, ("dW", _rel(dw_got, dw_ref))
    _rows_ok(dw_got, dw_ref, "dW rows")
