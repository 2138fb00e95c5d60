"""The no-allocation entry point (rlk_logprob_from_logits_noalloc) through the
C ABI against rlk_logprob_from_logits on the same inputs: every output
bitwise equal, on two calls in a row, the second with fewer rows. Its
scratch (the bf16 row kernel's per-row hand-off flags, and with top-k each
row's floor) is a static array that keeps the last call's contents, so the
rows handed on to the generic algorithm, and the top-k of each row, differ
between the two calls: a stale flag or floor would show."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from grpo_loss_rlk_amd import _native

from gpu_util import DEV, bf16_to_device, bits_equal, f32_to_device

pytestmark = pytest.mark.gpu


def _outs(n):
    f = dict(device=DEV, dtype=torch.float32)
    return {"lp_full": torch.full((n,), 7.0, **f), "lp_trunc": torch.full((n,), 7.0, **f),
            "entropy_trunc": torch.full((n,), 7.0, **f), "entropy_full": torch.full((n,), 7.0, **f),
            "nucleus_size": torch.full((n,), -7, device=DEV, dtype=torch.int32),
            "threshold": torch.full((n,), 7.0, **f),
            "flags": torch.full((n,), 0xEE, device=DEV, dtype=torch.uint8)}


def _call(L, x, dtype, y, T, p, noalloc, top_k=0, k_row=None):
    n, V = x.shape
    o = _outs(n)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    args = [ptr(x), dtype, n, V, x.stride(0), ptr(y), T, p, None, None, top_k,
            None if k_row is None else ptr(k_row),
            ptr(o["lp_full"]), ptr(o["lp_trunc"]), ptr(o["entropy_trunc"]), ptr(o["entropy_full"]),
            ptr(o["nucleus_size"]), ptr(o["threshold"]), ptr(o["flags"])]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if noalloc:
        st = L.rlk_logprob_from_logits_noalloc(*args, stream)
    else:
        ws_n = L.rlk_logprob_from_logits_workspace_size(n, V, dtype)
        ws = torch.empty(max(ws_n, 1), device=DEV, dtype=torch.uint8)
        st = L.rlk_logprob_from_logits(*args, ptr(ws), ws_n, stream)
    assert st == _native.RLK_OK, L.rlk_last_error()
    torch.cuda.synchronize()
    return o


def _bf16_rows(n, V, handoff_rows, seed):
    w = synth.workload("qwen", V=V)
    arr = synth.logits_rows(w, range(seed, seed + n)).copy()
    for r in handoff_rows:
        arr[r, 5] = 0x0001          # |z| far below the counted window: handed on
    arr[handoff_rows[0], 9] = 0x7F80      # +inf: handed on, NaN outputs
    y = synth.peak_targets(w, range(seed, seed + n))
    return bf16_to_device(arr), torch.as_tensor(y).to(DEV)


@pytest.mark.parametrize("T,p", [(0.7, 0.95), (1.0, 1.0)])
def test_noalloc_matches_the_workspace_entry_point(T, p):
    L = _native.lib()
    # bf16, V >= 16384: the histogram kernel, whose hand-off flags live in the
    # static scratch; the first call hands on rows 3, 40, 200, the second
    # (fewer rows) rows 1 and 60 only
    for n, handoff, seed in ((300, [3, 40, 200], 0), (100, [1, 60], 500)):
        x, y = _bf16_rows(n, 151936, handoff, seed)
        print(f"  rlk_logprob_from_logits_noalloc bf16 N={n} V=151936 T={T} p={p}", flush=True)
        got = _call(L, x, 1, y, T, p, noalloc=True)
        want = _call(L, x, 1, y, T, p, noalloc=False)
        for k in want:
            assert bits_equal(got[k], want[k]), (n, k)
        fl = got["flags"].cpu().numpy()
        assert fl[handoff[0]] & _native.FLAG_NONFINITE
        assert not (fl[handoff[1:]] & _native.FLAG_NONFINITE).any()
    # fp32 and small-V bf16 rows (kernels without scratch), two sizes in a row
    for n, V, dtype in ((64, 8192, 0), (17, 8192, 0), (40, 4000, 1), (9, 4000, 1)):
        r = np.random.default_rng(n + V)
        z = r.normal(0, 3, (n, V)).astype(np.float32)
        x = f32_to_device(z) if dtype == 0 else bf16_to_device(synth.bf16_bits_from_f32(z))
        y = torch.as_tensor(r.integers(0, V, n)).to(DEV)
        print(f"  rlk_logprob_from_logits_noalloc dtype={dtype} N={n} V={V}", flush=True)
        got = _call(L, x, dtype, y, T, p, noalloc=True)
        want = _call(L, x, dtype, y, T, p, noalloc=False)
        for k in want:
            assert bits_equal(got[k], want[k]), (n, V, k)


def test_noalloc_top_k_matches_the_workspace_entry_point():
    """Top-k (per-row k in the first call, a scalar k in the second, smaller
    one): the floors live in the static scratch too."""
    L = _native.lib()
    for n, handoff, seed, k_scalar in ((300, [3, 40, 200], 7, 0), (100, [1, 60], 900, 40)):
        x, y = _bf16_rows(n, 151936, handoff, seed)
        k_row = None
        if k_scalar == 0:
            k_row = torch.as_tensor(np.random.default_rng(seed).integers(0, 300, n),
                                    dtype=torch.int32).to(DEV)
        print(f"  rlk_logprob_from_logits_noalloc top-k N={n} k={k_scalar or 'per row'}",
              flush=True)
        got = _call(L, x, 1, y, 0.7, 0.95, True, k_scalar, k_row)
        want = _call(L, x, 1, y, 0.7, 0.95, False, k_scalar, k_row)
        for k in want:
            assert bits_equal(got[k], want[k]), (n, k)
