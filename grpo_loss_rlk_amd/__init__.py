"""rlk on MI355X: token log-probabilities, entropy and the GRPO token loss.

Thin Python binding over the C ABI in include/rlk.h (librlk.so, hand-written
HIP kernels for gfx950). This module only marshals arguments: it allocates the
output and workspace tensors with torch on the input's device and passes raw
pointers and the current HIP stream. Every step of the computation runs in the
library's kernels; there is no CPU or PyTorch fallback.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import _native
from ._native import (DTYPE_BF16, DTYPE_F32, FLAG_BAD_PARAM, FLAG_BAD_SUPPORT,  # noqa: F401
                      FLAG_BAD_TARGET, FLAG_BOUNDARY, FLAG_MISMATCH, FLAG_NONFINITE,
                      FLAG_OUTSIDE, RlkError, lib)

__all__ = ["logprob_from_logits", "logprob_fused_linear", "logprob_fused_linear_bwd",
           "grpo_token_loss", "lib", "RlkError"]


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _workspace(nbytes: int, device) -> torch.Tensor:
    # torch's caching allocator returns blocks aligned to at least 512 bytes
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _f32_opt(x, n, device):
    if x is None:
        return None
    x = torch.as_tensor(x, dtype=torch.float32, device=device).contiguous()
    assert x.numel() == n
    return x


def _i32_opt(x, n, device):
    if x is None:
        return None
    x = torch.as_tensor(x, dtype=torch.int32, device=device).contiguous()
    assert x.numel() == n
    return x


def logprob_from_logits(logits: torch.Tensor, targets: torch.Tensor, temperature: float,
                        top_p: float = 1.0, *, vocab: int | None = None,
                        temperature_per_row=None, top_p_per_row=None, top_k: int = 0,
                        top_k_per_row=None, want_entropy_full: bool = True,
                        want_nucleus: bool = True) -> dict:
    """Full and top-k/top-p truncated logprob / entropy for each row of ``logits``.

    ``logits`` is [N, row_stride] fp32 or bf16 on the GPU (row-major, rows may
    be padded: only the first ``vocab`` entries are scored). ``top_k`` = 0 is
    no top-k. Returns a dict of tensors: lp_full, lp_trunc, entropy_trunc,
    entropy_full, nucleus_size, threshold, flags.
    """
    if logits.dtype == torch.float32:
        dtype = DTYPE_F32
    elif logits.dtype == torch.bfloat16:
        dtype = DTYPE_BF16
    else:
        raise TypeError(f"logits dtype {logits.dtype} is not float32 or bfloat16")
    if logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be a 2-D tensor with unit column stride")
    N, width = logits.shape
    V = width if vocab is None else int(vocab)
    dev = logits.device
    targets = targets.to(device=dev, dtype=torch.int64).contiguous()
    f = dict(device=dev, dtype=torch.float32)
    out = {"lp_full": torch.empty(N, **f), "lp_trunc": torch.empty(N, **f),
           "entropy_trunc": torch.empty(N, **f),
           "entropy_full": torch.empty(N, **f) if want_entropy_full else None,
           "nucleus_size": torch.empty(N, device=dev, dtype=torch.int32) if want_nucleus else None,
           "threshold": torch.empty(N, **f) if want_nucleus else None,
           "flags": torch.empty(N, device=dev, dtype=torch.uint8)}
    t_row = _f32_opt(temperature_per_row, N, dev)
    p_row = _f32_opt(top_p_per_row, N, dev)
    k_row = _i32_opt(top_k_per_row, N, dev)
    L = lib()
    ws_n = L.rlk_logprob_from_logits_workspace_size(N, V, dtype)
    ws = _workspace(ws_n, dev)
    st = L.rlk_logprob_from_logits(
        _ptr(logits), dtype, N, V, logits.stride(0) if N > 0 else V, _ptr(targets),
        float(temperature), float(top_p), _ptr(t_row), _ptr(p_row), int(top_k), _ptr(k_row),
        _ptr(out["lp_full"]), _ptr(out["lp_trunc"]), _ptr(out["entropy_trunc"]),
        _ptr(out["entropy_full"]), _ptr(out["nucleus_size"]), _ptr(out["threshold"]),
        _ptr(out["flags"]), _ptr(ws), ws_n, _stream(dev))
    _native.check(st, "rlk_logprob_from_logits")
    return out


def logprob_from_support(logits: torch.Tensor, targets: torch.Tensor, temperature: float,
                         support_offsets: torch.Tensor, support_ids: torch.Tensor, *,
                         vocab: int | None = None, check_top_p: float = 0.0,
                         check_top_k: int = 0) -> dict:
    """Logprob / entropy of each row over a caller-supplied retained set (CSR).

    ``support_offsets`` [N + 1] int64 and ``support_ids`` int32 (strictly
    increasing ids per row) on the GPU. ``check_top_p`` in (0, 1] also
    recomputes each row's nucleus (with top-k ``check_top_k``, 0 = none) and
    flags a set that differs from it. Returns logprob, entropy, flags.
    """
    if logits.dtype == torch.float32:
        dtype = DTYPE_F32
    elif logits.dtype == torch.bfloat16:
        dtype = DTYPE_BF16
    else:
        raise TypeError(f"logits dtype {logits.dtype} is not float32 or bfloat16")
    if logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be a 2-D tensor with unit column stride")
    N, width = logits.shape
    V = width if vocab is None else int(vocab)
    dev = logits.device
    targets = targets.to(device=dev, dtype=torch.int64).contiguous()
    offsets = support_offsets.to(device=dev, dtype=torch.int64).contiguous()
    ids = support_ids.to(device=dev, dtype=torch.int32).contiguous()
    if offsets.numel() != N + 1:
        raise ValueError("support_offsets must hold n_rows + 1 entries")
    f = dict(device=dev, dtype=torch.float32)
    out = {"logprob": torch.empty(N, **f), "entropy": torch.empty(N, **f),
           "flags": torch.empty(N, device=dev, dtype=torch.uint8)}
    L = lib()
    ws_n = L.rlk_logprob_from_support_workspace_size(N, V, dtype, float(check_top_p))
    ws = _workspace(ws_n, dev)
    st = L.rlk_logprob_from_support(
        _ptr(logits), dtype, N, V, logits.stride(0) if N > 0 else V, _ptr(targets),
        float(temperature), _ptr(offsets), _ptr(ids) if ids.numel() else None, ids.numel(),
        float(check_top_p), int(check_top_k), _ptr(out["logprob"]), _ptr(out["entropy"]),
        _ptr(out["flags"]),
        _ptr(ws), ws_n, _stream(dev))
    _native.check(st, "rlk_logprob_from_support")
    return out


def sample_top_p(logits: torch.Tensor, temperature: float, top_p: float, seed: int,
                 offset: int = 0, *, row_keys=None, vocab: int | None = None, top_k: int = 0,
                 temperature_per_row=None, top_p_per_row=None, top_k_per_row=None) -> dict:
    """Draw one token per row from the tempered top-k/top-p nucleus (seeded
    Gumbel-max, Philox-4x32-10 uniforms) and score it with the logits-in
    kernel. Parameters are scalars or per-row arrays (``top_k`` 0: none).
    Returns samples (int64, -1 for a row without a finite logit or with an
    out-of-range parameter), logprob, entropy, nucleus_size, flags."""
    if logits.dtype == torch.float32:
        dtype = DTYPE_F32
    elif logits.dtype == torch.bfloat16:
        dtype = DTYPE_BF16
    else:
        raise TypeError(f"logits dtype {logits.dtype} is not float32 or bfloat16")
    if logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be a 2-D tensor with unit column stride")
    N, width = logits.shape
    V = width if vocab is None else int(vocab)
    dev = logits.device
    keys = None
    if row_keys is not None:
        keys = torch.as_tensor(row_keys).to(device=dev, dtype=torch.int64).contiguous()
        if keys.numel() != N:
            raise ValueError("row_keys must hold one key per row")
    f = dict(device=dev, dtype=torch.float32)
    out = {"samples": torch.empty(N, device=dev, dtype=torch.int64),
           "logprob": torch.empty(N, **f), "entropy": torch.empty(N, **f),
           "nucleus_size": torch.empty(N, device=dev, dtype=torch.int32),
           "flags": torch.empty(N, device=dev, dtype=torch.uint8)}
    t_row = _f32_opt(temperature_per_row, N, dev)
    p_row = _f32_opt(top_p_per_row, N, dev)
    k_row = _i32_opt(top_k_per_row, N, dev)
    L = lib()
    ws_n = L.rlk_sample_top_p_workspace_size(N, V, dtype)
    ws = _workspace(ws_n, dev)
    st = L.rlk_sample_top_p(
        _ptr(logits), dtype, N, V, logits.stride(0) if N > 0 else V, float(temperature),
        float(top_p), int(top_k), _ptr(t_row), _ptr(p_row), _ptr(k_row),
        int(seed) & 0xFFFFFFFFFFFFFFFF, int(offset) & 0xFFFFFFFF, _ptr(keys),
        _ptr(out["samples"]), _ptr(out["logprob"]), _ptr(out["entropy"]),
        _ptr(out["nucleus_size"]), _ptr(out["flags"]), _ptr(ws), ws_n, _stream(dev))
    _native.check(st, "rlk_sample_top_p")
    return out


def logprob_fused_linear(hidden: torch.Tensor, weight: torch.Tensor, targets: torch.Tensor,
                         temperature: float = 1.0, top_p: float = 1.0, *, top_k: int = 0,
                         want_saved: bool = True) -> dict:
    """Fused LM head: logprob / entropy of targets under softmax(hidden W^T / T).

    ``hidden`` [N, H] and ``weight`` [V, H] are bf16 on the GPU. Returns
    logprob, entropy, saved ([N, 4], for the backward), nucleus_size, flags.
    """
    if hidden.dtype != torch.bfloat16 or weight.dtype != torch.bfloat16:
        raise TypeError("hidden and weight must be bfloat16")
    N, H = hidden.shape
    V, H2 = weight.shape
    if H2 != H:
        raise ValueError("hidden and weight disagree on the hidden size")
    if hidden.stride(1) != 1 or weight.stride(1) != 1:
        raise ValueError("hidden and weight need unit column stride")
    dev = hidden.device
    targets = targets.to(device=dev, dtype=torch.int64).contiguous()
    f = dict(device=dev, dtype=torch.float32)
    out = {"logprob": torch.empty(N, **f), "entropy": torch.empty(N, **f),
           "saved": torch.empty(N, 4, **f) if want_saved else None,
           "nucleus_size": torch.empty(N, device=dev, dtype=torch.int32),
           "flags": torch.empty(N, device=dev, dtype=torch.uint8)}
    L = lib()
    ws_n = L.rlk_logprob_fused_linear_workspace_size(N, H, V, float(top_p), int(top_k))
    ws = _workspace(ws_n, dev)
    st = L.rlk_logprob_fused_linear(
        _ptr(hidden), _ptr(weight), N, H, V, hidden.stride(0), weight.stride(0), _ptr(targets),
        float(temperature), float(top_p), int(top_k), _ptr(out["logprob"]), _ptr(out["entropy"]),
        _ptr(out["saved"]), _ptr(out["nucleus_size"]), _ptr(out["flags"]), _ptr(ws), ws_n,
        _stream(dev))
    _native.check(st, "rlk_logprob_fused_linear")
    return out


def logprob_fused_linear_bwd(hidden: torch.Tensor, weight: torch.Tensor, targets: torch.Tensor,
                             saved: torch.Tensor, grad_logprob=None, grad_entropy=None,
                             temperature: float = 1.0, top_p: float = 1.0, *,
                             top_k: int = 0) -> tuple[torch.Tensor, torch.Tensor]:
    """Backward of the fused LM head: (dL/dhidden bf16 [N, H], dL/dW fp32 [V, H])."""
    N, H = hidden.shape
    V = weight.shape[0]
    dev = hidden.device
    targets = targets.to(device=dev, dtype=torch.int64).contiguous()
    g_lp = _f32_opt(grad_logprob, N, dev)
    g_h = _f32_opt(grad_entropy, N, dev)
    dh = torch.empty(N, H, device=dev, dtype=torch.bfloat16)
    dw = torch.empty(V, H, device=dev, dtype=torch.float32)
    L = lib()
    ws_n = L.rlk_logprob_fused_linear_bwd_workspace_size(N, H, V, float(top_p))
    ws = _workspace(ws_n, dev)
    st = L.rlk_logprob_fused_linear_bwd(
        _ptr(hidden), _ptr(weight), N, H, V, hidden.stride(0), weight.stride(0), _ptr(targets),
        _ptr(saved.contiguous()), _ptr(g_lp), _ptr(g_h), float(temperature), float(top_p),
        int(top_k), _ptr(dh), _ptr(dw), _ptr(ws), ws_n, _stream(dev))
    _native.check(st, "rlk_logprob_fused_linear_bwd")
    return dh, dw


def grpo_token_loss(lp_new: torch.Tensor, lp_old: torch.Tensor, lp_ref, cu_seqlens,
                    *, rewards=None, advantages=None, group_size: int = 8,
                    tis_cap: float = 2.0, eps_low: float = 0.2, eps_high: float = 0.28,
                    kl_coef: float = 0.01, adv_eps: float = 1e-6, std_ddof: int = 1,
                    normalize_std: bool = True, loss_type: str = "dapo",
                    correction: str = "tis", aggregation: str = "token_mean",
                    filter_zero_adv: bool = False, baseline: str = "mean",
                    ipo_eps: float = 0.3, icepop_lo: float = 0.5,
                    icepop_hi: float = 2.0) -> dict:
    """GRPO/DAPO token loss over packed responses.

    ``cu_seqlens`` [B + 1] int64 offsets: a device tensor is passed as it is
    (nothing is read on the host, so the call can be captured in a graph);
    a host array or tensor is copied to the device first. The token count is
    ``lp_new.numel()``; offsets that do not run from 0 to it, non-decreasing,
    give NaN outputs and ``status`` = 1 (checked on the device).
    loss_type: dapo | ipo | icepop | cispo | tis_pg; correction: tis | mis;
    aggregation: token_mean | prompt_mean; baseline: mean | length.
    Returns loss (device scalar), grad (dL/dlp_new), token_loss, token_flags,
    metrics [clipped/masked frac, TIS frac, mean k3, mean ratio], advantages,
    status (device int32).
    """
    dev = lp_new.device
    if torch.is_tensor(cu_seqlens) and cu_seqlens.device == dev:
        cu = cu_seqlens
        if cu.dtype != torch.int64 or not cu.is_contiguous():
            raise ValueError("a device cu_seqlens must be a contiguous int64 tensor")
    else:
        host = cu_seqlens.cpu() if torch.is_tensor(cu_seqlens) else cu_seqlens
        cu = torch.from_numpy(np.ascontiguousarray(np.asarray(host, dtype=np.int64))).to(dev)
    B = cu.numel() - 1
    T = lp_new.numel()
    lp_new = lp_new.to(torch.float32).contiguous()
    lp_old = lp_old.to(torch.float32).contiguous()
    lp_ref = None if lp_ref is None else lp_ref.to(torch.float32).contiguous()
    rw = _f32_opt(rewards, B, dev)
    ad = _f32_opt(advantages, B, dev)
    f = dict(device=dev, dtype=torch.float32)
    out = {"loss": torch.empty((), **f), "grad": torch.empty(T, **f),
           "token_loss": torch.empty(T, **f),
           "token_flags": torch.empty(T, device=dev, dtype=torch.uint8),
           "metrics": torch.empty(4, **f), "advantages": torch.empty(max(B, 0), **f),
           "status": torch.empty((), device=dev, dtype=torch.int32)}
    prm = _native.GrpoParams(ctypes.sizeof(_native.GrpoParams), tis_cap, eps_low, eps_high,
                             kl_coef, adv_eps, std_ddof, int(bool(normalize_std)),
                             _native.LOSS_TYPES[loss_type], _native.CORRECTIONS[correction],
                             _native.AGGREGATIONS[aggregation], int(bool(filter_zero_adv)),
                             _native.BASELINES[baseline], ipo_eps, icepop_lo, icepop_hi)
    L = lib()
    ws_n = L.rlk_grpo_token_loss_workspace_size(T, B)
    ws = _workspace(ws_n, dev)
    st = L.rlk_grpo_token_loss(
        _ptr(lp_new), _ptr(lp_old), _ptr(lp_ref), _ptr(cu), B, T,
        _ptr(rw), _ptr(ad), int(group_size), ctypes.byref(prm), _ptr(out["loss"]),
        _ptr(out["grad"]), _ptr(out["token_loss"]), _ptr(out["token_flags"]), _ptr(out["metrics"]),
        _ptr(out["advantages"]), _ptr(out["status"]), _ptr(ws), ws_n, _stream(dev))
    _native.check(st, "rlk_grpo_token_loss")
    return out
