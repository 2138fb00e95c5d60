"""Concurrent calls: every entry point enqueues on the caller's stream and
keeps no state between calls, so calls on two streams (default priority),
each with its own inputs, outputs and workspace, may overlap. Each result
must be bitwise the one the same call gives alone on the default stream."""
import numpy as np
import pytest
import torch

import synth
import grpo_loss_rlk_amd as rlk

from gpu_util import DEV, bf16_to_device, bits_equal

pytestmark = pytest.mark.gpu


def _tensors(o):
    if isinstance(o, dict):
        return [o[k] for k in sorted(o) if torch.is_tensor(o[k])]
    return [t for t in o if torch.is_tensor(t)]


def _concurrent_matches_alone(calls, rounds=3):
    """calls: zero-argument functions with distinct inputs. Each is run alone
    first; then all are enqueued round-robin on two side streams, several
    rounds in flight at once, and every result compared with its own."""
    alone = []
    for c in calls:
        alone.append([t.clone() for t in _tensors(c())])
        torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    got = []
    for _ in range(rounds):
        for k, c in enumerate(calls):
            with torch.cuda.stream(streams[k % 2]):
                got.append((k, _tensors(c())))
    torch.cuda.synchronize()
    for k, outs in got:
        for a, b in zip(outs, alone[k]):
            assert bits_equal(a, b), k


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_logits_in_on_two_streams(dtype):
    N, V = 96, 32768
    r = np.random.default_rng(21)
    make = (lambda a: bf16_to_device(synth.bf16_bits_from_f32(a)) if dtype == "bf16"
            else torch.as_tensor(a.astype(np.float32)).to(DEV))
    ins = [(make(r.normal(0, 2.5, (N, V))), torch.as_tensor(r.integers(0, V, N)).to(DEV))
           for _ in range(4)]
    print(f"  rlk_logprob_from_logits on two streams N={N} V={V} {dtype}", flush=True)
    _concurrent_matches_alone([lambda x=x, y=y: rlk.logprob_from_logits(x, y, 0.7, 0.95)
                               for x, y in ins])


@pytest.mark.parametrize("p", [1.0, 0.9])
def test_fused_forward_on_two_streams(p):
    N, H, V = 600, 256, 5003
    w = synth.workload("fused", N=N, H=H, V=V)
    r = np.random.default_rng(22)
    W = bf16_to_device(synth.weight_rows(w, range(V)))
    ins = [(bf16_to_device(synth.bf16_bits_from_f32(r.normal(0, 1, (N, H)))),
            torch.as_tensor(r.integers(0, V, N)).to(DEV)) for _ in range(4)]
    print(f"  rlk_logprob_fused_linear on two streams N={N} H={H} V={V} p={p}", flush=True)
    _concurrent_matches_alone([lambda h=h, y=y: rlk.logprob_fused_linear(h, W, y, 0.7, p)
                               for h, y in ins])


def test_fused_backward_on_two_streams():
    N, H, V = 300, 128, 40000
    w = synth.workload("fused", N=N, H=H, V=V)
    r = np.random.default_rng(23)
    W = bf16_to_device(synth.weight_rows(w, range(V)))
    glp = torch.full((N,), -1.0 / N, device=DEV)
    gh = torch.full((N,), -0.001 / N, device=DEV)
    ins = []
    for _ in range(2):
        h = bf16_to_device(synth.bf16_bits_from_f32(r.normal(0, 1, (N, H))))
        y = torch.as_tensor(r.integers(0, V, N)).to(DEV)
        saved = rlk.logprob_fused_linear(h, W, y, 0.7, 0.95)["saved"]
        ins.append((h, y, saved))
    torch.cuda.synchronize()
    print(f"  rlk_logprob_fused_linear_bwd on two streams N={N} H={H} V={V}", flush=True)
    _concurrent_matches_alone(
        [lambda h=h, y=y, s=s: rlk.logprob_fused_linear_bwd(h, W, y, s, glp, gh, 0.7, 0.95)
         for h, y, s in ins], rounds=2)


def test_sampler_on_two_streams():
    N, V = 64, 20000
    r = np.random.default_rng(24)
    xs = [bf16_to_device(synth.bf16_bits_from_f32(r.normal(0, 2.5, (N, V)))) for _ in range(4)]
    print(f"  rlk_sample_top_p on two streams N={N} V={V}", flush=True)
    _concurrent_matches_alone([lambda x=x, k=k: rlk.sample_top_p(x, 0.7, 0.95, 1234 + k, 3)
                               for k, x in enumerate(xs)])


def test_grpo_loss_on_two_streams():
    B, T = 32, 4000
    r = np.random.default_rng(25)
    mk = lambda a: torch.as_tensor(a.astype(np.float32)).to(DEV)
    ins = []
    for _ in range(4):
        cut = np.sort(r.choice(np.arange(1, T), B - 1, replace=False))
        cu = torch.as_tensor(np.concatenate([[0], cut, [T]]).astype(np.int64)).to(DEV)
        lp = r.normal(-2, 1, T)
        ins.append((mk(lp), mk(lp + r.normal(0, 0.4, T)), mk(lp + r.normal(0, 0.3, T)), cu,
                    mk(r.integers(0, 2, B).astype(np.float32))))
    print(f"  rlk_grpo_token_loss on two streams B={B} T={T}", flush=True)
    _concurrent_matches_alone(
        [lambda a=a: rlk.grpo_token_loss(a[0], a[1], a[2], a[3], rewards=a[4], group_size=8)
         for a in ins])
