"""Changed-input graph replay (a test category of the pages' own GPU suite):
an entry point captured once into a HIP graph (torch.cuda.graph) and
replayed with new inputs copied into the same buffers must give, on every
replay, bitwise the outputs of an eager call on those inputs. The program's
own eager work and a synchronisation come between replays. Every entry
point reads its inputs from device memory only, so each is captured as it is."""
import numpy as np
import pytest
import torch

import synth
import grpo_loss_rlk_amd as rlk

from gpu_util import DEV, bf16_to_device, bits_equal

pytestmark = pytest.mark.gpu


def _tensors(o):
    return [o[k] for k in sorted(o) if torch.is_tensor(o[k])]


def _replay_matches_eager(static_inputs, new_inputs, call):
    """Capture call() on static_inputs; for each input set, copy it in,
    replay, and compare with an eager call on a fresh copy."""
    call()                                   # warm up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = call()
    prev = None
    for k, inputs in enumerate(new_inputs):
        print(f"  replay {k}", flush=True)
        for dst, src in zip(static_inputs, inputs):
            dst.copy_(src)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in _tensors(out)]
        want = _tensors(call())              # eager, same inputs
        torch.cuda.synchronize()
        for a, b in zip(got, want):
            assert bits_equal(a, b), k
        # the inputs changed, so the replay must not have returned the last outputs
        assert prev is None or not all(bits_equal(a, b) for a, b in zip(got, prev)), k
        prev = got
        _ = torch.randn(1000, device=DEV).sum()   # unrelated eager work
        torch.cuda.synchronize()


@pytest.mark.parametrize("V,dtype", [(20000, "bf16"), (151936, "bf16"), (8192, "f32")])
def test_logits_in_graph_replay(V, dtype):
    N = 64
    r = np.random.default_rng(V)
    make = (lambda a: bf16_to_device(synth.bf16_bits_from_f32(a)) if dtype == "bf16"
            else torch.as_tensor(a.astype(np.float32)).to(DEV))
    sets = [(make(r.normal(0, 2.5, (N, V))), torch.as_tensor(r.integers(0, V, N)).to(DEV))
            for _ in range(3)]
    x, y = sets[0][0].clone(), sets[0][1].clone()
    print(f"  rlk_logprob_from_logits in a graph N={N} V={V} {dtype}", flush=True)
    _replay_matches_eager([x, y], sets, lambda: rlk.logprob_from_logits(x, y, 0.7, 0.95))


@pytest.mark.parametrize("p", [1.0, 0.9])
def test_fused_forward_graph_replay(p):
    N, H, V = 300, 128, 3001
    w = synth.workload("fused", N=N, H=H, V=V)
    r = np.random.default_rng(7)
    W = bf16_to_device(synth.weight_rows(w, range(V)))
    sets = [(bf16_to_device(synth.bf16_bits_from_f32(r.normal(0, 1, (N, H)))),
             torch.as_tensor(r.integers(0, V, N)).to(DEV)) for _ in range(3)]
    h, y = sets[0][0].clone(), sets[0][1].clone()
    print(f"  rlk_logprob_fused_linear in a graph N={N} H={H} V={V} p={p}", flush=True)
    _replay_matches_eager([h, y], sets, lambda: rlk.logprob_fused_linear(h, W, y, 0.7, p))


def test_sampler_graph_replay():
    N, V = 64, 20000
    r = np.random.default_rng(3)
    sets = [(bf16_to_device(synth.bf16_bits_from_f32(r.normal(0, 2.5, (N, V)))),) for _ in range(3)]
    x = sets[0][0].clone()
    print(f"  rlk_sample_top_p in a graph N={N} V={V}", flush=True)
    _replay_matches_eager([x], sets, lambda: rlk.sample_top_p(x, 0.7, 0.95, 99, 5))


def test_fused_backward_graph_replay():
    """Forward and backward (two vocabulary chunks, so the first and last dh
    modes both run) captured together; dh and dW on every replay."""
    N, H, V = 200, 64, 40000
    w = synth.workload("fused", N=N, H=H, V=V)
    r = np.random.default_rng(11)
    W = bf16_to_device(synth.weight_rows(w, range(V)))
    glp = torch.full((N,), -1.0 / N, device=DEV)
    gh = torch.full((N,), -0.001 / N, device=DEV)
    sets = [(bf16_to_device(synth.bf16_bits_from_f32(r.normal(0, 1, (N, H)))),
             torch.as_tensor(r.integers(0, V, N)).to(DEV)) for _ in range(3)]
    h, y = sets[0][0].clone(), sets[0][1].clone()

    def step():
        f = rlk.logprob_fused_linear(h, W, y, 0.7, 0.95)
        dh, dw = rlk.logprob_fused_linear_bwd(h, W, y, f["saved"], glp, gh, 0.7, 0.95)
        return {"dh": dh, "dw": dw, "lp": f["logprob"]}

    print(f"  rlk fused forward + backward in a graph N={N} H={H} V={V}", flush=True)
    _replay_matches_eager([h, y], sets, step)


@pytest.mark.parametrize("kw", [dict(), dict(loss_type="cispo", correction="mis",
                                             aggregation="prompt_mean", filter_zero_adv=True,
                                             baseline="length")])
def test_grpo_loss_graph_replay(kw):
    """The loss with device offsets: new log-probabilities, new response
    lengths (same token count) and new rewards on every replay."""
    B, T = 32, 4000
    r = np.random.default_rng(5)

    def one():
        cut = np.sort(r.choice(np.arange(1, T), B - 1, replace=False))
        cu = torch.as_tensor(np.concatenate([[0], cut, [T]]).astype(np.int64)).to(DEV)
        lp = r.normal(-2, 1, T)
        mk = lambda a: torch.as_tensor(a.astype(np.float32)).to(DEV)
        rew = r.integers(0, 2, B).astype(np.float32)
        rew[:8] = 1.0                              # a constant group
        return (mk(lp), mk(lp + r.normal(0, 0.4, T)), mk(lp + r.normal(0, 0.3, T)), cu, mk(rew))

    sets = [one() for _ in range(3)]
    lpn, lpo, lpr, cu, rew = (t.clone() for t in sets[0])
    print(f"  rlk_grpo_token_loss in a graph B={B} T={T} {kw}", flush=True)
    _replay_matches_eager([lpn, lpo, lpr, cu, rew], sets,
                          lambda: rlk.grpo_token_loss(lpn, lpo, lpr, cu, rewards=rew,
                                                      group_size=8, **kw))
