"""The fused step captured in a HIP graph (torch.cuda.CUDAGraph on ROCm) and
replayed: the library allocates nothing and keeps no per-call state, so a
captured step reads the caller's buffers at replay time.  Every replay is
checked bit for bit against an eager call on the same inputs, with eager
work, input changes and synchronizations between replays."""
import numpy as np
import pytest
import torch

from top_sparse_decode_amd import api, synth

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def say(*a):
    print(*a, flush=True)


CASES = {
    "dsa_fast": (4, dict(batch=2, kv_len=[9000, 4100], topk=2048), api.FAST),
    "dsa_exact": (4, dict(batch=2, kv_len=[5000, 300], topk=1024), api.EXACT),
    "dsa_next_n2": (4, dict(batch=2, kv_len=[6000, 3000], topk=1024, next_n=2), api.FAST),
    "gqa_exact": (3, dict(batch=2, kv_len=[3000, 2049], topk=1024), api.EXACT),
}


def outputs(step):
    torch.cuda.synchronize()
    return (step.indices.cpu().numpy().copy(), step.counts.cpu().numpy().copy(),
            step.out.view(torch.int16 if step.out.dtype == torch.bfloat16 else torch.int32).cpu().numpy().copy())


def clobber(step):
    step.indices.fill_(-7)
    step.counts.fill_(-7)
    step.out.fill_(float("nan"))


def same(a, b):
    return all(np.array_equal(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replay_matches_eager(name):
    cfg, kw, precision = CASES[name]
    w = synth.make_workload(cfg, **kw)
    say(f"[graph] {name}")
    step = api.prepare(w, precision=precision)
    # the query inputs of two steps, swapped into the same buffers
    qs = [step.q.clone(), torch.randn_like(step.q.float()).to(step.q.dtype)]
    sqs = [step.score_q.clone(), torch.randn_like(step.score_q.float()).to(step.score_q.dtype)]

    def set_inputs(i):
        step.q.copy_(qs[i])
        if step.score_q.data_ptr() != step.q.data_ptr():
            step.score_q.copy_(sqs[i])

    refs = []
    for i in range(2):
        set_inputs(i)
        step.run()
        refs.append(outputs(step))
    assert not same(refs[0], refs[1]), "the two inputs should give different steps"

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream
        set_inputs(0)
        step.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step.run()
    torch.cuda.synchronize()

    a = torch.randn(512, 512, device="cuda")
    for rep, i in enumerate([0, 1, 1, 0]):
        set_inputs(i)
        clobber(step)
        (a @ a).sum().item()  # unrelated eager work, synchronizing
        g.replay()
        got = outputs(step)
        assert same(got, refs[i]), f"replay {rep} (inputs {i}) differs from the eager step"
