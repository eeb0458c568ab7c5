"""The step recorded in a HIP graph (gpt_step_async + muon_update captured once, then
replayed on new batches copied into the captured token buffers) against the same steps
run eagerly on an identical model: every replay's loss (read back with
gpt_step_result) and the updated weights must match bit for bit, with eager work and
synchronisations between the replays.  The launch-bound small configurations are the
ones a graph serves."""
import numpy as np
import pytest
import torch

from gpt_pretraining_step_train_amd import binding, configs, inputs
from tests.gpu_util import say

pytestmark = pytest.mark.gpu
LR = 0.02


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.lib()
    torch.cuda.set_device(0)


@pytest.mark.parametrize("name", ["tiny", "laptop"])
def test_graph_replays_match_eager_steps(name):
    cfg = configs.get(name)
    params = inputs.init_weights(cfg, 0)
    batches = [inputs.token_batch(cfg["batch"], cfg["seq_len"], cfg["vocab"], dist=cfg["tokens"], seed=s)
               for s in range(4)]
    dev = [(torch.from_numpy(t).cuda(), torch.from_numpy(y).cuda()) for t, y in batches]
    L = cfg["depth"]
    watch = [1, 5, 1 + 6 * (L - 1) + 6, 1 + 6 * L]  # Wq and W1 of layer 0, W2 of the last layer, U
    eager = binding.Model(cfg, seed=0)
    eager.set_all_params(params)
    ref = []
    for tk, tg in dev:
        loss = eager.step(tk, tg)
        eager.muon_update(LR)
        ref.append((loss, [eager.get_params(i) for i in watch]))
    # every kernel of the step and the update loaded before the capture
    warm = binding.Model(cfg, seed=1)
    warm.step(*dev[0])
    warm.muon_update(LR)
    torch.cuda.synchronize()
    model = binding.Model(cfg, seed=0)
    model.set_all_params(params)
    tok = torch.empty_like(dev[0][0])
    tgt = torch.empty_like(dev[0][1])
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        model.step_async(tok, tgt)
        model.muon_update(LR)
    for s, (tk, tg) in enumerate(dev):
        tok.copy_(tk)
        tgt.copy_(tg)
        graph.replay()
        torch.cuda.synchronize()
        loss = model.step_result()
        got = [model.get_params(i) for i in watch]
        say(f"  {name} replay {s}: loss {loss:.6f} (eager {ref[s][0]:.6f})")
        assert loss == ref[s][0]
        for a, b in zip(got, ref[s][1]):
            np.testing.assert_array_equal(a, b)
        torch.cuda.synchronize()
