"""The seeded device inputs: a prefix drawn alone equals the same elements of the
whole fill. bench.py times the CPU oracle on the first 2^26 elements of the
inputs before it allocates the shard, so those elements must be the ones the
timed steps see."""
import pytest
import torch

import workloads as W
from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,S", [("gpt2s", None), ("llama7b", (1 << 27) + 4099)])
def test_prefix_equals_whole_fill(name, S):
    w = W.get(name)
    if S is None:
        S = 15_554_976
    covered = [(0, S // 3), (S // 3 + 100, S - S // 3 - 100)]
    n = min(S, 1 << 26)
    say(f"prefix of {n} of {S} ({name})")
    whole = torch.empty(S, dtype=torch.bfloat16, device="cuda")
    W.device_fill_replica(whole, w, covered, 0, 0, 5)
    pre = W.device_prefix(W.device_fill_replica, S, n, torch.bfloat16, "cuda", w, covered, 0, 0, 5)
    assert torch.equal(pre.view(torch.int16), whole[:n].view(torch.int16))
    del whole
    whole = torch.empty(S, dtype=torch.float32, device="cuda")
    W.device_fill_params(whole, w, covered, 0)
    pre = W.device_prefix(W.device_fill_params, S, n, torch.float32, "cuda", w, covered, 0)
    assert torch.equal(pre.view(torch.int32), whole[:n].view(torch.int32))
    with pytest.raises(ValueError):
        W.device_prefix(W.device_fill_params, S, (1 << 27) + 1, torch.float32, "cuda", w, covered, 0)
