"""The prefill's schedule metadata, read back from the binding's workspace
after a call, against its definition:

* the chunk map: chunk slot c holds (sequence, local chunk) for c below the
  total chunk count, and (-1, -1) after it;
* the chunk offsets: the first chunk slot of each sequence (the exclusive
  prefix sum of the chunk counts ceil(length / 64)), then the total;
* the state-kernel order: longest sequence first, equal lengths by index
  (lengths above 2^20 - 2 tokens count as equal), for up to 4096 sequences
  (counted ranks up to 512, a sorting network beyond); the natural order
  beyond 4096.

The outputs cannot show the order (the chains are independent), so it is
checked here directly.  Workspace layout (the library's own): the chunk map
at offset 0 (an int32 pair per chunk slot, (T + 63 N) / 64 slots), then the
N + 1 chunk offsets and the N order entries (int32), each starting at the
next 256-byte boundary.
"""
import numpy as np
import pytest
import torch

import kda_workloads as W
from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    import gated_delta_rule_51_amd as kda
    kda.lib()
    return kda


def align256(x):
    return (x + 255) // 256 * 256


@pytest.mark.parametrize("n", [1, 2, 16, 300, 512, 513, 1025, 4096, 4200])
def test_schedule_metadata(K, n):
    rng = np.random.default_rng(500 + n)
    lens = [int(rng.choice([0, 1, 5, 64, 65, 128, int(rng.integers(0, 300))])) for _ in range(n)]
    inp = W.make_prefill(500 + n, lens, 1, 1, 32, 32, io="f32")
    say("schedule: N=%d T=%d" % (n, int(inp.cu_seqlens[-1])))
    K.chunk_prefill(inp.q.cuda(), inp.k.cuda(), inp.v.cuda(), inp.g.cuda(), inp.beta.cuda(),
                    inp.cu_seqlens.cuda())
    torch.cuda.synchronize()
    dev = torch.device("cuda", torch.cuda.current_device())
    ws = K._WS[(dev.index, torch.cuda.current_stream(dev).cuda_stream)].cpu().numpy()

    T = int(inp.cu_seqlens[-1])
    slots = (T + 63 * n) // 64
    cnt = [(L + 63) // 64 for L in lens]
    off = np.concatenate([[0], np.cumsum(cnt)]).astype(np.int32)
    total = int(off[-1])
    want_map = np.full((slots, 2), -1, np.int32)
    for s in range(n):
        for j in range(cnt[s]):
            want_map[off[s] + j] = (s, j)
    cap = (1 << 20) - 2
    want_order = sorted(range(n), key=lambda s: (-min(lens[s], cap), s)) if n <= 4096 else list(range(n))

    o_off = align256(slots * 8)
    o_order = align256(o_off + (n + 1) * 4)
    got_map = ws[:slots * 8].view(np.int32).reshape(slots, 2)
    got_off = ws[o_off:o_off + (n + 1) * 4].view(np.int32)
    got_order = ws[o_order:o_order + n * 4].view(np.int32)
    assert total <= slots
    np.testing.assert_array_equal(got_map, want_map)
    np.testing.assert_array_equal(got_off, off)
    np.testing.assert_array_equal(got_order, np.asarray(want_order, np.int32))
