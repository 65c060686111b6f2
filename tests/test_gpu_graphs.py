"""HIP graph capture of the entry points added for the loop's neighbours: the
adapter recurrence (device-side concatenation and one linear per loop), the
trajectory Hessian (tile and piece kernels) and the per-token loop (transform
kernel with per-row steps, weight expansion, GEMM).  None records a memset.
Each graph is replayed several times with eager work between replays; every
replay must equal the eager result bit for bit.
"""

import numpy as np
import pytest
import torch

from bit_ptq_looped_amd import synth

pytestmark = pytest.mark.gpu


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def pack(lq, w32, gw):
    N, K = w32.shape
    codes, scales = lq.empty_packed_weights(K, N, gw)
    lq.loopq_pack_weights(dev(w32), gw, codes, scales)
    return codes, scales


def capture(step):
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            step()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    return graph


def replay_and_compare(graph, step, out, eager, reset=None):
    for rep in range(3):
        if reset:
            reset()
        else:
            out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep}"
        if reset:
            reset()
        step()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, eager)


@pytest.mark.parametrize("M", [1, 40])
def test_recurrence_graph_replays_match_eager(lq, M):
    N, T = 1024, 6
    rng = synth.seeded_rng(synth.TEST, 230, M)
    P1, P2 = dev(synth.haar_orthogonal(32, rng)), dev(synth.haar_orthogonal(64, rng))
    s0 = dev(synth.gaussian((M, N), 231, M))
    e = dev(synth.gaussian((M, N), 232, M))
    codes, scales = pack(lq, synth.gaussian((N, 2 * N), 233, scale=0.5 / np.sqrt(2 * N)), 32)
    clips = [1.0 - 0.05 * t for t in range(T)]
    y = torch.zeros((T, M, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(lq.loopq_workspace_bytes(lq.LOOPQ_OP_RECURRENT_ADAPTER, 0, M, 0, N, 4), dtype=torch.uint8,
                     device="cuda")

    def step():
        lq.loopq_recurrent_adapter(s0, e, P1, P2, clips, 4, codes, scales, 32, y, ws)

    step()
    torch.cuda.synchronize()
    eager = y.clone()
    assert torch.isfinite(eager).all() and not torch.equal(eager[1], eager[0])
    replay_and_compare(capture(step), step, y, eager)


def test_hessian_graph_replays_match_eager(lq):
    rows, K = 300, 2048
    x = dev(synth.gaussian((rows, K), 234))
    H0 = dev(synth.gaussian((K, K), 235))
    H0 = (H0 + H0.T) * 0.5
    H = H0.clone()
    ws = torch.empty(lq.loopq_workspace_bytes(lq.LOOPQ_OP_HESSIAN, 0, rows, K, 0, 0), dtype=torch.uint8,
                     device="cuda")

    def step():
        lq.loopq_hessian_accumulate(x, H, ws)

    step()
    torch.cuda.synchronize()
    eager = H.clone()
    assert not torch.equal(eager, H0)
    H.copy_(H0)
    torch.cuda.synchronize()
    replay_and_compare(capture(step), step, H, eager, reset=lambda: H.copy_(H0))


def test_per_token_loop_graph_replays_match_eager(lq):
    T, M, K, N = 2, 100, 2048, 160
    rng = synth.seeded_rng(synth.TEST, 236)
    P1, P2 = dev(synth.haar_orthogonal(32, rng)), dev(synth.haar_orthogonal(64, rng))
    x = dev(synth.gaussian((T, M, K), 237))
    codes, scales = pack(lq, synth.gaussian((N, K), 238, scale=0.02), 32)
    y = torch.zeros((T, M, N), dtype=torch.float32, device="cuda")
    ws = lq.empty_workspace(lq.LOOPQ_OP_LOOPED_FORWARD_PER_TOKEN, T, M, K, N, 4)

    def step():
        lq.loopq_looped_forward_per_token(x, P1, P2, [0.9, 0.8], 4, codes, scales, 32, N, y, ws)

    step()
    torch.cuda.synchronize()
    eager = y.clone()
    replay_and_compare(capture(step), step, y, eager)
