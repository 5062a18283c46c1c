"""One step (layout, dispatch, combine) captured once as a HIP graph and
replayed with new inputs.

Every call only enqueues kernels on the caller's stream: no allocation, no
memset, no host synchronisation (the layout's ticket is reset by its own
last workgroup).  So a caller can capture a step and replay it after copying
new routes, hidden states and expert outputs into the captured tensors.
Each replay is checked against an eager run on separate buffers and against
the oracle, with unrelated eager work and synchronisations between replays.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import combine_get_dispatch_amd as ep  # noqa: E402
import ep_workloads as W  # noqa: E402
import oracle  # noqa: E402
from tests.gpu_backend import dev_bf16, host_bf16, say  # noqa: E402

CASES = [
    # T, H, k, E, R, A, fp8, fused (layout and dispatch in one launch)
    (1000, 256, 4, 32, 4, 1, True, False),     # four tiles: the ticket path
    (300, 264, 3, 24, 4, 4, False, False),     # alignment padding (pad fill kernel)
    (128, 7168, 8, 256, 8, 1, False, False),   # the Decode shape
    (128, 7168, 8, 256, 8, 1, False, True),    # the Decode shape, fused
    (200, 512, 4, 32, 4, 4, True, True),       # fused, FP8 rows and padding
]


def _bf16_tensor(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).view(
        torch.bfloat16)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "T{}_H{}_k{}_E{}_A{}_{}{}".format(
    c[0], c[1], c[2], c[3], c[5], "fp8" if c[6] else "bf16", "_fused" if c[7] else ""))
def test_graph_replay_matches_eager_and_oracle(case):
    T, H, k, E, R, A, fp8, fused = case
    say(f"graph T={T} H={H} k={k} E={E} R={R} A={A} fp8={fp8} fused={fused}")
    rng = np.random.default_rng(4242 + T)
    b = ep.EpBuffers(T, H, k, E, R, A, fp8=fp8)
    cap = b.capacity
    x_d = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    idx_d = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w_d = torch.empty((T, k), dtype=torch.float32, device="cuda")
    y_d = torch.empty((cap, H), dtype=torch.bfloat16, device="cuda")

    def draw():
        idx = W.random_routes(rng, T, E, k, mask_prob=0.1)
        w = rng.random((T, k)).astype(np.float32)
        x = W.normal_bf16(rng, (T, H))
        y = W.normal_bf16(rng, (cap, H))
        return idx, w, x, y

    def load(inputs):
        idx, w, x, y = inputs
        idx_d.copy_(torch.from_numpy(idx))
        w_d.copy_(torch.from_numpy(w))
        x_d.copy_(_bf16_tensor(x))
        y_d.copy_(_bf16_tensor(y))

    def step():
        if fused:
            b.layout_dispatch(x_d, idx_d, w_d)
        else:
            b.layout(idx_d)
            b.dispatch(x_d, idx_d, w_d)
        b.combine(y_d, w_d)

    load(draw())
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    b.check_status()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    eager = ep.EpBuffers(T, H, k, E, R, A, fp8=fp8)
    for rep in range(4):
        say(f"graph replay {rep}")
        inputs = draw()
        load(inputs)
        # unrelated eager work and a synchronisation between replays
        junk = torch.arange(1 << 16, device="cuda", dtype=torch.float32).sum()
        torch.cuda.synchronize()
        assert float(junk.item()) > 0
        g.replay()
        torch.cuda.synchronize()
        b.check_status()

        idx, w, x, y = inputs
        idx_e = torch.from_numpy(idx).cuda()
        w_e = torch.from_numpy(w).cuda()
        eager.layout(idx_e)
        eager.dispatch(dev_bf16(x), idx_e, w_e)
        out_e = eager.combine(dev_bf16(y), w_e)
        eager.check_status()

        used = int(b.expert_offsets[-1].item())
        assert used == int(eager.expert_offsets[-1].item())
        for name in ("num_tokens_per_expert", "num_tokens_per_rank", "is_token_in_rank",
                     "expert_offsets", "rank_offsets", "tok_slot_row"):
            assert torch.equal(getattr(b, name), getattr(eager, name)), name
        assert torch.equal(b.row_src[:used], eager.row_src[:used])
        assert torch.equal(b.recv_weights[:used].view(torch.int32),
                           eager.recv_weights[:used].view(torch.int32))
        if fp8:
            assert torch.equal(b.recv_x[:used], eager.recv_x[:used])
            assert torch.equal(b.recv_scales[:used].view(torch.int32),
                               eager.recv_scales[:used].view(torch.int32))
        else:
            assert torch.equal(b.recv_x[:used].view(torch.int16),
                               eager.recv_x[:used].view(torch.int16))
        assert torch.equal(b.out.view(torch.int16), out_e.view(torch.int16))

        lay = oracle.layout(idx, E, R, A)
        d = oracle.dispatch(x, idx, w, E, R, A, fp8=fp8)
        assert np.array_equal(b.expert_offsets.cpu().numpy(), lay["expert_offsets"])
        assert np.array_equal(b.tok_slot_row.cpu().numpy(), d["tok_slot_row"])
        got = b.recv_x[:used].cpu().numpy() if fp8 else host_bf16(b.recv_x[:used])
        assert np.array_equal(got, d["recv_x"][:used])
        ref, _ = oracle.combine(y, d["tok_slot_row"], w)
        assert np.array_equal(host_bf16(b.out), ref)


def test_calls_enqueue_on_torch_current_stream():
    """The binding's default stream is torch's current one, also inside a
    `torch.cuda.stream` block."""
    say("current stream handle")

    def handle():
        return ep._stream(None).value or 0  # the null stream marshals as None

    assert handle() == torch.cuda.current_stream().cuda_stream
    side = torch.cuda.Stream()
    assert side.cuda_stream != 0
    with torch.cuda.stream(side):
        assert handle() == side.cuda_stream
    assert handle() == torch.cuda.current_stream().cuda_stream
