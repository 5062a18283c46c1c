"""GPU parity of the non-expanded (rank-deduplicated) path against the
oracle: ep_dispatch_ranked (rank partitions, rows, local top-k slices,
handles), ep_expand (identical to the expanded dispatch) and
ep_combine_ranked (fp32 per-rank partials and the rank-ordered sum,
bit-exact against the oracle's two-stage sum)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import combine_get_dispatch_amd as ep  # noqa: E402
import ep_workloads as W  # noqa: E402
import oracle  # noqa: E402
from tests.gpu_backend import dev, dev_bf16, host_bf16, say  # noqa: E402


def check(T, H, k, E, R, A, fp8, idx, w, x, y, weighted=True):
    say(f"ranked T={T} H={H} k={k} E={E} R={R} A={A} fp8={fp8}")
    b = ep.EpBuffers(T, H, k, E, R, A, fp8=fp8)
    idx_d, w_d = dev(idx), dev(w)
    b.row_src.fill_(-2)
    used = b.layout(idx_d, sync=True)
    b.dispatch_ranked(dev_bf16(x), idx_d, w_d)
    b.expand()
    y_d = dev_bf16(y)
    out = b.combine_ranked(y_d, weighted=weighted)
    b.check_status()
    torch.cuda.synchronize()

    ne = oracle.dispatch_ranked(x, idx, w, E, R, fp8=fp8)
    rows = int(ne["rank_token_offsets"][-1])
    assert np.array_equal(b.rank_token_offsets.cpu().numpy(), ne["rank_token_offsets"])
    assert np.array_equal(b.tok_rank_row.cpu().numpy(), ne["tok_rank_row"])
    assert np.array_equal(b.ne_src[:rows].cpu().numpy(), ne["recv_src"][:rows])
    assert np.array_equal(b.ne_topk_idx[:rows].cpu().numpy(), ne["recv_topk_idx"][:rows])
    assert np.array_equal(b.ne_topk_weights[:rows].cpu().numpy().view(np.uint32),
                          ne["recv_topk_weights"][:rows].view(np.uint32))
    if fp8:
        assert np.array_equal(b.ne_x[:rows].cpu().numpy(), ne["recv_x"][:rows])
        assert np.array_equal(b.ne_scales[:rows].cpu().numpy().view(np.uint32),
                              ne["recv_scales"][:rows].view(np.uint32))
    else:
        assert np.array_equal(host_bf16(b.ne_x[:rows]), ne["recv_x"][:rows])
    d = oracle.dispatch(x, idx, w, E, R, A, fp8=fp8)
    assert np.array_equal(b.tok_slot_row.cpu().numpy(), d["tok_slot_row"])
    got_x = b.recv_x[:used].cpu().numpy() if fp8 else host_bf16(b.recv_x[:used])
    assert np.array_equal(got_x, d["recv_x"][:used])
    assert np.array_equal(b.row_src[:used].cpu().numpy(), d["row_src"][:used])
    assert np.array_equal(b.recv_weights[:used].cpu().numpy().view(np.uint32),
                          d["recv_weights"][:used].view(np.uint32))
    if fp8:
        assert np.array_equal(b.recv_scales[:used].cpu().numpy().view(np.uint32),
                              d["recv_scales"][:used].view(np.uint32))
    ref, acc, part = oracle.combine_ranked(y, d["tok_slot_row"], ne, weighted=weighted)
    assert np.array_equal(b.partials[:rows].cpu().numpy().view(np.uint32), part.view(np.uint32))
    assert np.array_equal(host_bf16(out), ref)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "skewed", "large"])
def test_ranked_workloads(name):
    w = W.WORKLOADS[name]
    inp = W.generate(w)
    check(w.num_tokens, w.hidden, w.num_topk, w.num_experts, w.num_ranks, w.alignment, w.fp8,
          inp["topk_idx"], inp["topk_weights"], inp["x"], inp["y"])


@pytest.mark.parametrize("case", [
    (300, 24, 3, 16, 4, 1, False), (257, 136, 2, 80, 40, 1, False), (100, 128, 4, 128, 64, 2, True),
    (1000, 1032, 8, 64, 8, 4, False), (513, 384, 6, 24, 3, 8, True), (1, 256, 2, 4, 2, 1, True),
    (700, 2056, 5, 40, 5, 1, False), (64, 128, 8, 8, 8, 1, False),
    # Rows wider than one expand wave's batch of 8 column chunks (H > 8192).
    (40, 9216, 4, 16, 4, 1, True), (33, 8200, 3, 12, 3, 2, False), (17, 16512, 8, 8, 2, 1, True),
])
def test_ranked_random_small(case):
    T, H, k, E, R, A, fp8 = case
    rng = np.random.default_rng(T * 7 + H)
    idx = W.random_routes(rng, T, E, k, mask_prob=0.15)
    w = rng.random((T, k)).astype(np.float32)
    x = W.normal_bf16(rng, (T, H))
    y = W.normal_bf16(rng, (T * k + E * (A - 1), H))
    check(T, H, k, E, R, A, fp8, idx, w, x, y, weighted=bool(T % 2))


@pytest.mark.parametrize("seed", range(24))
def test_ranked_random_shapes(seed):
    """Random shapes: tokens across several tiles, hidden sizes with ragged
    chunks, experts, ranks, top-k, alignment, payload type and gates drawn
    from the seed."""
    rng = np.random.default_rng(8000 + seed)
    R = int(rng.choice([1, 2, 4, 8, 16]))
    E = R * int(rng.integers(1, 9))
    k = int(rng.integers(1, min(E, 8) + 1))
    fp8 = bool(rng.integers(0, 2))
    H = 128 * int(rng.integers(1, 7)) if fp8 else 8 * int(rng.integers(1, 161))
    T = int(rng.integers(0, 1500))
    A = int(rng.choice([1, 2, 4]))
    idx = W.random_routes(rng, T, E, k, mask_prob=float(rng.choice([0.0, 0.1, 0.3])))
    w = rng.random((T, k)).astype(np.float32)
    x = W.normal_bf16(rng, (T, H))
    y = W.normal_bf16(rng, (T * k + E * (A - 1), H))
    check(T, H, k, E, R, A, fp8, idx, w, x, y, weighted=bool(rng.integers(0, 2)))
