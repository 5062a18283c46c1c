"""Calls from several host threads on different streams at once: each
thread has its own buffers and its own (default-priority) stream and runs
repeated layout -> dispatch -> combine steps while the other does the same.
Every thread's last results are compared with the CPU oracle."""
import threading

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import combine_get_dispatch_amd as ep  # noqa: E402
import ep_workloads as W  # noqa: E402
import oracle  # noqa: E402
from tests.gpu_backend import dev, dev_bf16, host_bf16, say  # noqa: E402


def _case(seed, T, H, k, E, R, fp8):
    rng = np.random.default_rng(seed)
    idx = W.random_routes(rng, T, E, k, mask_prob=0.03)
    x = W.normal_bf16(rng, (T, H))
    w = rng.random((T, k)).astype(np.float32)
    y = W.normal_bf16(rng, (T * k, H))
    return dict(T=T, H=H, k=k, E=E, R=R, fp8=fp8, idx=idx, x=x, w=w, y=y)


def test_two_threads_two_streams():
    cases = [_case(31, 700, 1024, 8, 64, 8, False), _case(32, 1500, 512, 4, 32, 4, True)]
    for c in cases:
        say(f"concurrent case T={c['T']} H={c['H']} k={c['k']} E={c['E']} R={c['R']} "
            f"fp8={c['fp8']}")
        c["b"] = ep.EpBuffers(c["T"], c["H"], c["k"], c["E"], c["R"], 1, fp8=c["fp8"])
        c["d"] = [dev(c["idx"]), dev_bf16(c["x"]), dev(c["w"]), dev_bf16(c["y"])]
    torch.cuda.synchronize()
    errors = []

    def run(c):
        try:
            s = torch.cuda.Stream()
            idx_d, x_d, w_d, y_d = c["d"]
            b = c["b"]
            with torch.cuda.stream(s):
                for _ in range(20):
                    b.layout(idx_d)
                    b.dispatch(x_d, idx_d, w_d)
                    c["out"] = b.combine(y_d, w_d)
            s.synchronize()
        except Exception as e:  # reported in the main thread
            errors.append(e)

    threads = [threading.Thread(target=run, args=(c,)) for c in cases]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    torch.cuda.synchronize()
    for c in cases:
        b = c["b"]
        b.check_status()
        lo = oracle.layout(c["idx"], c["E"], c["R"], 1)
        do = oracle.dispatch(c["x"], c["idx"], c["w"], c["E"], c["R"], 1, fp8=c["fp8"],
                             capacity=c["T"] * c["k"])
        ref, _ = oracle.combine(c["y"], do["tok_slot_row"], c["w"])
        rows = int(lo["expert_offsets"][-1])
        assert np.array_equal(b.expert_offsets.cpu().numpy(), lo["expert_offsets"])
        assert np.array_equal(b.tok_slot_row.cpu().numpy(), do["tok_slot_row"])
        got = b.recv_x[:rows].cpu()
        got = got.numpy() if c["fp8"] else host_bf16(got)
        assert np.array_equal(got, do["recv_x"][:rows])
        if c["fp8"]:
            assert np.array_equal(b.recv_scales[:rows].cpu().numpy(), do["recv_scales"][:rows])
        assert np.array_equal(host_bf16(c["out"]), ref)
