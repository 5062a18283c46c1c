"""numpy-in / numpy-out wrapper over the HIP library, for parity tests.

Everything here goes through the C ABI of libep.so via the package's thin
binding; host arrays are copied to device tensors and back.  Each method
prints the case it is about to run (flushed) so that a failing GPU step is
named in the log.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import combine_get_dispatch_amd as ep


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).view(
        torch.bfloat16).cuda()


def host_bf16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def say(msg: str):
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


class GpuBackend:
    hidden_multiple = 8

    def layout(self, idx, E, R, A):
        T, k = idx.shape
        say(f"layout T={T} k={k} E={E} R={R} A={A}")
        b = ep.EpBuffers(T, 8, k, E, R, A, capacity=0)
        b.layout(dev(idx.astype(np.int32)))
        b.check_status()
        return dict(num_tokens_per_rank=b.num_tokens_per_rank.cpu().numpy(),
                    num_tokens_per_expert=b.num_tokens_per_expert.cpu().numpy(),
                    is_token_in_rank=b.is_token_in_rank.cpu().numpy(),
                    expert_offsets=b.expert_offsets.cpu().numpy(),
                    rank_offsets=b.rank_offsets.cpu().numpy())

    def dispatch(self, x, idx, w, E, R, A, fp8, cap):
        T, H = x.shape
        k = idx.shape[1]
        say(f"dispatch T={T} H={H} k={k} E={E} R={R} A={A} fp8={fp8} cap={cap}")
        b = ep.EpBuffers(T, H, k, E, R, A, fp8=fp8, capacity=cap)
        b.row_src.fill_(-2)
        idx_d = dev(idx.astype(np.int32))
        b.layout(idx_d)
        b.dispatch(dev_bf16(x), idx_d, None if w is None else dev(w.astype(np.float32)))
        b.check_status()
        recv = b.recv_x.cpu().numpy() if fp8 else host_bf16(b.recv_x)
        return dict(recv_x=recv,
                    recv_scales=b.recv_scales.cpu().numpy() if fp8 else None,
                    recv_weights=b.recv_weights.cpu().numpy() if w is not None else None,
                    tok_slot_row=b.tok_slot_row.cpu().numpy(),
                    row_src=b.row_src.cpu().numpy(),
                    buffers=b)

    def combine(self, y, tsr, w):
        cap, H = y.shape
        T, k = tsr.shape
        say(f"combine T={T} H={H} k={k} cap={cap} weighted={w is not None}")
        tsr_d = dev(tsr.astype(np.int32))
        h = ep.make_handle(T, H, k, cap, tsr_d)
        out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        ep.ep_combine(h, dev_bf16(y), None if w is None else dev(w.astype(np.float32)), out)
        torch.cuda.synchronize()
        return host_bf16(out)
