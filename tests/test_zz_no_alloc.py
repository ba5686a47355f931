"""tree_logprob_noalloc (the log-prob entry point for callers that cannot
allocate) called through the raw C ABI: two calls in a row on one device,
the second smaller, each bitwise equal to tree_logprob with a workspace on
the same inputs (the same kernels over the same entry table, summed in a
fixed order). The size limit is checked on the host."""
import ctypes

import numpy as np
import pytest
import torch

import tree_packed_attention_amd as ta
import workloads

pytestmark = pytest.mark.gpu


def _inputs(R, V, reps, seed):
    src, tgt, w = workloads.repeated_rows_entries(R, V, reps, seed)
    z = workloads.logits_input(R, V, "bf16", seed, device="cuda")
    dev = lambda a: torch.as_tensor(a, device="cuda")
    return z, dev(src), dev(tgt), dev(w)


def _noalloc(z, src, tgt, w):
    R, V = z.shape
    M = src.numel()
    logp = torch.empty(M, dtype=torch.float32, device="cuda")
    row_lse = torch.empty(R, dtype=torch.float32, device="cuda")
    loss = torch.empty((), dtype=torch.float32, device="cuda")
    dz = torch.empty_like(z)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    rc = ta.library().tree_logprob_noalloc(p(z), ta.TA_BF16, R, V, p(src), p(tgt), p(w), M, p(logp), p(row_lse),
                                           p(loss), p(dz), 1.0,
                                           ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == ta.TA_OK, ta.last_error()
    return logp, row_lse, loss, dz


def test_noalloc_equals_workspace_entry_point_twice_second_smaller():
    for R, V, reps, seed in ((4096, 32000, 3, 11), (777, 5003, 2, 12)):
        z, src, tgt, w = _inputs(R, V, reps, seed)
        got = _noalloc(z, src, tgt, w)
        ref = ta.tree_logprob(z, src, tgt, w)
        torch.cuda.synchronize()
        for name, a, b in zip(("logp", "row_lse", "loss", "dlogits"), got, ref):
            assert torch.equal(a, b), (R, name)


def test_noalloc_rejects_sizes_beyond_its_scratch():
    lib = ta.library()
    bogus = ctypes.c_void_p(0x1000)
    # 16 MiB of scratch holds about 1.3 million rows plus entries; this asks for more
    rc = lib.tree_logprob_noalloc(bogus, ta.TA_BF16, 1 << 20, 1000, bogus, bogus, bogus, 1 << 21, bogus, None, None,
                                  None, 1.0, None)
    assert rc == ta.TA_ECAPACITY and "scratch" in ta.last_error()
