"""The entry point that allocates nothing, kda_chunk_fwd_fused_gate_noalloc, against the
workspace form of kda_chunk_fwd_fused_gate (the same kernels): two calls in a row, the
second smaller, each equal to the workspace form bit for bit and within the bf16 bar of
the oracle; no device memory is allocated by the call."""
import numpy as np
import pytest
import torch

import synth
from tests.helpers import assert_close, oracle_prefill

pytestmark = pytest.mark.gpu

kda = pytest.importorskip("gated_delta_rule_31_amd")


def _case(msg):
    print("[case] " + msg, flush=True)


def _noalloc_vs_workspace(inp, C):
    d = lambda x: None if x is None else x.cuda()
    q, k, v, z, ls, be, s0 = (d(x) for x in (inp.q, inp.k, inp.v, inp.z, inp.log_scale, inp.beta,
                                             inp.initial_state))
    B, T, H, K, V = inp.dims
    N = inp.num_seqs
    cu = d(inp.cu_seqlens)
    out = torch.full((B, T, H, V), float("nan"), dtype=torch.float32, device="cuda")
    fin = torch.full((N, H, K, V), float("nan"), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    kda.chunk_fwd_fused_gate_noalloc(q, k, v, z, ls, be, out, initial_state=s0, final_state=fin, cu_seqlens=cu,
                                     chunk_size=C)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before  # nothing allocated on the way
    ro, rf = kda.chunk_fwd_fused_gate(q, k, v, z, ls, be, initial_state=s0, cu_seqlens=cu, chunk_size=C,
                                      out_dtype=torch.float32, two_pass=True)
    assert torch.equal(out, ro) and torch.equal(fin, rf)
    eo, ef = oracle_prefill(inp)
    assert_close(out, eo, False, "out")
    assert_close(fin, ef, False, "final state")


def test_noalloc_two_calls_second_smaller():
    cap = kda.noalloc_scratch_bytes()
    assert cap == 64 << 20
    _case("noalloc: K3 widths, 600 tokens, 96 heads (a segmented call)")
    big = synth.make_prefill(1, 600, 96, 128, 128, seed=61, qk="silu", v_kind="silu", z_std=1.5, alog_std=0.5,
                             state_std=0.1)
    assert 0 < kda.chunk_fwd_workspace_size(torch.bfloat16, 1, 600, 96, 128, 128, 32) <= cap
    _noalloc_vs_workspace(big, 32)
    _case("noalloc: packed sequences, 3 heads, K=V=64")
    small = synth.make_prefill(1, 150, 3, 64, 64, seed=62, state_std=0.1, seqlens=[70, 0, 80])
    _noalloc_vs_workspace(small, 32)


def test_noalloc_refuses_beyond_its_array():
    _case("noalloc: a shape beyond the array is refused")
    T = 4096
    assert kda.chunk_fwd_workspace_size(torch.bfloat16, 1, T, 96, 128, 128, 32) > kda.noalloc_scratch_bytes()
    x = torch.zeros(1, T, 96, 128, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(1, T, 96, 128, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="unsupported"):
        kda.chunk_fwd_fused_gate_noalloc(x, x, x, x, torch.zeros(96, device="cuda"),
                                         torch.zeros(1, T, 96, device="cuda"), out)


def test_noalloc_chunk64_k128():
    """The same entry point at chunk size 64 with K = V = 128 (the pre-pass that stages the
    key columns in two halves), on packed sequences with an empty one."""
    _case("noalloc: chunk size 64, K=V=128, packed sequences")
    inp = synth.make_prefill(1, 300, 4, 128, 128, seed=63, state_std=0.1, seqlens=[130, 0, 170], alog_std=0.5)
    assert 0 < kda.chunk_fwd_workspace_size(torch.bfloat16, 1, 300, 4, 128, 128, 64) <= kda.noalloc_scratch_bytes()
    _noalloc_vs_workspace(inp, 64)
