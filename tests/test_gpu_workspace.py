"""Workspaces shared between calls: the per-stream default workspace of the
binding, the fixed ticket header (a call's partial states never land where a
later call keeps its tickets), and the ticket reset."""
import numpy as np
import pytest
import torch

import quantized_kv_cache_amd as qkv
from tests._cases import assert_close, oracle_attention, oracle_pack, to_dev, W

pytestmark = pytest.mark.gpu

TICKETS = qkv._lib.QKV_TICKET_BYTES


def _case(seed, B, Hq, Hk, L, D=128, mode="affine", bits=4, gs=64):
    q = W.random_case(seed, (B, Hq, 1, D), "normal", "f16")
    k = W.random_case(seed + 1, (B, Hk, L, D), "normal", "f16")
    v = W.random_case(seed + 2, (B, Hk, L, D), "normal", "f16")
    kp = qkv.qkv_quantize(to_dev(k, "f16"), mode, bits, gs)
    vp = qkv.qkv_quantize(to_dev(v, "f16"), mode, bits, gs)
    ref = oracle_attention(q, "f16", oracle_pack(k, "f16", mode, bits, gs),
                           oracle_pack(v, "f16", mode, bits, gs), L, mode, bits, gs, 0.1)
    return to_dev(q, "f16"), kp, vp, ref


def test_default_workspace_is_per_stream():
    """Two streams run split decodes (fused merge, tickets in the workspace)
    at the same time on the binding's default workspace: each stream has its
    own buffer, so every result is right."""
    a = _case(11, 2, 16, 4, 9000)
    b = _case(12, 1, 32, 8, 12000)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    n = 40
    outs = [[torch.empty_like(c[0]) for _ in range(n)] for c in (a, b)]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for i in range(n):
        for j, (s, (qd, kp, vp, _)) in enumerate(zip(streams, (a, b))):
            with torch.cuda.stream(s):
                qkv.qsdpa_decode(qd, kp, vp, kp.L_cap, 0.1, num_splits=16, out=outs[j][i])
    torch.cuda.synchronize()
    bufs = {k: v for k, v in qkv.api._default_ws._buf.items()
            if k[1] in [s.cuda_stream for s in streams]}
    assert len(bufs) == 2
    for j, c in enumerate((a, b)):
        assert qkv.qsdpa_plan(c[0], c[1], c[1].L_cap, num_splits=16)["kernel"] == "attn_decode_narrow"
        for i in range(n):
            assert_close(outs[j][i], c[3], f"stream {j} call {i}")
        assert all(torch.equal(o, outs[j][0]) for o in outs[j])


def test_states_of_small_calls_never_reach_tickets_of_large_ones():
    """A generic-kernel call with many row tiles writes partial states; then a
    fused-merge decode with 128 (batch, kv head) tickets runs on the same
    workspace.  The ticket header has one fixed size, so the states stay out
    of it and the decode is right, repeatedly."""
    ws = qkv.Workspace()
    small = _case(21, 1, 64, 2, 3000)                     # GQA 32: 4 row tiles of states
    big = _case(22, 16, 32, 8, 2100)                      # 128 narrow-decode tickets
    assert qkv.qsdpa_plan(big[0], big[1], 2100, num_splits=3)["kernel"] == "attn_decode_narrow"
    for rep in range(3):
        for splits in (7, 3):
            out = qkv.qsdpa_decode(small[0], small[1], small[2], 3000, 0.1, num_splits=splits,
                                   algo="generic", workspace=ws)
            assert_close(out, small[3], f"generic rep {rep}")
            out = qkv.qsdpa_decode(big[0], big[1], big[2], 2100, 0.1, num_splits=splits,
                                   workspace=ws)
            assert_close(out, big[3], f"narrow rep {rep} splits {splits}")
    torch.cuda.synchronize()
    assert not ws.get(1, big[0].device)[:TICKETS].any()


def test_reset_recovers_from_stale_tickets():
    """Tickets left non-zero (as by a call that never completed) would make
    the fused merge run at the wrong moment; qsdpa_workspace_reset zeroes
    them, after which the decode is right again."""
    qd, kp, vp, ref = _case(31, 2, 16, 4, 8000)
    ws = qkv.Workspace()
    need = qkv.qsdpa_plan(qd, kp, 8000, num_splits=16)["workspace_bytes"]
    buf = ws.get(need, qd.device)
    buf[:TICKETS].view(torch.int32).fill_(5)              # 5 < S - 1: wrong counts
    ws.reset(qd.device)
    torch.cuda.synchronize()
    assert not buf[:TICKETS].any()
    for _ in range(3):
        out = qkv.qsdpa_decode(qd, kp, vp, 8000, 0.1, num_splits=16, workspace=ws)
        assert_close(out, ref, "after reset")
    torch.cuda.synchronize()
    assert not buf[:TICKETS].any()
