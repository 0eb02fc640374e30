"""GPU: the entry points inside a captured graph (torch.cuda.CUDAGraph over HIP graphs).

The library allocates, frees and synchronises nothing and records no memset, so a caller can
capture its launches, as serving loops do.  Each graph is replayed several times with eager
work (the outputs overwritten with NaN) and a device synchronisation between replays; every
replay must reproduce the eager result bitwise (same kernels on the same inputs).

Covered: the forward's pipelined kernel and its two key-split kernels for small grids, the FP8
forward, a decoding step of the packed forward (split-key kernel, merge, caller workspace), a
packed prefill with its keys split into ranges (split tile kernel, merge) and the backward pass.
"""

import pytest
import torch

import exact_tiled_attention_19_amd as fa
from exact_tiled_attention_19_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    fa.load_library()


def _capture_and_replay(fn, outs, replays=4):
    fn()                                   # eager reference into the same output buffers
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    side = torch.cuda.Stream()             # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                               # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for i in range(replays):
        for o in outs:                     # eager work between replays
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), f"replay {i} differs from the eager result"


@pytest.mark.parametrize("shape", [(2, 4, 1024, 128, True), (1, 1, 4096, 64, False), (1, 4, 2048, 64, True)],
                         ids=["pipelined", "key-split-16-rows", "key-split-32-rows"])
def test_forward_in_graph(shape):
    B, H, N, d, causal = shape
    q, k, v, _ = W.random_qkv(B, H, N, d, torch.bfloat16, seed=81)
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    o = torch.empty(B, H, N, d, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(B, H, N, dtype=torch.float32, device=DEV)
    _capture_and_replay(lambda: fa.forward(q, k, v, causal=causal, out=o, lse_out=lse), [o, lse])


def test_forward_fp8_in_graph():
    q8, k8, v8, ds = W.random_qkv_fp8(1, 2, 700, 128, seed=82)
    q8, k8, v8 = q8.to(DEV), k8.to(DEV), v8.to(DEV)
    o = torch.empty(1, 2, 700, 128, dtype=torch.float32, device=DEV)
    lse = torch.empty(1, 2, 700, dtype=torch.float32, device=DEV)
    _capture_and_replay(lambda: fa.forward_fp8(q8, k8, v8, descale_q=ds[0], descale_k=ds[1], descale_v=ds[2],
                                               causal=True, out_dtype=torch.float32, out=o, lse_out=lse), [o, lse])


def test_decode_step_in_graph():
    lq, lk, H, d = [1, 1], [3000, 700], 2, 64
    qp, kp, vp, cq, ck = W.random_packed(lq, lk, H, d, torch.bfloat16, seed=83)
    qp, kp, vp, cq, ck = (t.to(DEV) for t in (qp, kp, vp, cq, ck))
    o = torch.empty(sum(lq), H, d, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(H, sum(lq), dtype=torch.float32, device=DEV)      # [H, Tq]
    ws_bytes = fa.varlen_workspace_size(len(lq), H, max(lq), max(lk), d)
    assert ws_bytes > 0   # several key ranges: the split-key kernel and the merge both run
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    # the longest lengths are passed, so the binding reads nothing back from the device
    _capture_and_replay(lambda: fa.forward_varlen(qp, kp, vp, cq, ck, max(lq), max(lk), causal=True, out=o,
                                                  lse_out=lse, workspace=ws), [o, lse])


def test_split_prefill_in_graph():
    lq, lk, H, d = [300, 77], [3000, 1100], 2, 128
    qp, kp, vp, cq, ck = W.random_packed(lq, lk, H, d, torch.bfloat16, seed=86)
    qp, kp, vp, cq, ck = (t.to(DEV) for t in (qp, kp, vp, cq, ck))
    o = torch.empty(sum(lq), H, d, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(H, sum(lq), dtype=torch.float32, device=DEV)
    ws_bytes = fa.varlen_workspace_size(len(lq), H, max(lq), max(lk), d)
    assert ws_bytes > 0   # the keys are split into ranges: the split tile kernel and its merge run
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    _capture_and_replay(lambda: fa.forward_varlen(qp, kp, vp, cq, ck, max(lq), max(lk), causal=True, out=o,
                                                  lse_out=lse, workspace=ws), [o, lse])


def test_backward_in_graph():
    B, H, N, d = 1, 2, 300, 64
    q, k, v, _ = W.random_qkv(B, H, N, d, torch.bfloat16, seed=84)
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    o, lse = fa.forward(q, k, v, causal=True)
    g = torch.Generator("cpu").manual_seed(85)
    do = torch.randn(B, H, N, d, generator=g).to(torch.bfloat16).to(DEV)
    grads = tuple(torch.empty(B, H, N, d, dtype=torch.float32, device=DEV) for _ in range(3))
    delta = torch.empty(B, H, N, dtype=torch.float32, device=DEV)
    _capture_and_replay(lambda: fa.backward(q, k, v, o, lse, do, causal=True, out=grads, delta=delta), list(grads))
