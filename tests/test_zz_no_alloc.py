"""GPU test of fa_fwd_varlen_noalloc, the packed forward without a workspace argument.

Its decoding kernels keep their partial states in the library's fixed device array instead of a
caller workspace.  Checked through the C ABI against fa_fwd_varlen with a caller workspace (same
kernels, so the outputs must be equal bit for bit) and against the fp64 oracle, on two calls in
a row whose second input is smaller (fewer sequences, heads and keys, so fewer key ranges): the
array keeps the first call's contents, which must not leak into the second.  Once the library is
loaded, the call must not change the device's free memory.
"""

import numpy as np
import pytest
import torch

import exact_tiled_attention_19_amd as fa
import oracle
from exact_tiled_attention_19_amd import workloads as W
from tests import parity_util as PU

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    fa.load_library()
    # The first kernel launch of a process loads the library's code object, and with it every
    # device global of the library (the 9 MiB array among them): free memory drops then, whatever
    # entry point launches first.  One call of the workspace entry point does that here, so the
    # measurements below see only what the allocation-free calls themselves do.
    q, k, v, cu_q, cu_k = W.random_packed([1, 1], [3000, 700], 2, 64, BF16, 1)
    fa.forward_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cu_q.to(DEV), cu_k.to(DEV), 1, 3000)
    torch.cuda.synchronize()


def _inputs(lq, lk, H, d, seed):
    q, k, v, cu_q, cu_k = W.random_packed(lq, lk, H, d, BF16, seed)
    return q, k, v, cu_q, cu_k


def _both(q, k, v, cu_q, cu_k, lq, lk, d, causal, align, out_dtype):
    dq, dk, dv, dcq, dck = (t.to(DEV) for t in (q, k, v, cu_q, cu_k))
    Tq, H = q.shape[0], q.shape[1]
    # outputs allocated before the call: the entry point itself allocates nothing
    o_na = torch.empty((Tq, H, d), dtype=out_dtype, device=DEV)
    l_na = torch.empty((H, Tq), dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    free_before = torch.cuda.mem_get_info()[0]
    fa.forward_varlen(dq, dk, dv, dcq, dck, max(lq), max(lk), scale=W.scale_for(d), causal=causal, align=align,
                      out_dtype=out_dtype, out=o_na, lse_out=l_na, noalloc=True)
    torch.cuda.synchronize()
    free_after = torch.cuda.mem_get_info()[0]
    o_ws, l_ws = fa.forward_varlen(dq, dk, dv, dcq, dck, max(lq), max(lk), scale=W.scale_for(d), causal=causal,
                                   align=align, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o_na.cpu(), l_na.cpu(), o_ws.cpu(), l_ws.cpu(), free_before, free_after


# (first call, second call): decoding shapes whose keys are split into several ranges (so the
# fixed array is used), the second smaller than the first
PAIRS = {
    "one_row": (([1] * 4, [8192] * 4, 16, 128), ([1] * 2, [3000, 700], 8, 128)),
    "four_rows": (([4, 3, 4], [5000, 4100, 9000], 8, 64), ([2, 4], [1500, 2600], 4, 64)),
    "decode_then_prefill": (([1, 1, 1], [4000, 0, 1200], 4, 128), ([30, 20], [700, 100], 2, 128)),
    # prefill shapes whose keys are split into ranges (the split tile kernel and its merge)
    "prefill_split": (([300, 77], [3000, 1100], 2, 128), ([200], [1500], 1, 128)),
}


@pytest.mark.parametrize("out_dtype", [BF16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("pair", list(PAIRS))
def test_noalloc_equals_workspace_entry_point_on_two_calls(pair, out_dtype):
    for i, (lq, lk, H, d) in enumerate(PAIRS[pair]):
        causal, align = (True, "bottom_right") if i == 0 else (True, "top_left")
        q, k, v, cu_q, cu_k = _inputs(lq, lk, H, d, seed=700 + i)
        label = f"{pair} call {i + 1}: lq={lq} lk={lk} H={H} d={d} out={out_dtype}"
        print(f"[noalloc] {label} (workspace {fa.varlen_workspace_size(len(lq), H, max(lq), max(lk), d)} B)",
              flush=True)
        o_na, l_na, o_ws, l_ws, fb, fa_ = _both(q, k, v, cu_q, cu_k, lq, lk, d, causal, align, out_dtype)
        assert torch.equal(o_na, o_ws), label
        assert torch.equal(l_na, l_ws), label
        assert fb == fa_, f"{label}: free device memory changed by {fb - fa_} bytes"
        O_ref, L_ref = oracle.attention_varlen_ref(q, k, v, cu_q.tolist(), cu_k.tolist(), W.scale_for(d),
                                                   causal=causal, align=align)
        res = PU.compare(o_na, l_na, O_ref, L_ref, out_dtype, label=label)
        print(f"[noalloc] {label}: {res}", flush=True)


def test_noalloc_prefill_split_beyond_the_array_runs_unsplit():
    """A prefill shape whose split keys need more workspace than the fixed array holds: the
    allocation-free entry point runs the tiled kernel unsplit (no error, nothing allocated), and
    its output matches the oracle; the workspace entry point splits."""
    lq, lk, H, d = [3000], [3000], 4, 128
    assert fa.varlen_workspace_size(len(lq), H, max(lq), max(lk), d) > fa.binding.scratch_bytes()
    q, k, v, cu_q, cu_k = _inputs(lq, lk, H, d, seed=720)
    for out_dtype in (BF16, torch.float32):
        label = f"prefill beyond the array: lq={lq} H={H} d={d} out={out_dtype}"
        print(f"[noalloc] {label}", flush=True)
        o_na, l_na, o_ws, l_ws, fb, fa_ = _both(q, k, v, cu_q, cu_k, lq, lk, d, True, "bottom_right", out_dtype)
        assert fb == fa_, f"{label}: free device memory changed by {fb - fa_} bytes"
        O_ref, L_ref = oracle.attention_varlen_ref(q, k, v, cu_q.tolist(), cu_k.tolist(), W.scale_for(d),
                                                   causal=True, align="bottom_right")
        for name, (o, l) in (("noalloc", (o_na, l_na)), ("workspace", (o_ws, l_ws))):
            res = PU.compare(o, l, O_ref, L_ref, out_dtype, label=f"{label} {name}")
            print(f"[noalloc] {label} {name}: {res}", flush=True)
