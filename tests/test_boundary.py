"""CPU tests of the C ABI boundary and the host-side logic (no GPU work is launched).

* libfa.so loads and exports every function include/fa.h declares.
* Every invalid argument is rejected on the host with the documented status before any HIP
  call (the arguments below always fail validation, so nothing reaches the GPU).
* The workgroup -> (head, query tile) mapping is a bijection (host compile of fa_sched.h).
"""

import ctypes
import math
import os
import re
import subprocess

import pytest

import exact_tiled_attention_19_amd as fa
from exact_tiled_attention_19_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

F32, BF16 = fa.FA_DTYPE_F32, fa.FA_DTYPE_BF16
P = 0x10000          # a 16-byte-aligned stand-in address; validation fails before any use
P2 = 0x40000000
P3 = 0x80000000
P4 = 0xC0000000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(fa_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_expected_api():
    assert declared_functions() == sorted(binding.SIGNATURES)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(fa.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", fa.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (fa_\w+)$", out, flags=re.M))
    assert set(declared_functions()) <= exported


def test_version_matches_header():
    m = re.search(r"#define FA_VERSION (\d+)", open(HEADER).read())
    assert fa.version() == int(m.group(1))


def test_status_strings():
    lib = fa.load_library()
    for code in (fa.FA_OK, fa.FA_ERR_INVALID_ARG, fa.FA_ERR_UNSUPPORTED, fa.FA_ERR_HIP):
        s = lib.fa_status_str(code)
        assert s and s.decode().startswith(("FA_OK", "FA_ERR"))
    assert lib.fa_status_str(12345).decode() == "unknown fa_status"
    assert lib.fa_status_str(-1)
    assert lib.fa_last_hip_error() == 0
    assert fa.variant_count() >= 1


def call(q=P, k=P2, v=P3, o=P4, lse=None, B=1, H=1, N=16, d=64, scale=0.125, mask=0, seqlens=None,
         ind=BF16, outd=BF16, variant=0):
    return fa.fa_fwd(q, k, v, o, lse, B, H, N, d, scale, mask, seqlens, ind, outd, None, variant)


INVALID = {
    "null q": dict(q=None),
    "null k": dict(k=None),
    "null v": dict(v=None),
    "null o": dict(o=None),
    "negative B": dict(B=-1),
    "negative H": dict(H=-2),
    "negative N": dict(N=-16),
    "mask bit 4": dict(mask=4),
    "mask -1": dict(mask=-1),
    "padding without seqlens": dict(mask=fa.FA_MASK_KEY_PADDING),
    "causal+padding without seqlens": dict(mask=3),
    "nan scale": dict(scale=float("nan")),
    "inf scale": dict(scale=float("inf")),
    "negative scale": dict(scale=-0.125),
    "misaligned q": dict(q=P + 2),
    "misaligned k": dict(k=P2 + 8),
    "misaligned v": dict(v=P3 + 4),
    "misaligned o": dict(o=P4 + 2),
    "misaligned lse": dict(lse=P4 + (1 << 24) + 2),
    "misaligned seqlens": dict(mask=2, seqlens=P4 + (1 << 24) + 1),
    "o aliases q": dict(o=P),
    "o overlaps v": dict(o=P3 + 16),
    "lse inside o": dict(lse=P4 + 64),
    "bad in dtype": dict(ind=7),
    "bad out dtype": dict(outd=-1),
    "d zero": dict(d=0),
    "too many workgroups": dict(B=1 << 20, H=1 << 10, N=1 << 20),
}

UNSUPPORTED = {
    "d 32": dict(d=32),
    "d 96": dict(d=96),
    "d 256": dict(d=256),
    "f32 in bf16 out": dict(ind=F32, outd=BF16),
    "unknown variant": dict(variant=99),
    "negative variant": dict(variant=-1),
    "f32 with variant 1": dict(ind=F32, outd=F32, variant=1),
    "eight-wave variant at d 64": dict(variant=3),
}


@pytest.mark.parametrize("name", sorted(INVALID))
def test_invalid_argument_rejected_on_host(name):
    assert call(**INVALID[name]) == fa.FA_ERR_INVALID_ARG, name


@pytest.mark.parametrize("name", sorted(UNSUPPORTED))
def test_unsupported_rejected_on_host(name):
    assert call(**UNSUPPORTED[name]) == fa.FA_ERR_UNSUPPORTED, name


@pytest.mark.parametrize("dims", [(0, 1, 16), (1, 0, 16), (1, 1, 0), (0, 0, 0)])
def test_empty_problem_is_a_noop(dims):
    B, H, N = dims
    # null pointers are fine for an empty problem: nothing is read, written or launched
    assert fa.fa_fwd(None, None, None, None, None, B, H, N, 64, 0.125, 0, None, BF16, BF16, None) == fa.FA_OK
    assert fa.fa_fwd(None, None, None, None, None, B, H, N, 128, 0.125, 3, None, BF16, F32, None) == fa.FA_OK


def bwd_call(q=P, k=P2, v=P3, o=P4, lse=P4 + (1 << 26), dout=P + (1 << 26), delta=P2 + (1 << 26),
             dq=P3 + (1 << 26), dk=P + (1 << 27), dv=P2 + (1 << 27), B=1, H=1, N=16, d=64, scale=0.125, mask=0,
             seqlens=None, ind=BF16, gd=F32):
    return fa.fa_bwd(q, k, v, o, lse, dout, delta, dq, dk, dv, B, H, N, d, scale, mask, seqlens, ind, gd, None)


BWD_INVALID = {
    "null q": dict(q=None), "null lse": dict(lse=None), "null dout": dict(dout=None),
    "null delta": dict(delta=None), "null dq": dict(dq=None), "null dv": dict(dv=None),
    "negative N": dict(N=-1), "mask bit 4": dict(mask=4), "padding without seqlens": dict(mask=2),
    "nan scale": dict(scale=float("nan")), "misaligned o": dict(o=P4 + 2), "misaligned dk": dict(dk=P + (1 << 27) + 8),
    "misaligned delta": dict(delta=P2 + (1 << 26) + 2), "dq aliases q": dict(dq=P), "dk overlaps dv": dict(dk=P2 + (1 << 27) + 64),
    "delta inside dq": dict(delta=P3 + (1 << 26) + 64), "bad grad dtype": dict(gd=5), "d zero": dict(d=0),
}
BWD_UNSUPPORTED = {"d 96": dict(d=96), "f32 inputs": dict(ind=F32), "bf16 gradients": dict(gd=BF16)}


@pytest.mark.parametrize("name", sorted(BWD_INVALID))
def test_bwd_invalid_argument_rejected_on_host(name):
    assert bwd_call(**BWD_INVALID[name]) == fa.FA_ERR_INVALID_ARG, name


@pytest.mark.parametrize("name", sorted(BWD_UNSUPPORTED))
def test_bwd_unsupported_rejected_on_host(name):
    assert bwd_call(**BWD_UNSUPPORTED[name]) == fa.FA_ERR_UNSUPPORTED, name


def test_bwd_empty_problem_is_a_noop():
    assert fa.fa_bwd(*([None] * 10), 0, 4, 16, 64, 0.125, 1, None, BF16, F32, None) == fa.FA_OK


# ---- packed variable-length entry point --------------------------------------------------------
VQ, VK, VV, VO = 0x10000, 0x40000000, 0x80000000, 0xC0000000
VCQ, VCK, VL, VW = 0x100000000, 0x100001000, 0x140000000, 0x180000000


def varlen_call(q=VQ, k=VK, v=VV, o=VO, lse=VL, cu_q=VCQ, cu_k=VCK, B=2, H=2, total_q=64, total_k=64, max_q=32,
                max_k=32, d=64, scale=0.125, mask=0, align=fa.FA_ALIGN_BOTTOM_RIGHT, ws=None, ws_bytes=0, ind=BF16,
                outd=BF16):
    return fa.fa_fwd_varlen(q, k, v, o, lse, cu_q, cu_k, B, H, total_q, total_k, max_q, max_k, d, scale, mask, align,
                            ws, ws_bytes, ind, outd, None)


DEC = dict(max_q=1, total_q=2, max_k=8192)   # decoding shape: needs a workspace for these sizes
VARLEN_INVALID = {
    "null q": dict(q=None), "null o": dict(o=None), "null cu_q": dict(cu_q=None), "null cu_k": dict(cu_k=None),
    "null k with keys": dict(k=None), "null v with keys": dict(v=None),
    "negative B": dict(B=-1), "negative H": dict(H=-1), "negative total_q": dict(total_q=-1),
    "negative total_k": dict(total_k=-5), "negative max_q": dict(max_q=-1), "negative max_k": dict(max_k=-1),
    "key padding bit": dict(mask=fa.FA_MASK_KEY_PADDING), "causal and padding": dict(mask=3), "mask -1": dict(mask=-1),
    "alignment 2": dict(align=2), "alignment -1": dict(align=-1, mask=1),
    "nan scale": dict(scale=float("nan")), "negative scale": dict(scale=-1.0),
    "misaligned q": dict(q=VQ + 2), "misaligned k": dict(k=VK + 8), "misaligned o": dict(o=VO + 4),
    "misaligned lse": dict(lse=VL + 2), "misaligned cu_q": dict(cu_q=VCQ + 2), "misaligned cu_k": dict(cu_k=VCK + 1),
    "bad in dtype": dict(ind=9), "bad out dtype": dict(outd=3), "d zero": dict(d=0),
    "o aliases q": dict(o=VQ), "o overlaps v": dict(o=VV + 32), "lse inside o": dict(lse=VO + 64),
    "lse overlaps cu_q": dict(lse=VCQ), "o overlaps cu_k": dict(o=VCK - 64),
    "key range beyond 32-bit buffer": dict(H=64, d=128, max_k=300000),
    "decode without workspace": dict(DEC),
    "decode workspace too small": dict(DEC, ws=VW, ws_bytes=16),
    "decode workspace misaligned": dict(DEC, ws=VW + 8, ws_bytes=1 << 24),
    "decode workspace overlaps o": dict(DEC, ws=VO, ws_bytes=1 << 24),
}
VARLEN_UNSUPPORTED = {"d 96": dict(d=96), "d 256": dict(d=256), "f32 inputs": dict(ind=F32, outd=F32)}


@pytest.mark.parametrize("name", sorted(VARLEN_INVALID))
def test_varlen_invalid_argument_rejected_on_host(name):
    assert varlen_call(**VARLEN_INVALID[name]) == fa.FA_ERR_INVALID_ARG, name


@pytest.mark.parametrize("name", sorted(VARLEN_UNSUPPORTED))
def test_varlen_unsupported_rejected_on_host(name):
    assert varlen_call(**VARLEN_UNSUPPORTED[name]) == fa.FA_ERR_UNSUPPORTED, name


@pytest.mark.parametrize("dims", [dict(B=0), dict(H=0), dict(total_q=0), dict(max_q=0)])
def test_varlen_empty_problem_is_a_noop(dims):
    args = dict(q=None, k=None, v=None, o=None, lse=None, cu_q=None, cu_k=None)
    args.update(dims)
    assert varlen_call(**args) == fa.FA_OK


def test_varlen_workspace_size():
    """Workspace only where keys are split into ranges: decoding shapes (<= 4 query rows),
    B*H*ranges*rows*(d+2)*4 bytes; and prefill shapes whose 128-row tiles number at most 128
    with at least 1024 keys, ranges*B*H*max_q*(d+1)*4 bytes.  A pure function of the sizes."""
    ws = fa.varlen_workspace_size
    assert ws(64, 64, 300, 8192, 128) == 0              # prefill, 12288 tiles fill the chip: unsplit
    assert ws(4, 16, 512, 8192, 128) == 0               # prefill, 256 tiles (one workgroup per CU): unsplit
    assert ws(4, 16, 300, 1000, 128) == 0               # prefill, too few keys to split
    for B, H, mq, mk, d in [(4, 16, 5, 8192, 128), (1, 2, 8192, 8192, 128), (1, 1, 4096, 4096, 64), (2, 3, 300, 1100, 64)]:
        n = ws(B, H, mq, mk, d)
        unit = B * H * mq * (d + 1) * 4
        tiles = B * H * -(-mq // 128)
        assert n > 0 and n % unit == 0, (B, H, mq, mk, d, n)
        S = n // unit
        assert 2 <= S <= min(16, mk // 512, -(-512 // tiles)), S
        assert ws(B, H, mq, mk, d) == n                 # deterministic
    assert ws(64, 64, 1, 8192, 128) == 0                # 4096 heads fill the chip: one range
    assert ws(4, 16, 1, 500, 128) == 0                  # too few keys to split
    assert ws(-1, 16, 1, 8192, 128) == 0 and ws(4, 16, 1, 8192, 96) == 0
    for B, H, mq, mk, d in [(4, 16, 1, 8192, 128), (1, 8, 1, 131072, 128), (2, 3, 4, 5000, 64), (1, 1, 2, 1 << 20, 64)]:
        g = 1 if mq == 1 else 4
        n = ws(B, H, mq, mk, d)
        unit = B * H * g * (d + 2) * 4
        assert n > 0 and n % unit == 0, (B, H, mq, mk, d, n)
        S = n // unit
        assert 2 <= S <= max(2, -(-2048 // (B * H))) and S <= -(-mk // 512), S
        assert ws(B, H, mq, mk, d) == n                 # deterministic


def drop_call(p=0.1, seed=1, offset=0, ind=BF16, outd=BF16, d=64, N=16, **kw):
    a = dict(q=P, k=P2, v=P3, o=P4, lse=None, B=1, H=1, scale=0.125, mask=0, seqlens=None)
    a.update(kw)
    return fa.fa_fwd_dropout(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], N, d, a["scale"], a["mask"],
                             a["seqlens"], p, seed, offset, ind, outd, None)


DROP_INVALID = {"p negative": dict(p=-0.01), "p one": dict(p=1.0), "p nan": dict(p=float("nan")),
                "p inf": dict(p=float("inf")), "null q": dict(q=None), "o aliases q": dict(o=P),
                "misaligned v": dict(v=P3 + 2), "mask bit 4": dict(mask=4)}


@pytest.mark.parametrize("name", sorted(DROP_INVALID))
def test_dropout_invalid_argument_rejected_on_host(name):
    assert drop_call(**DROP_INVALID[name]) == fa.FA_ERR_INVALID_ARG, name


def test_dropout_unsupported_and_empty():
    assert drop_call(ind=F32, outd=F32) == fa.FA_ERR_UNSUPPORTED
    assert drop_call(d=96) == fa.FA_ERR_UNSUPPORTED
    assert drop_call(N=0, q=None, k=None, v=None, o=None) == fa.FA_OK


def test_python_forward_rejects_host_tensors():
    import torch
    x = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.forward(x, x, x)


def test_sched_mapping_is_bijective(tmp_path):
    """Host compile of the work-mapping header: every logical item is visited once."""
    src = tmp_path / "sched_test.cpp"
    src.write_text(
        '#include "fa_sched.h"\n#include <cstdio>\n#include <vector>\n'
        "int main() {\n"
        "  int bad = 0;\n"
        "  for (int total = 1; total <= 3000; ++total) {\n"
        "    std::vector<int> seen(total, 0);\n"
        "    for (int w = 0; w < total; ++w) { int l = fa::xcd_remap(w, total);\n"
        "      if (l < 0 || l >= total) { ++bad; continue; } ++seen[l]; }\n"
        "    for (int i = 0; i < total; ++i) if (seen[i] != 1) ++bad;\n"
        "    // items that share an XCD are contiguous in logical order\n"
        "    for (int w = 8; w < total; ++w) if (fa::xcd_remap(w, total) != fa::xcd_remap(w - 8, total) + 1) ++bad;\n"
        "  }\n"
        "  for (int nq : {1, 2, 7, 64}) for (int causal = 0; causal < 2; ++causal) {\n"
        "    std::vector<int> seen(3 * nq, 0);\n"
        "    for (int l = 0; l < 3 * nq; ++l) { fa::TileCoord t = fa::tile_of(l, nq, causal);\n"
        "      if (t.qt < 0 || t.qt >= nq || t.bh < 0 || t.bh >= 3) { ++bad; continue; } ++seen[t.bh * nq + t.qt]; }\n"
        "    for (int x : seen) if (x != 1) ++bad;\n"
        "    if (causal && fa::tile_of(0, nq, true).qt != nq - 1) ++bad;\n"
        "  }\n"
        "  // causal pairing: every (head, tile) exactly once, equal work (t+1 + n-t) per pair\n"
        "  for (int nq = 1; nq <= 70; ++nq) for (int causal = 0; causal < 2; ++causal) {\n"
        "    const int per = fa::items_per_head(nq, causal);\n"
        "    std::vector<int> seen(3 * nq, 0);\n"
        "    for (int l = 0; l < 3 * per; ++l) { fa::TilePair t = fa::pair_of(l, nq, causal);\n"
        "      if (t.bh < 0 || t.bh >= 3 || t.qt0 < 0 || t.qt0 >= nq) { ++bad; continue; } ++seen[t.bh * nq + t.qt0];\n"
        "      if (t.qt1 >= 0) { if (!causal || t.qt1 >= nq) ++bad; else ++seen[t.bh * nq + t.qt1];\n"
        "        if (t.qt0 + t.qt1 != nq - 1) ++bad; } }\n"
        "    for (int x : seen) if (x != 1) ++bad;\n"
        "  }\n"
        "  // packed sequences: head bh on XCD bh % 8, every (head, item) exactly once\n"
        "  for (int nh : {1, 3, 8, 13, 256, 300}) for (int per : {1, 2, 5, 16}) {\n"
        "    const int grid = (nh + 7) / 8 * 8 * per;\n"
        "    std::vector<int> seen(nh * per, 0);\n"
        "    for (int w = 0; w < grid; ++w) { fa::HeadItem t = fa::head_item_xcd(w, nh, per);\n"
        "      if (t.bh < 0) continue; if (t.bh >= nh || t.it < 0 || t.it >= per || t.bh % 8 != w % 8) { ++bad; continue; }\n"
        "      ++seen[t.bh * per + t.it]; }\n"
        "    for (int x : seen) if (x != 1) ++bad;\n"
        "  }\n"
        '  std::printf("bad=%d\\n", bad);\n'
        "  return bad != 0;\n"
        "}\n")
    exe = tmp_path / "sched_test"
    inc = os.path.join(ROOT, "exact_tiled_attention_19_amd", "csrc")
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", inc, str(src), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr


def test_no_undefined_kernel_symbols():
    """Every kernel the dispatcher can launch has its host stub in the library (a kernel whose
    host-side instantiation is dropped shows up as an undefined symbol and breaks loading)."""
    out = subprocess.run(["nm", "-D", "--undefined-only", fa.LIB_PATH], capture_output=True, text=True).stdout
    assert not [l for l in out.splitlines() if "fa_fwd" in l or "_ZN2fa" in l], out


def fp8_call(dq=1.0, dk=1.0, dv=1.0, outd=BF16, d=64, N=16, **kw):
    a = dict(q=P, k=P2, v=P3, o=P4, lse=None, B=1, H=1, scale=0.125, mask=0, seqlens=None)
    a.update(kw)
    return fa.fa_fwd_fp8(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], N, d, a["scale"], dq, dk, dv,
                         a["mask"], a["seqlens"], outd, None)


FP8_INVALID = {"descale_q nan": dict(dq=float("nan")), "descale_k negative": dict(dk=-1.0),
               "descale_v inf": dict(dv=float("inf")), "scale * descales overflows float32": dict(dq=1e30, dk=1e30),
               "null k": dict(k=None), "o aliases v": dict(o=P3), "misaligned q": dict(q=P + 8),
               "mask bit 4": dict(mask=4), "padding without seqlens": dict(mask=fa.FA_MASK_KEY_PADDING),
               "unknown out dtype": dict(outd=fa.FA_DTYPE_FP8_E4M3)}


@pytest.mark.parametrize("name", sorted(FP8_INVALID))
def test_fp8_invalid_argument_rejected_on_host(name):
    assert fp8_call(**FP8_INVALID[name]) == fa.FA_ERR_INVALID_ARG, name


def test_fp8_unsupported_and_empty():
    assert fp8_call(d=96) == fa.FA_ERR_UNSUPPORTED
    assert fp8_call(d=32) == fa.FA_ERR_UNSUPPORTED
    assert fp8_call(N=0, q=None, k=None, v=None, o=None) == fa.FA_OK
    # 8-bit inputs have only the production kernel, and no dropout path
    assert call(ind=fa.FA_DTYPE_FP8_E4M3, variant=1) == fa.FA_ERR_UNSUPPORTED
    assert drop_call(ind=fa.FA_DTYPE_FP8_E4M3) == fa.FA_ERR_UNSUPPORTED


def test_python_fp8_forward_rejects_bad_tensors():
    import torch
    x = torch.zeros(1, 1, 4, 64, dtype=torch.uint8)
    with pytest.raises(ValueError):
        fa.forward_fp8(x, x, x)


# ---- allocation-free packed entry point ----------------------------------------------------------

def varlen_noalloc_call(q=VQ, k=VK, v=VV, o=VO, lse=VL, cu_q=VCQ, cu_k=VCK, B=2, H=2, total_q=64, total_k=64,
                        max_q=32, max_k=32, d=64, scale=0.125, mask=0, align=fa.FA_ALIGN_BOTTOM_RIGHT, ind=BF16,
                        outd=BF16, **_ignored):
    return fa.binding.fa_fwd_varlen_noalloc(q, k, v, o, lse, cu_q, cu_k, B, H, total_q, total_k, max_q, max_k, d,
                                            scale, mask, align, ind, outd, None)


# every check of fa_fwd_varlen except those about the caller's workspace, which this entry point
# does not take
NOALLOC_INVALID = {n: a for n, a in VARLEN_INVALID.items() if "workspace" not in n}


@pytest.mark.parametrize("name", sorted(NOALLOC_INVALID))
def test_varlen_noalloc_invalid_argument_rejected_on_host(name):
    assert varlen_noalloc_call(**NOALLOC_INVALID[name]) == fa.FA_ERR_INVALID_ARG, name


@pytest.mark.parametrize("name", sorted(VARLEN_UNSUPPORTED))
def test_varlen_noalloc_unsupported_rejected_on_host(name):
    assert varlen_noalloc_call(**VARLEN_UNSUPPORTED[name]) == fa.FA_ERR_UNSUPPORTED, name


@pytest.mark.parametrize("dims", [dict(B=0), dict(H=0), dict(total_q=0), dict(max_q=0)])
def test_varlen_noalloc_empty_problem_is_a_noop(dims):
    args = dict(q=None, k=None, v=None, o=None, lse=None, cu_q=None, cu_k=None)
    args.update(dims)
    assert varlen_noalloc_call(**args) == fa.FA_OK


def test_scratch_holds_every_decode_plan():
    """The fixed array (9 MiB) is at least the workspace of every size fa_fwd_varlen accepts: the
    plan aims at 2048 workgroups, so (sequence, head) pairs times key ranges stay below 4096."""
    cap = fa.binding.scratch_bytes()
    assert cap == 9 << 20
    lib = fa.load_library()
    assert lib.fa_status_str(fa.binding.FA_ERR_SCRATCH_LIMIT).decode().startswith("FA_ERR_SCRATCH_LIMIT")
    worst = 0
    for d in (64, 128):
        for mq in (1, 2, 4):
            for bh in list(range(1, 130)) + list(range(130, 2100, 7)) + [2047, 2048, 2049, 4096, 100000]:
                for mk in (512, 513, 1000, 4097, 8192, 65536, 131072, 1 << 20, 1 << 24):
                    worst = max(worst, fa.varlen_workspace_size(1, bh, mq, mk, d))
    assert 0 < worst <= cap, worst
