"""CPU tests of the C ABI: the library loads, exports every function that
include/dah.h declares, and rejects bad host-visible arguments with the
documented status before touching the GPU.  The split planner is pure host
code and is checked here too.  No kernel is launched by these tests.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dah.h")

native = pytest.importorskip("decode_attention_head_amd._native")


def _lib():
    if not os.path.exists(native.LIB_PATH):
        pytest.fail("libdah.so is not built: run `python -m decode_attention_head_amd.build`")
    return native.lib()


def _declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([A-Za-z_]\w*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "defined")))


def test_header_declares_the_entry_points():
    decl = _declared_functions()
    for name in ("qk_norm_rope_append", "paged_decode_gqa", "decode_attn_step"):
        assert name in decl


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for name in _declared_functions():
        assert hasattr(lib, name), f"libdah.so does not export {name}"
    assert sorted(native.SIGNATURES) == _declared_functions()


def test_every_header_in_include_is_covered():
    import glob
    headers = sorted(os.path.basename(h) for h in glob.glob(os.path.join(ROOT, "include", "*.h")))
    assert headers == ["dah.h", "dah_probe.h"]


def test_probe_library_exports_every_declared_symbol():
    if not os.path.exists(native.PROBE_LIB_PATH):
        pytest.fail("libdah_probe.so is not built")
    plib = native.probe_lib()
    declared = _declared_functions(os.path.join(ROOT, "include", "dah_probe.h"))
    assert sorted(native.PROBE_SIGNATURES) == declared
    for name in declared:
        assert hasattr(plib, name)
    # argument checks happen before any launch
    assert plib.dah_probe_copy(None, A, 16, None) == 1
    assert plib.dah_probe_copy(A, A, 15, None) == 2
    assert plib.dah_probe_copy(A + 4, A, 16, None) == 4
    assert plib.dah_probe_read(A, 0, A, 1, None) == 2
    assert plib.dah_probe_read(A, 16, A, 0, None) == 2
    # paged read: NULL, unknown dtype, B < 1, max_seq_len past the table, misaligned pool
    assert plib.dah_probe_paged_read(None, A, 1, 16, A, 4, A, 2, 64, A, None) == 1
    assert plib.dah_probe_paged_read(A, A, 7, 16, A, 4, A, 2, 64, A, None) == 3
    assert plib.dah_probe_paged_read(A, A, 1, 16, A, 4, A, 0, 64, A, None) == 2
    assert plib.dah_probe_paged_read(A, A, 1, 16, A, 4, A, 2, 65, A, None) == 2
    assert plib.dah_probe_paged_read(A + 4, A, 1, 16, A, 4, A, 2, 64, A, None) == 4


def test_header_constants_match_spec_fixture():
    import json
    text = open(HEADER).read()
    consts = dict(re.findall(r"#define (DAH_\w+) (\d+)", text))
    with open(os.path.join(ROOT, "tests", "golden", "qwen3_0_6b_constants.json")) as f:
        c = json.load(f)
    assert int(consts["DAH_NUM_HEADS"]) == c["num_attention_heads"]["value"]
    assert int(consts["DAH_NUM_KV_HEADS"]) == c["num_key_value_heads"]["value"]
    assert int(consts["DAH_HEAD_DIM"]) == c["head_dim"]["value"]
    assert int(consts["DAH_PAGE_SIZE"]) == c["page_size"]["value"]


def test_status_strings():
    lib = _lib()
    for code, name in native.STATUS_NAMES.items():
        assert lib.dah_status_string(code).decode() == name
    assert lib.dah_status_string(99).decode() == "unknown status"


def _plan(B, L, n=0, cus=256):
    lib = _lib()
    p = native.DecodePlan()
    st = lib.dah_plan_decode(B, L, n, cus, ctypes.byref(p))
    return st, p


SHAPES = [(1, 1), (2, 12), (32, 4096), (256, 2048), (4, 40960), (128, 16384), (256, 40960),
          (1, 17), (7, 999), (4096, 64), (5000, 2048)]


@pytest.mark.parametrize("B,L", SHAPES)
@pytest.mark.parametrize("n", [0, 1, 2, 3, 7, 16, 1000])
def test_planner_is_consistent(B, L, n):
    st, p = _plan(B, L, n)
    assert st == 0
    pages = -(-L // 16)
    mode = native.PLAN_MODES[p.mode]
    slot_bytes = 16 * 130 * 4
    if mode == "per_sequence":
        assert p.splits == 1 and p.workgroups == B and p.workspace_bytes == 0
        assert p.pages_per_split == pages
    elif mode == "split":
        assert p.splits >= 2 and p.pages_per_split >= 1
        assert p.splits * p.pages_per_split >= pages          # every page is covered
        assert (p.splits - 1) * p.pages_per_split < pages     # the last split is not empty
        assert p.workgroups == B * (-(-p.splits // 8) * 8)   # padded for the XCD mapping
        assert p.workspace_bytes == B * p.splits * slot_bytes
    else:
        assert mode == "balanced" and n == 0 and 64 <= B <= 4096
        assert p.workgroups == 256
        # partial slots, then B + 1 int32 page prefix sums for the merge
        assert p.workspace_bytes == (B + p.workgroups - 1) * slot_bytes + (B + 1) * 4
    if n == 1:
        assert mode == "per_sequence"
    if n > 1:
        assert p.splits <= n and mode in ("split", "per_sequence")
    assert _lib().dah_workspace_bytes_for(B, L, n, 256) == p.workspace_bytes


def test_planner_choices_for_the_measured_shapes():
    # B=256, S=2048: one workgroup per sequence fills 256 compute units
    st, p = _plan(256, 2048)
    assert native.PLAN_MODES[p.mode] == "per_sequence"
    # 64+ sequences that do not fill the device or run long: balanced
    for B, L in [(128, 14464), (64, 100), (255, 2048), (256, 2064), (4096, 40960)]:
        st, p = _plan(B, L)
        assert native.PLAN_MODES[p.mode] == "balanced", (B, L)
    # fewer sequences: fixed splits spread over the XCDs (measured best at
    # B=32 up to 4096 positions: 8 splits; B=4 up to 40,960: 64 splits)
    assert (native.PLAN_MODES[_plan(32, 4096)[1].mode], _plan(32, 4096)[1].splits) == ("split", 8)
    assert (native.PLAN_MODES[_plan(4, 40960)[1].mode], _plan(4, 40960)[1].splits) == ("split", 64)
    assert native.PLAN_MODES[_plan(2, 12)[1].mode] == "per_sequence"
    # beyond the balanced scan's 4096 sequences: fixed splits
    st, p = _plan(5000, 4096)
    assert native.PLAN_MODES[p.mode] == "split"


@pytest.mark.parametrize("args,status", [
    ((0, 10, 0, 256), 2), ((1, 0, 0, 256), 2), ((1, 10, -1, 256), 2), ((1, 10, 0, 0), 2),
])
def test_planner_rejects_bad_arguments(args, status):
    lib = _lib()
    p = native.DecodePlan()
    assert lib.dah_plan_decode(*args, ctypes.byref(p)) == status
    assert lib.dah_last_error().decode() != ""
    assert lib.dah_plan_decode(1, 10, 0, 256, None) == 1


# Fake, aligned addresses: every call below must fail validation before any
# pointer is used, so nothing is dereferenced.
A = 0x100000


def _decode(**kw):
    lib = _lib()
    a = dict(q=A, k=A, v=A, dt=1, num_pages=16, bt=A, mpps=4, sl=A, B=2, max_len=64, ns=0, o=A,
             ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return lib.paged_decode_gqa(a["q"], a["k"], a["v"], a["dt"], a["num_pages"], a["bt"], a["mpps"],
                                a["sl"], a["B"], a["max_len"], a["ns"], a["o"], a["ws"],
                                a["ws_bytes"], a["stream"])


def _append(**kw):
    lib = _lib()
    a = dict(q=A, kn=A, vn=A, qg=A, kg=A, eps=1e-6, theta=1e6, k=A, v=A, dt=1, num_pages=16,
             bt=A, mpps=4, sl=A, B=2, qo=A, stream=None)
    a.update(kw)
    return lib.qk_norm_rope_append(a["q"], a["kn"], a["vn"], a["qg"], a["kg"], a["eps"], a["theta"],
                                   a["k"], a["v"], a["dt"], a["num_pages"], a["bt"], a["mpps"],
                                   a["sl"], a["B"], a["qo"], a["stream"])


def _step(**kw):
    lib = _lib()
    a = dict(q=A, kn=A, vn=A, qg=A, kg=A, eps=1e-6, theta=1e6, k=A, v=A, dt=1, num_pages=16,
             bt=A, mpps=4, sl=A, B=2, max_len=64, ns=0, qo=A, o=A, ws=None, ws_bytes=0,
             stream=None)
    a.update(kw)
    return lib.decode_attn_step(a["q"], a["kn"], a["vn"], a["qg"], a["kg"], a["eps"], a["theta"],
                                a["k"], a["v"], a["dt"], a["num_pages"], a["bt"], a["mpps"],
                                a["sl"], a["B"], a["max_len"], a["ns"], a["qo"], a["o"], a["ws"],
                                a["ws_bytes"], a["stream"])


BAD_DECODE = [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(bt=None), 1),
    (dict(sl=None), 1), (dict(o=None), 1),
    (dict(dt=2), 3), (dict(dt=-1), 3),
    (dict(B=0), 2), (dict(B=-5), 2), (dict(num_pages=0), 2), (dict(num_pages=2 ** 31), 2),
    (dict(mpps=0), 2), (dict(max_len=0), 2), (dict(max_len=65), 2), (dict(ns=-1), 2),
    (dict(q=A + 4), 4), (dict(o=A + 8), 4), (dict(k=A + 2), 4), (dict(bt=A + 2), 4),
]


@pytest.mark.parametrize("kw,status", BAD_DECODE)
def test_paged_decode_rejects(kw, status):
    assert _decode(**kw) == status
    assert _lib().dah_last_error().decode() != ""


BAD_APPEND = [
    (dict(q=None), 1), (dict(kn=None), 1), (dict(vn=None), 1), (dict(qg=None), 1),
    (dict(kg=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(bt=None), 1),
    (dict(sl=None), 1), (dict(qo=None), 1),
    (dict(dt=7), 3), (dict(B=0), 2), (dict(num_pages=0), 2), (dict(mpps=0), 2),
    (dict(eps=-1.0), 2), (dict(theta=0.0), 2), (dict(eps=float("nan")), 2),
    (dict(q=A + 4), 4), (dict(qo=A + 4), 4), (dict(kn=A + 8), 4), (dict(v=A + 2), 4),
    (dict(sl=A + 1), 4),
]


@pytest.mark.parametrize("kw,status", BAD_APPEND)
def test_append_rejects(kw, status):
    assert _append(**kw) == status


# decode_attn_step accepts a NULL q_out (o only); its other checks still apply
BAD_STEP = [case for case in BAD_APPEND if case[0] != dict(qo=None)] + [
    (dict(max_len=65), 2), (dict(o=None), 1), (dict(ns=-2), 2), (dict(max_len=0), 2),
    (dict(qo=None, q=A + 4), 4), (dict(qo=None, o=None), 1), (dict(qo=None, max_len=65), 2),
    (dict(qo=None, kn=None), 1), (dict(qo=None, dt=5), 3)]


@pytest.mark.parametrize("kw,status", BAD_STEP)
def test_step_rejects(kw, status):
    assert _step(**kw) == status


def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


@pytest.mark.skipif(_gpu_visible(), reason="valid arguments would launch on a real GPU")
def test_valid_arguments_without_gpu_report_hip_error():
    # With no GPU the call passes validation and fails on the device query.
    assert _decode() == 6
    assert "hip" in _lib().dah_last_error().decode().lower() or _lib().dah_last_error()
    assert _lib().dah_workspace_bytes(2, 64, 0) == 0


def test_probe_wrappers_refuse_host_tensors():
    torch = pytest.importorskip("torch")
    from decode_attention_head_amd.probes import probe_copy, probe_read
    a = torch.zeros(64, dtype=torch.uint8)
    with pytest.raises(ValueError):
        probe_copy(a, a.clone())
    with pytest.raises(ValueError):
        probe_read(a, torch.zeros(4, dtype=torch.int32), 1)


# The family's other head counts (nnterp qwen3 page, "Grouped-query attention,
# with 128-wide heads on every size"): 32, 40 and 64 query heads over 8 KV heads.
FAMILY_HEADS = [16, 32, 40, 64]


@pytest.mark.parametrize("H", FAMILY_HEADS)
@pytest.mark.parametrize("dt", [0, 1])
@pytest.mark.parametrize("B,L,n", [(256, 2048, 0), (32, 4096, 0), (4, 40960, 0), (128, 16384, 0),
                                   (7, 999, 3), (48, 3000, 0), (63, 5000, 0)])
def test_planner_ex_scales_the_workspace_with_heads(H, dt, B, L, n):
    lib = _lib()
    p16, ph = native.DecodePlan(), native.DecodePlan()
    assert lib.dah_plan_decode(B, L, n, 256, ctypes.byref(p16)) == 0
    assert lib.dah_plan_decode_ex(B, H, dt, L, n, 256, ctypes.byref(ph)) == 0
    mfma = dt == 1 and H >= 32
    if mfma and n == 0 and 32 <= B < 64:
        # the matrix-core kernel takes the balanced plan from 32 sequences
        assert native.PLAN_MODES[ph.mode] == "balanced"
        assert native.PLAN_MODES[p16.mode] == "split"
        assert ph.workspace_bytes == (B + ph.workgroups - 1) * H * 130 * 4 + (B + 1) * 4
        return
    # otherwise the cut of the positions does not depend on the head count,
    # and the partial slots scale with it (the balanced plan's prefix sums do not)
    assert (ph.mode, ph.splits, ph.pages_per_split, ph.workgroups) == \
        (p16.mode, p16.splits, p16.pages_per_split, p16.workgroups)
    prefix = (B + 1) * 4 if native.PLAN_MODES[ph.mode] == "balanced" else 0
    assert (ph.workspace_bytes - prefix) * 16 == (p16.workspace_bytes - prefix) * H


@pytest.mark.parametrize("H", [0, 8, 15, 24, 48, 65, -16])
def test_ex_calls_reject_other_head_counts(H):
    lib = _lib()
    p = native.DecodePlan()
    assert lib.dah_plan_decode_ex(2, H, 1, 64, 0, 256, ctypes.byref(p)) == 2
    assert "num_heads" in lib.dah_last_error().decode()
    assert lib.paged_decode_gqa_ex(A, A, A, 1, 16, A, 4, A, 2, H, 64, 0, A, None, 0, None) == 2
    assert lib.qk_norm_rope_append_ex(A, A, A, A, A, 1e-6, 1e6, A, A, 1, 16, A, 4, A, 2, H, A,
                                      None) == 2
    assert lib.decode_attn_step_ex(A, A, A, A, A, 1e-6, 1e6, A, A, 1, 16, A, 4, A, 2, H, 64, 0, A,
                                   A, None, 0, None) == 2


@pytest.mark.parametrize("H", FAMILY_HEADS)
def test_ex_calls_validate_like_the_base_calls(H):
    lib = _lib()
    # a NULL pointer, a bad dtype, a misaligned pointer, a too-long max_seq_len
    assert lib.paged_decode_gqa_ex(None, A, A, 1, 16, A, 4, A, 2, H, 64, 0, A, None, 0, None) == 1
    assert lib.paged_decode_gqa_ex(A, A, A, 5, 16, A, 4, A, 2, H, 64, 0, A, None, 0, None) == 3
    assert lib.paged_decode_gqa_ex(A, A, A, 1, 16, A, 4, A, 2, H, 64, 0, A + 4, None, 0, None) == 4
    assert lib.paged_decode_gqa_ex(A, A, A, 1, 16, A, 4, A, 2, H, 65, 0, A, None, 0, None) == 2
    assert lib.qk_norm_rope_append_ex(A, A, A, A, A, -1.0, 1e6, A, A, 1, 16, A, 4, A, 2, H, A,
                                      None) == 2
    assert lib.decode_attn_step_ex(A, A, A, A, A, 1e-6, 1e6, A, A, 1, 16, A, 4, A, 2, H, 64, 0,
                                   A, None, None, 0, None) == 1


def test_planner_ex_rejects_unknown_dtype():
    lib = _lib()
    p = native.DecodePlan()
    assert lib.dah_plan_decode_ex(8, 32, 2, 64, 0, 256, ctypes.byref(p)) == 3
    assert lib.dah_plan_decode_ex(8, 32, 1, 64, 0, 256, None) == 1
    assert lib.dah_workspace_bytes_ex(8, 32, 7, 64, 0) == 0


@pytest.mark.parametrize("B,L,n", [(256, 2048, 0), (32, 4096, 0), (4, 40960, 0), (128, 16384, 0),
                                   (2, 12, 0), (7, 999, 3), (64, 100, 1)])
@pytest.mark.parametrize("H", FAMILY_HEADS)
def test_planner_kernel_choice(B, L, n, H):
    """bfloat16: matrix cores for 4+ query heads per KV head, and for 2 unless
    the plan is fixed splits; float32: always the VALU kernel."""
    lib = _lib()
    p = native.DecodePlan()
    assert lib.dah_plan_decode_ex(B, H, 1, L, n, 256, ctypes.byref(p)) == 0
    mode = native.PLAN_MODES[p.mode]
    assert p.kernel == (1 if (H >= 32 or mode != "split") else 0), (mode, p.kernel)
    assert lib.dah_plan_decode_ex(B, H, 0, L, n, 256, ctypes.byref(p)) == 0
    assert p.kernel == 0
    if H == 16:
        q = native.DecodePlan()
        assert lib.dah_plan_decode(B, L, n, 256, ctypes.byref(q)) == 0
        r = native.DecodePlan()
        assert lib.dah_plan_decode_ex(B, 16, 1, L, n, 256, ctypes.byref(r)) == 0
        assert (q.mode, q.splits, q.workgroups, q.workspace_bytes, q.kernel) == \
            (r.mode, r.splits, r.workgroups, r.workspace_bytes, r.kernel)


@pytest.mark.parametrize("args,status", [
    ((None, A, 4, 64, 256, A), 1), ((A, None, 4, 64, 256, A), 1), ((A, A, 4, 64, 256, None), 1),
    ((A, A, 0, 64, 256, A), 2), ((A, A, 4, 96, 256, A), 2), ((A, A, 4, 0, 256, A), 2),
    ((A, A, 4, 64, 128, A), 2), ((A, A, 4, 64, 300, A), 2),
    ((A + 4, A, 4, 64, 256, A), 4), ((A, A + 2, 4, 64, 256, A), 4), ((A, A, 4, 64, 256, A + 8), 4),
])
def test_linear_rejects(args, status):
    lib = _lib()
    assert lib.dah_linear(*args, None) == status
    assert lib.dah_last_error().decode() != ""


def test_projection_entry_points_reject():
    lib = _lib()
    # heads outside the family, a NULL output, misaligned k, bad hidden
    assert lib.attn_qkv_proj(A, A, 4, 1024, 24, A, A, A, None) == 2
    assert lib.attn_qkv_proj(A, A, 4, 1024, 16, A, None, A, None) == 1
    assert lib.attn_qkv_proj(A, A, 4, 1024, 16, A, A + 4, A, None) == 4
    assert lib.attn_qkv_proj(A, A, 4, 1000, 16, A, A, A, None) == 2
    assert lib.attn_o_proj(A, A, 4, 48, 1024, A, None) == 2
    assert lib.attn_o_proj(A, A, 4, 16, 1000, A, None) == 2


def test_linear_kernel_choice():
    """The tile rule of dah_linear (host only): decode's few rows take the
    split-k kernel, the measured projection shapes at B = 256 the tiles the
    sweep found fastest, invalid shapes -1; and the GPU parity cases of
    dah_linear reach every kernel."""
    lib = _lib()
    assert lib.dah_linear_kernel(1, 4096, 1024) == 0
    assert lib.dah_linear_kernel(16, 6144, 1024) == 0
    assert lib.dah_linear_kernel(48, 1024, 2048) == 0          # few tiles: split-k
    assert lib.dah_linear_kernel(256, 4096, 1024) == 3         # qkv at 16 heads
    assert lib.dah_linear_kernel(256, 1024, 2048) == 5         # o_proj
    assert lib.dah_linear_kernel(256, 6144, 1024) == 3         # gate_up
    assert lib.dah_linear_kernel(256, 1024, 3072) == 5         # down
    assert lib.dah_linear_kernel(256, 10240, 1024) == 2        # qkv at 64 heads
    assert lib.dah_linear_kernel(4096, 4096, 1024) == 1        # prefill-sized
    assert lib.dah_linear_kernel(1000, 192, 256) == 4          # N not a multiple of 128
    for bad in ((0, 64, 256), (4, 96, 256), (4, 64, 128), (4, 0, 256)):
        assert lib.dah_linear_kernel(*bad) == -1
    import test_gpu_projections as tp
    reached = {lib.dah_linear_kernel(T, N, K) for T in tp.LINEAR_T for N, K in tp.LINEAR_NK}
    assert reached == {0, 1, 2, 3, 4, 5}


MIB8 = 8 << 20   # dah_linear_ws's workspace for T = 256, N = 1024, K = 8192 (8 slices)


@pytest.mark.parametrize("args,status", [
    ((None, A, None, 256, 1024, 8192, A, A, MIB8), 1),
    ((A, A, None, 256, 1000, 8192, A, A, MIB8), 2),
    ((A, A, None, 256, 1024, 8000, A, A, MIB8), 2),
    ((A, A, A + 4, 256, 1024, 8192, A, A, MIB8), 4),
    ((A, A, None, 256, 1024, 8192, A + 8, A, MIB8), 4),
    ((A, A, None, 256, 1024, 8192, A, None, 0), 5),
    ((A, A, None, 256, 1024, 8192, A, A, MIB8 - 1), 5),
    ((A, A, None, 256, 1024, 8192, A, A + 16, MIB8), 4),
])
def test_linear_ws_rejects(args, status):
    lib = _lib()
    assert lib.dah_linear_ws(*args, None) == status
    assert lib.dah_last_error().decode() != ""
    assert lib.attn_o_proj_ws(A, A, 4, 48, 1024, A, A, MIB8, None) == 2


def _ws_plan(lib, T, N, K):
    ks = ctypes.c_int(0)
    kernel = lib.dah_linear_ws_kernel(T, N, K, ctypes.byref(ks))
    return kernel, ks.value


def test_linear_ws_plan():
    """The k-split rule of dah_linear_ws (host only): the measured o_proj and
    down shapes take the tiles and slice counts the sweep found fastest; short
    k, or enough tiles without slices, keep dah_linear's choice unsplit; the
    workspace is slices x T x N floats; and the GPU parity cases reach every
    tile shape over 8 slices and some over 4."""
    lib = _lib()
    want = {(512, 1024, 8192): (1, 8), (256, 1024, 8192): (2, 8), (128, 1024, 8192): (3, 8),
            (64, 1024, 8192): (4, 8), (16, 1024, 8192): (5, 8), (16, 1024, 3072): (4, 8),
            (256, 1024, 3072): (2, 8), (256, 1024, 2048): (3, 4), (128, 1024, 2048): (4, 4),
            (1, 1024, 2048): (4, 8)}
    for (T, N, K), plan in want.items():
        assert _ws_plan(lib, T, N, K) == plan, (T, N, K)
        assert lib.dah_linear_workspace_bytes(T, N, K) == plan[1] * T * N * 4
    for T, N, K in ((1, 4096, 1024), (256, 4096, 1024), (256, 10240, 1024), (4096, 4096, 1024),
                    (4096, 1024, 2048), (1000, 192, 256)):
        assert _ws_plan(lib, T, N, K) == (lib.dah_linear_kernel(T, N, K), 1), (T, N, K)
        assert lib.dah_linear_workspace_bytes(T, N, K) == 0
    for bad in ((0, 64, 256), (4, 96, 2048), (4, 64, 2000)):
        assert _ws_plan(lib, *bad)[0] == -1
        assert lib.dah_linear_workspace_bytes(*bad) == 0
    import test_gpu_projections as tp
    reached = {_ws_plan(lib, *c) for c in tp.LINEAR_WS_CASES}
    assert {k for k, s in reached if s == 8} == {1, 2, 3, 4, 5}
    assert {k for k, s in reached if s == 4} == {3, 4}


@pytest.mark.parametrize("B,H,L", [(256, 16, 2048), (256, 64, 2048), (32, 16, 16384),
                                   (4, 40, 40960)])
def test_layer_workspace_shares_one_region(B, H, L):
    """dah_layer_workspace_bytes: the intermediates q, k, v, q_out, o, x1 and
    the activation (each rounded up to 256 bytes; gate_up's output is never
    stored, the activation is applied in its product), then one region as
    large as the larger of the attention's workspace and the k-slice partials
    of o_proj and down."""
    lib = _lib()
    hidden, inter = 1024, 3072
    r = lambda n: (n + 255) // 256 * 256   # noqa: E731
    f = 4
    inter_bytes = sum(r(n) for n in (B * H * 128 * f, B * 8 * 128 * f, B * 8 * 128 * f,
                                     B * H * 128 * f, B * H * 128 * f, B * hidden * f,
                                     B * inter * f))
    attn = lib.dah_workspace_bytes_ex(B, H, 1, L, 0)
    split = max(lib.dah_linear_workspace_bytes(B, hidden, H * 128),
                lib.dah_linear_workspace_bytes(B, hidden, inter))
    assert split > 0
    assert lib.dah_layer_workspace_bytes(B, hidden, inter, H, 1, L, 0) == \
        inter_bytes + r(max(attn, split))


def _noalloc(**kw):
    lib = _lib()
    a = dict(q=A, kn=A, vn=A, qg=A, kg=A, eps=1e-6, theta=1e6, k=A, v=A, dt=1, num_pages=16,
             bt=A, mpps=4, sl=A, B=2, H=16, max_len=64, ns=0, qo=A, o=A, stream=None)
    a.update(kw)
    return lib.decode_attn_step_noalloc(a["q"], a["kn"], a["vn"], a["qg"], a["kg"], a["eps"],
                                        a["theta"], a["k"], a["v"], a["dt"], a["num_pages"],
                                        a["bt"], a["mpps"], a["sl"], a["B"], a["H"],
                                        a["max_len"], a["ns"], a["qo"], a["o"], a["stream"])


@pytest.mark.parametrize("kw,status", BAD_STEP + [(dict(H=24), 2), (dict(H=0), 2)])
def test_noalloc_step_rejects(kw, status):
    """The allocation-free step validates exactly like decode_attn_step
    before it looks at the device or its scratch."""
    assert _noalloc(**kw) == status
    assert _lib().dah_last_error().decode() != ""


@pytest.mark.skipif(_gpu_visible(), reason="valid arguments would launch on a real GPU")
def test_noalloc_without_gpu_reports_hip_error():
    assert _noalloc() == 6


def test_scratch_size_constant():
    text = open(HEADER).read()
    m = re.search(r"#define DAH_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    import decode_attention_head_amd as dah
    assert m and int(m.group(1)) << int(m.group(2)) == dah.SCRATCH_BYTES == 16 << 20
