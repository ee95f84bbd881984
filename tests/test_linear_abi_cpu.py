"""Host-side validation of linear_logp_partials(_ex) (no GPU: every case fails before any HIP
call) and the constants the binding shares with include/linear_logp.h."""

from __future__ import annotations

import ctypes
import os
import re

import pytest

from deterministic_selected_token_amd import linear

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, NULL, SHAPE, SHARD, ARG = 0, 1, 2, 3, 8
A = ctypes.c_void_p(0x10000)  # 16-byte aligned, never dereferenced
U = ctypes.c_void_p(0x10002)  # misaligned
lib = linear._lib


def call(**over):
    a = dict(h=A, ld_h=64, n=10, H=64, w=A, ld_w=64, vr=5000, vp=5000, c0=0, c1=5000, y=A,
             act=None, ign=-100, p=A, ldp=2)
    a.update(over)
    return lib.linear_logp_partials(a["h"], a["ld_h"], a["n"], a["H"], a["w"], a["ld_w"],
                                    a["vr"], a["vp"], a["c0"], a["c1"], a["y"], a["act"],
                                    a["ign"], a["p"], a["ldp"], None)


def call_ex(inv_t, **over):
    a = dict(h=A, ld_h=64, n=10, H=64, w=A, ld_w=64, vr=5000, vp=5000, c0=0, c1=5000, y=A,
             act=None, ign=-100, p=A, ldp=2)
    a.update(over)
    return lib.linear_logp_partials_ex(inv_t, a["h"], a["ld_h"], a["n"], a["H"], a["w"],
                                       a["ld_w"], a["vr"], a["vp"], a["c0"], a["c1"], a["y"],
                                       a["act"], a["ign"], a["p"], a["ldp"], None)


@pytest.mark.parametrize("inv_t", [0.0, -0.0, -1.0, float("inf"), float("-inf"), float("nan")])
def test_linear_partials_ex_rejects_bad_temperature(inv_t):
    assert call_ex(inv_t) == ARG
    assert call_ex(inv_t, n=0) == ARG  # checked before anything else


@pytest.mark.parametrize("over,want", [
    (dict(n=-1), SHAPE), (dict(c0=100), SHARD), (dict(n=0), OK), (dict(h=None), NULL),
    (dict(w=U), SHAPE), (dict(ldp=1), SHAPE)], ids=lambda v: str(v))
def test_linear_partials_ex_validates_like_the_plain_entry(over, want):
    assert call_ex(1.0 / 0.7, **over) == want == call(**over)


def call_bwd(inv_t=None, **over):
    a = dict(h=A, ld_h=64, n=10, H=64, w=A, ld_w=64, vr=5000, vp=5000, c0=0, c1=5000, y=A,
             act=None, ign=-100, g=A, st=A, dh=A, ld_dh=64, dw=A, ld_dw=64, ws=A,
             wsb=1 << 40, chunk=4096)
    a.update(over)
    args = (a["h"], a["ld_h"], a["n"], a["H"], a["w"], a["ld_w"], a["vr"], a["vp"], a["c0"],
            a["c1"], a["y"], a["act"], a["ign"], a["g"], a["st"], a["dh"], a["ld_dh"], a["dw"],
            a["ld_dw"], a["ws"], a["wsb"], a["chunk"], None)
    if inv_t is None:
        return lib.linear_logp_backward(*args)
    return lib.linear_logp_backward_ex(inv_t, *args)


W16 = ctypes.c_void_p(0x10010)  # 16-byte but not 256-byte aligned


@pytest.mark.parametrize("over,want", [
    (dict(n=-1), SHAPE), (dict(vr=0), SHAPE), (dict(c0=100), SHARD), (dict(c1=4097), SHARD),
    (dict(chunk=0), SHAPE), (dict(chunk=4000), SHAPE), (dict(chunk=2 ** 21), SHAPE),
    (dict(n=0), OK), (dict(n=2 ** 23 + 1), SHAPE),
    (dict(h=None), NULL), (dict(w=None), NULL), (dict(y=None), NULL), (dict(g=None), NULL),
    (dict(st=None), NULL), (dict(dh=None), NULL), (dict(dw=None), NULL), (dict(ws=None), NULL),
    (dict(H=60, ld_h=64, ld_w=64), SHAPE), (dict(ld_dh=32), SHAPE), (dict(ld_dw=32), SHAPE),
    (dict(h=U), SHAPE), (dict(w=U), SHAPE), (dict(ws=W16), SHAPE), (dict(wsb=1000), SHAPE),
], ids=lambda v: str(v))
def test_linear_backward_host_validation(over, want):
    assert call_bwd(**over) == want


@pytest.mark.parametrize("inv_t", [0.0, -1.0, float("inf"), float("nan")])
def test_linear_backward_rejects_bad_temperature(inv_t):
    assert call_bwd(inv_t) == ARG
    assert call_bwd(1.0 / 0.7, n=-1) == SHAPE


def test_linear_backward_workspace_size():
    ws = linear.linear_logp_backward_workspace
    # 2 bytes x (H_pad n_pad + H_pad chunk + 2 n_pad chunk), pads to 256
    assert ws(8192, 4096, 4096) == 2 * (4096 * 8192 + 4096 * 4096 + 2 * 8192 * 4096)
    assert ws(1, 8, 4096) == 2 * (256 * 256 + 256 * 4096 + 2 * 256 * 4096)
    assert ws(0, 8, 4096) == ws(1, 8, 4096)
    assert ws(-1, 8, 4096) == -1 and ws(10, 0, 4096) == -1 and ws(10, 8, 0) == -1
    assert ws(linear.BWD_MAX_ROWS + 1, 8, 4096) == -1
    assert ws(10, 8, linear.BWD_MAX_CHUNK + 1) == -1


DEVICE = 4


def test_weight_may_be_null_for_an_all_padding_view():
    """No real row in [col_begin, col_end): the weight pointer is not needed, so NULL passes
    the NULL check (and fails later only at the device check, this machine having no GPU)."""
    pad = dict(w=None, vr=4000, vp=8192, c0=4096, c1=8192)
    assert call(**pad) == DEVICE
    assert call(**dict(pad, c0=0)) == NULL  # real rows in range: weight required
    assert call_bwd(**pad) == DEVICE
    assert call_bwd(**dict(pad, c0=0)) == NULL
    assert call_bwd(**dict(pad, dw=None)) == NULL  # dweight is always required


def test_header_constant():
    text = open(os.path.join(ROOT, "include", "linear_logp.h")).read()
    assert int(re.search(r"#define LINEAR_LOGP_MAX_HIDDEN (\d+)", text).group(1)) == \
        linear.MAX_HIDDEN
    assert int(re.search(r"#define LINEAR_LOGP_MAX_LD (\d+)", text).group(1)) == linear.MAX_LD
    assert int(re.search(r"#define LINEAR_LOGP_BWD_MAX_ROWS (\d+)", text).group(1)) == \
        linear.BWD_MAX_ROWS
    assert int(re.search(r"#define LINEAR_LOGP_BWD_MAX_CHUNK (\d+)", text).group(1)) == \
        linear.BWD_MAX_CHUNK


@pytest.mark.parametrize("over,want", [
    (dict(n=-1), SHAPE), (dict(vr=0), SHAPE), (dict(vp=4000), SHAPE),
    (dict(c0=100), SHARD), (dict(c1=4097), SHARD), (dict(c1=6000), SHARD),
    (dict(n=0), OK), (dict(c0=4096, c1=4096), OK),
    (dict(h=None), NULL), (dict(w=None), NULL), (dict(y=None), NULL), (dict(p=None), NULL),
    (dict(H=0), SHAPE), (dict(H=60, ld_h=64, ld_w=64), SHAPE), (dict(H=65544, ld_h=65544,
                                                                     ld_w=65544), SHAPE),
    (dict(ld_h=60), SHAPE), (dict(ld_w=68), SHAPE), (dict(ld_h=72, H=72, ld_w=71), SHAPE),
    (dict(h=U), SHAPE), (dict(w=U), SHAPE), (dict(ldp=1), SHAPE),
    (dict(ld_h=262152), SHAPE), (dict(ld_w=262152), SHAPE),
], ids=lambda v: str(v))
def test_linear_partials_host_validation(over, want):
    assert call(**over) == want


def test_binding_rejects_cpu_and_wrong_dtype():
    import torch
    h = torch.zeros((2, 8), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        linear.linear_logp_forward(h, h, torch.zeros(2, dtype=torch.int64))
    with pytest.raises(TypeError):
        linear.linear_logp_forward(h.float(), h, torch.zeros(2, dtype=torch.int64))


def test_binding_rejects_partials_too_narrow_for_the_shard():
    import torch
    T = linear.TILE_COLS
    n, H = 2, 8
    h = torch.zeros((n, H), dtype=torch.bfloat16)
    w = torch.zeros((19 * T, H), dtype=torch.bfloat16)
    y = torch.zeros(n, dtype=torch.int64)
    with pytest.raises(ValueError, match="run past"):
        linear.linear_logp_partials(h, w, y, 39 * T, 39 * T, 20 * T, 39 * T,
                                    torch.zeros((n, 30, 3)))
    with pytest.raises(ValueError, match="GPU tensor"):
        linear.linear_logp_partials(h, w, y, 39 * T, 39 * T, 20 * T, 39 * T,
                                    torch.zeros((n, 39, 3)))


SCRATCH = 9


def call_noalloc(inv_t=1.0, **over):
    a = dict(h=A, ld_h=64, n=10, H=64, w=A, ld_w=64, vr=5000, vp=5000, c0=0, c1=5000, y=A,
             act=None, ign=-100, g=A, st=A, dh=A, ld_dh=64, dw=A, ld_dw=64, chunk=4096)
    a.update(over)
    return lib.linear_logp_backward_noalloc(
        inv_t, a["h"], a["ld_h"], a["n"], a["H"], a["w"], a["ld_w"], a["vr"], a["vp"], a["c0"],
        a["c1"], a["y"], a["act"], a["ign"], a["g"], a["st"], a["dh"], a["ld_dh"], a["dw"],
        a["ld_dw"], a["chunk"], None)


@pytest.mark.parametrize("over,want", [
    (dict(n=-1), SHAPE), (dict(c0=100), SHARD), (dict(chunk=4000), SHAPE), (dict(n=0), OK),
    (dict(h=None), NULL), (dict(dh=None), NULL), (dict(dw=None), NULL), (dict(h=U), SHAPE),
], ids=lambda v: str(v))
def test_noalloc_backward_validates_like_the_workspace_entry(over, want):
    assert call_noalloc(**over) == want == call_bwd(1.0, **over)
    assert call_noalloc(0.0, **over) == ARG


def test_noalloc_backward_rejects_work_beyond_its_scratch_array():
    """The static scratch array holds LINEAR_LOGP_NOALLOC_SCRATCH_BYTES; a call whose
    workspace would be larger is refused on the host, before any device check."""
    text = open(os.path.join(ROOT, "include", "linear_logp.h")).read()
    m = re.search(r"#define LINEAR_LOGP_NOALLOC_SCRATCH_BYTES \((\d+)ll << (\d+)\)", text)
    assert int(m.group(1)) << int(m.group(2)) == linear.NOALLOC_SCRATCH_BYTES
    ws = linear.linear_logp_backward_workspace
    assert ws(4096, 4096, 4096) == linear.NOALLOC_SCRATCH_BYTES  # the largest that fits
    big = dict(n=4096, H=4096, ld_h=4096, ld_w=4096, ld_dh=4096, ld_dw=4096)
    assert call_noalloc(**big, chunk=8192) == SCRATCH
    assert call_noalloc(**dict(big, n=4097)) == SCRATCH
    assert call_noalloc(**dict(big, n=8192), chunk=16384) == SCRATCH
    # the workspace entry point takes the same sizes when its workspace is large enough
    # (then fails here only at the device check of the fake pointers)
    assert call_bwd(**big, chunk=8192) == DEVICE
    assert "static scratch" in linear._lib.logp_status_string(SCRATCH).decode()


def call_bwd16(inv_t=1.0, **over):
    a = dict(h=A, ld_h=64, n=10, H=64, w=A, ld_w=64, vr=5000, vp=5000, c0=0, c1=5000, y=A,
             act=None, ign=-100, g=A, st=A, dh=A, ld_dh=64, dw=A, ld_dw=64, ws=A,
             wsb=1 << 40, chunk=4096)
    a.update(over)
    return lib.linear_logp_backward_bf16(
        inv_t, a["h"], a["ld_h"], a["n"], a["H"], a["w"], a["ld_w"], a["vr"], a["vp"], a["c0"],
        a["c1"], a["y"], a["act"], a["ign"], a["g"], a["st"], a["dh"], a["ld_dh"], a["dw"],
        a["ld_dw"], a["ws"], a["wsb"], a["chunk"], None)


@pytest.mark.parametrize("over,want", [
    (dict(n=-1), SHAPE), (dict(vr=0), SHAPE), (dict(c0=100), SHARD), (dict(c1=4097), SHARD),
    (dict(chunk=4000), SHAPE), (dict(n=0), OK), (dict(n=2 ** 23 + 1), SHAPE),
    (dict(h=None), NULL), (dict(w=None), NULL), (dict(dh=None), NULL), (dict(dw=None), NULL),
    (dict(ws=None), NULL), (dict(ld_dh=32), SHAPE), (dict(ld_dw=32), SHAPE), (dict(h=U), SHAPE),
    (dict(ws=W16), SHAPE), (dict(wsb=1000), SHAPE),
], ids=lambda v: str(v))
def test_bf16_backward_validates_like_the_fp32_entry(over, want):
    assert call_bwd16(**over) == want == call_bwd(1.0, **over)
    assert call_bwd16(float("nan"), **over) == ARG


def test_bf16_backward_workspace_adds_the_fp32_dh_accumulator():
    import torch
    ws, ws16 = linear.linear_logp_backward_workspace, lib.linear_logp_backward_bf16_workspace
    for n, H, c in ((8192, 4096, 16384), (1, 8, 4096), (0, 8, 4096), (300, 200, 8192)):
        n_pad, h_pad = -(-max(n, 1) // 256) * 256, -(-H // 256) * 256
        assert ws16(n, H, c) == ws(n, H, c) + 4 * n_pad * h_pad
        assert linear.linear_logp_backward_workspace(n, H, c, torch.bfloat16) == ws16(n, H, c)
    assert ws16(-1, 8, 4096) == -1 and ws16(10, 0, 4096) == -1 and ws16(10, 8, 0) == -1
    # a workspace that holds the FP32 staging but not the accumulator is short for BF16
    fp32_only = ws(10, 64, 4096)
    assert call_bwd16(wsb=fp32_only) == SHAPE
    assert call_bwd16(wsb=ws16(10, 64, 4096)) == DEVICE  # then the fake pointers' device check
    assert call_bwd(wsb=fp32_only) == DEVICE
    with pytest.raises(ValueError, match="out_dtype"):
        linear.linear_logp_backward_workspace(10, 64, 4096, torch.float16)


def test_binding_bf16_output_arguments():
    import torch
    h = torch.zeros((2, 8), dtype=torch.bfloat16)
    y = torch.zeros(2, dtype=torch.int64)
    st = torch.zeros((2, 2))
    with pytest.raises(ValueError, match="out_dtype"):
        linear.linear_logp_backward(h, h, y, st[:, 0], st, out_dtype=torch.float16)
    with pytest.raises(ValueError, match="noalloc"):
        linear.linear_logp_backward(h, h, y, st[:, 0], st, noalloc=True,
                                    out_dtype=torch.bfloat16)


def call_ws(inv_t=1.0, ws=A, wsb=1 << 30, **over):
    a = dict(h=A, ld_h=64, n=10, H=64, w=A, ld_w=64, vr=5000, vp=5000, c0=0, c1=5000, y=A,
             act=None, ign=-100, p=A, ldp=2)
    a.update(over)
    return lib.linear_logp_partials_ws(inv_t, a["h"], a["ld_h"], a["n"], a["H"], a["w"],
                                       a["ld_w"], a["vr"], a["vp"], a["c0"], a["c1"], a["y"],
                                       a["act"], a["ign"], a["p"], a["ldp"], ws, wsb, None)


@pytest.mark.parametrize("over,want", [
    (dict(n=-1), SHAPE), (dict(c0=100), SHARD), (dict(n=0), OK), (dict(h=None), NULL),
    (dict(w=U), SHAPE), (dict(ldp=1), SHAPE), (dict(H=60, ld_h=64, ld_w=64), SHAPE),
], ids=lambda v: str(v))
def test_balanced_partials_validate_like_the_plain_entry(over, want):
    assert call_ws(**over) == want == call_ex(1.0, **over)
    assert call_ws(0.0, **over) == ARG


def test_balanced_partials_workspace_checks():
    # a workspace must be 256-byte aligned and its size non-negative; NULL means no split
    assert call_ws(ws=ctypes.c_void_p(0x10010)) == SHAPE
    assert call_ws(wsb=-1) == SHAPE
    assert call_ws(ws=None, wsb=0) == DEVICE  # then the fake pointers' device check
    assert call_ws() == DEVICE


def test_balanced_partials_workspace_size():
    """3072 bytes (a float2 and a float per row of a 256-row block) per row block and
    256-column sub-block holding real columns of the view."""
    q = linear.linear_logp_partials_workspace
    assert q(8192, 151936, 0, 151936) == 32 * 594 * 3072            # 593.5 sub-blocks, rounded up
    assert q(8192, 151936, 0, 152064) == q(8192, 151936, 0, 151936)   # padding adds nothing
    assert q(8192, 151936, 16384, 36864) == 32 * 80 * 3072            # 5 tiles of a view
    assert q(300, 8200, 0, 12288) == 2 * 33 * 3072                    # ragged rows and columns
    assert q(0, 100, 0, 4096) == q(1, 100, 0, 4096) == 3072
    assert q(10, 5000, 8192, 12288) == 0                              # an all-padding view
    assert q(-1, 10, 0, 10) == -1 and q(10, 0, 0, 10) == -1 and q(10, 10, 5, 4) == -1


def call_save(z=A, ld_z=5000, ws=None, wsb=0, inv_t=1.0, **over):
    a = dict(h=A, ld_h=64, n=10, H=64, w=A, ld_w=64, vr=5000, vp=5000, c0=0, c1=5000, y=A,
             act=None, ign=-100, p=A, ldp=2)
    a.update(over)
    return lib.linear_logp_partials_save(inv_t, a["h"], a["ld_h"], a["n"], a["H"], a["w"],
                                         a["ld_w"], a["vr"], a["vp"], a["c0"], a["c1"], a["y"],
                                         a["act"], a["ign"], a["p"], a["ldp"], z, ld_z, ws, wsb,
                                         None)


@pytest.mark.parametrize("over,want", [
    (dict(n=-1), SHAPE), (dict(c0=100), SHARD), (dict(h=None), NULL), (dict(w=U), SHAPE),
    (dict(ldp=1), SHAPE), (dict(n=0), OK)], ids=lambda v: str(v))
def test_saving_partials_validate_like_the_plain_entry(over, want):
    assert call_save(**over) == want == call(**over)


@pytest.mark.parametrize("kw,want", [
    (dict(z=None), NULL), (dict(ld_z=4999), SHAPE), (dict(ld_z=5002), SHAPE),
    (dict(z=ctypes.c_void_p(0x10008)), SHAPE), (dict(ld_z=(1 << 31) + 4), SHAPE),
    (dict(ld_z=1 << 31, n=1 << 10), SHAPE), (dict(inv_t=0.0), ARG)], ids=lambda v: str(v))
def test_saving_partials_check_the_logits_buffer(kw, want):
    """The kept logits: non-NULL, 16-byte aligned, a row stride of at least the view's width,
    a multiple of 4, at most LINEAR_LOGP_MAX_SAVED_LD and with n * ld_logits <= 2^40; all
    checked before any device query (a valid call fails only at the device check here)."""
    assert call_save(**kw) == want
    assert call_save() == DEVICE


def call_saved_bwd(z=A, ld_z=5000, dt=2, inv_t=1.0, **over):
    a = dict(h=A, ld_h=64, n=10, H=64, w=A, ld_w=64, vr=5000, vp=5000, c0=0, c1=5000, y=A,
             act=None, ign=-100, g=A, st=A, dh=A, ld_dh=64, dw=A, ld_dw=64, ws=A,
             wsb=1 << 40, chunk=4096)
    a.update(over)
    return lib.linear_logp_backward_saved(
        inv_t, z, ld_z, a["h"], a["ld_h"], a["n"], a["H"], a["w"], a["ld_w"], a["vr"], a["vp"],
        a["c0"], a["c1"], a["y"], a["act"], a["ign"], a["g"], a["st"], a["dh"], a["ld_dh"],
        a["dw"], a["ld_dw"], dt, a["ws"], a["wsb"], a["chunk"], None)


@pytest.mark.parametrize("over,want", [
    (dict(n=-1), SHAPE), (dict(c0=100), SHARD), (dict(chunk=4000), SHAPE), (dict(n=0), OK),
    (dict(h=None), NULL), (dict(dw=None), NULL), (dict(ws=W16), SHAPE), (dict(wsb=1000), SHAPE),
], ids=lambda v: str(v))
def test_saved_backward_validates_like_the_workspace_entry(over, want):
    assert call_saved_bwd(**over) == want == call_bwd(**over)
    assert call_saved_bwd(dt=0, **over) == want


@pytest.mark.parametrize("kw,want", [
    (dict(z=None), NULL), (dict(ld_z=4999), SHAPE), (dict(z=ctypes.c_void_p(0x10002)), SHAPE),
    (dict(ld_z=(1 << 31) + 1), SHAPE), (dict(dt=1), ARG), (dict(dt=7), ARG),
    (dict(inv_t=float("nan")), ARG)], ids=lambda v: str(v))
def test_saved_backward_checks_the_logits_and_dtype(kw, want):
    """The saved logits may be any 4-byte aligned rows (row stride >= the view's width, at
    most LINEAR_LOGP_MAX_SAVED_LD); out_dtype is FP32 or BF16."""
    assert call_saved_bwd(**kw) == want
    assert call_saved_bwd(ld_z=5001) == DEVICE  # any stride >= the width
    assert call_saved_bwd(dt=0) == DEVICE


def test_saved_ld_constant():
    text = open(os.path.join(ROOT, "include", "linear_logp.h")).read()
    assert int(re.search(r"#define LINEAR_LOGP_MAX_SAVED_LD (\d+)ll", text).group(1)) == \
        linear.MAX_SAVED_LD
