"""C-ABI checks that need no GPU: the library loads, exports every function that
include/*.h declares, and rejects bad arguments on the host before any HIP call."""

from __future__ import annotations

import ctypes
import os
import re
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "logp.h")
INCLUDE = os.path.join(ROOT, "include")
HEADERS = [os.path.join(INCLUDE, f) for f in sorted(os.listdir(INCLUDE)) if f.endswith(".h")]
PKG = os.path.join(ROOT, "deterministic_selected_token_amd")

import deterministic_selected_token_amd as dst  # noqa: E402
from deterministic_selected_token_amd import grpo, linear  # noqa: E402

OK, NULL, SHAPE, SHARD, ARG = 0, 1, 2, 3, 8
T = 4096
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every case below fails host checks


def declared_functions() -> list[str]:
    names = []
    for h in HEADERS:
        text = open(h).read()
        names += re.findall(r"^LOGP_API\s+[\w\s\*]+?\b((?:logp|grpo|linear)_\w+)\s*\(",
                            text, flags=re.M)
    return names


def test_every_declared_function_is_exported():
    names = declared_functions()
    assert sorted(names) == sorted(dst.EXPORTED + grpo.EXPORTED + linear.EXPORTED)
    lib = ctypes.CDLL(dst.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", dst.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+((?:logp|grpo|linear)_\w+)$", out, flags=re.M))
    assert exported == set(names)  # nothing else with the prefixes leaks out


C_CONSUMER = r"""
#include <stdio.h>
#include <string.h>
#include "logp.h"
#include "grpo_loss.h"
#include "linear_logp.h"

typedef void (*fn_t)(void);
/* every declared entry point, so that the link must resolve each one */
static const fn_t entry_points[] = {
%(table)s
};

int main(void) {
    const uint16_t* fake = (const uint16_t*)(uintptr_t)0x1000; /* never dereferenced */
    if (logp_num_tiles(151936) != 38 || logp_num_tiles(159744) != 39) return 1;
    if (strcmp(logp_status_string(LOGP_OK), "ok") != 0) return 2;
    /* host validation only: nothing is launched for these */
    if (logp_forward(fake, 151936, -1, 151936, 151936, (const int64_t*)fake, NULL, -100,
                     (float*)(uintptr_t)0x1000, NULL, NULL, NULL) != LOGP_ERR_SHAPE) return 3;
    if (logp_forward(fake, 151936, 0, 151936, 151936, NULL, NULL, -100, NULL, NULL, NULL,
                     NULL) != LOGP_OK) return 4;
    if (linear_logp_partials_workspace(8192, 151936, 0, 151936) != (int64_t)32 * 594 * 3072)
        return 5;
    printf("%%d entry points linked\n", (int)(sizeof entry_points / sizeof entry_points[0]));
    return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs gcc and the ROCm headers")
def test_headers_compile_and_link_as_c99():
    """include/*.h are plain C: a C99 program (the HIP runtime's own headers taken as system
    headers, ours under -pedantic -Werror) that names every declared entry point links
    against the built library and runs its host-side calls."""
    names = declared_functions()
    table = "\n".join(f"    (fn_t){name}," for name in names)
    with tempfile.TemporaryDirectory() as tmp:
        src = os.path.join(tmp, "consumer.c")
        exe = os.path.join(tmp, "consumer")
        with open(src, "w") as f:
            f.write(C_CONSUMER % {"table": table})
        cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
               "-D__HIP_PLATFORM_AMD__", "-I", INCLUDE, "-isystem", "/opt/rocm/include", src,
               "-L", PKG, "-llogp_mi355x", f"-Wl,-rpath,{PKG}",
               "-Wl,-rpath-link,/opt/rocm/lib", "-o", exe]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
        assert r.returncode == 0, (r.returncode, r.stderr)
        assert r.stdout.strip() == f"{len(names)} entry points linked"


def test_header_constants_match_binding():
    text = open(HEADER).read()
    assert re.search(r"#define LOGP_TILE_COLS (\d+)", text).group(1) == str(dst.TILE_COLS)
    assert re.search(r"#define LOGP_FWD_MAX_TILES (\d+)", text).group(1) == \
        str(dst.FWD_MAX_TILES)
    for code, name in dst.STATUS.items():
        assert re.search(rf"{name}\s*=\s*{code}\b", text), name


def test_library_is_built_for_gfx950():
    # The offload bundle inside the shared object names its target.
    blob = open(dst.LIB_PATH, "rb").read()
    assert b"gfx950" in blob


def test_num_tiles_and_status_strings():
    assert dst.logp_num_tiles(151936) == 38
    assert dst.logp_num_tiles(152064) == 38
    assert dst.logp_num_tiles(159744) == 39
    assert dst.logp_num_tiles(4096) == 1 and dst.logp_num_tiles(4097) == 2
    assert dst.logp_num_tiles(1) == 1 and dst.logp_num_tiles(0) == 0
    for code in range(10):
        s = dst.logp_status_string(code)
        assert s and (code == 0) == (s == "ok")
    assert dst.logp_status_string(99) == "unknown status"


def fwd(**kw):
    a = dict(logits=FAKE, ld=152064, n=4, vocab_real=151936, vocab_padded=152064,
             targets=FAKE, active=None, ignore_index=-100, logp=FAKE, lse=None, stats=None,
             stream=None)
    a.update(kw)
    return dst.library().logp_forward(*a.values())


def bwd(**kw):
    a = dict(logits=FAKE, ld=151936, n=4, vocab_real=151936, vocab_padded=151936, col_begin=0,
             col_end=151936, targets=FAKE, active=None, ignore_index=-100, grad=FAKE,
             stats=FAKE, dlogits=FAKE, ld_out=151936, stream=None)
    a.update(kw)
    return dst.library().logp_backward(*a.values())


def part(**kw):
    a = dict(logits=FAKE, ld=159744, n=4, vocab_real=151936, vocab_padded=159744, col_begin=0,
             col_end=159744, targets=FAKE, active=None, ignore_index=-100, partials=FAKE,
             ldp=39, stream=None)
    a.update(kw)
    return dst.library().logp_partials(*a.values())


def merge(**kw):
    a = dict(partials=FAKE, ldp=39, n=4, num_tiles=39, vocab_real=151936, targets=FAKE,
             active=None, ignore_index=-100, logp=FAKE, lse=None, stats=None, stream=None)
    a.update(kw)
    return dst.library().logp_merge(*a.values())


@pytest.mark.parametrize("kw,want", [
    (dict(n=-1), SHAPE), (dict(vocab_real=0), SHAPE), (dict(vocab_padded=100), SHAPE),
    (dict(ld=152000), SHAPE), (dict(vocab_padded=2 ** 31 - T, ld=2 ** 31), SHAPE),
    (dict(vocab_real=T * 4096 + 1, vocab_padded=T * 4096 + 1, ld=T * 4097), SHAPE),
    (dict(n=2 ** 31), SHAPE),
    (dict(n=0), OK), (dict(n=0, logits=None, targets=None, logp=None), OK),
    (dict(logits=None), NULL), (dict(targets=None), NULL), (dict(logp=None), NULL),
])
def test_forward_host_validation(kw, want):
    assert fwd(**kw) == want


@pytest.mark.parametrize("kw,want", [
    (dict(n=-1), SHAPE), (dict(vocab_real=0), SHAPE), (dict(col_begin=-1), SHARD),
    (dict(col_end=151937), SHARD), (dict(col_begin=100, col_end=99), SHARD),
    (dict(ld=1000), SHAPE), (dict(ld_out=1000), SHAPE),
    (dict(n=0), OK), (dict(col_begin=500, col_end=500), OK),
    (dict(logits=None), NULL), (dict(stats=None), NULL), (dict(grad=None), NULL),
    (dict(dlogits=None), NULL), (dict(targets=None), NULL),
    # the backward accepts any sub-range, aligned or not: these fail later, not as SHARD
    (dict(col_begin=3, col_end=1000, logits=None), NULL),
])
def test_backward_host_validation(kw, want):
    assert bwd(**kw) == want


@pytest.mark.parametrize("kw,want", [
    (dict(col_begin=100), SHARD), (dict(col_begin=T, col_end=T + 100), SHARD),
    (dict(col_begin=T, col_end=T), SHARD), (dict(col_end=159745), SHARD),
    (dict(col_begin=-T), SHARD), (dict(ldp=38), SHAPE), (dict(ld=100), SHAPE),
    (dict(vocab_padded=151935), SHAPE), (dict(n=0), OK),
    (dict(partials=None), NULL), (dict(targets=None), NULL),
    # valid shard bounds (interior multiples of T; the last may end at vocab_padded):
    # with a NULL logits pointer they stop at the NULL check, after the shard check
    (dict(col_begin=T * 38, col_end=159744, logits=None), NULL),
    (dict(col_begin=T * 13, col_end=T * 26, logits=None), NULL),
    (dict(vocab_padded=159000, col_begin=T * 38, col_end=159000, ld=159000, logits=None),
     NULL),
])
def test_partials_host_validation(kw, want):
    assert part(**kw) == want


@pytest.mark.parametrize("kw,want", [
    (dict(num_tiles=37), SHAPE), (dict(ldp=38), SHAPE), (dict(n=-2), SHAPE),
    (dict(vocab_real=0), SHAPE), (dict(n=0), OK), (dict(partials=None), NULL),
    (dict(logp=None), NULL),
])
def test_merge_host_validation(kw, want):
    assert merge(**kw) == want


@pytest.mark.parametrize("dtype,inv_t", [(3, 1.0), (-1, 1.0), (0, 0.0), (1, -2.0),
                                         (2, float("nan")), (0, float("inf"))])
def test_ex_entry_points_reject_bad_dtype_or_temperature(dtype, inv_t):
    lib = dst.library()
    fa = dict(logits=FAKE, ld=152064, n=4, vocab_real=151936, vocab_padded=152064,
              targets=FAKE, active=None, ignore_index=-100, logp=FAKE, lse=None, stats=None,
              stream=None)
    assert lib.logp_forward_ex(dtype, inv_t, *fa.values()) == ARG
    ba = dict(logits=FAKE, ld=151936, n=4, vocab_real=151936, vocab_padded=151936,
              col_begin=0, col_end=151936, targets=FAKE, active=None, ignore_index=-100,
              grad=FAKE, stats=FAKE, dlogits=FAKE, ld_out=151936, stream=None)
    assert lib.logp_backward_ex(dtype, inv_t, *ba.values()) == ARG
    pa = dict(logits=FAKE, ld=159744, n=4, vocab_real=151936, vocab_padded=159744,
              col_begin=0, col_end=159744, targets=FAKE, active=None, ignore_index=-100,
              partials=FAKE, ldp=39, stream=None)
    assert lib.logp_partials_ex(dtype, inv_t, *pa.values()) == ARG


def test_ex_entry_points_validate_like_the_plain_ones():
    lib = dst.library()
    for dtype in (0, 1, 2):
        assert lib.logp_forward_ex(dtype, 0.7, FAKE, 152064, -1, 151936, 152064, FAKE, None,
                                   -100, FAKE, None, None, None) == SHAPE
        assert lib.logp_forward_ex(dtype, 0.7, None, 152064, 0, 151936, 152064, None, None,
                                   -100, None, None, None, None) == OK
        assert lib.logp_backward_ex(dtype, 1.5, FAKE, 100, 4, 100, 100, 50, 40, FAKE, None,
                                    -100, FAKE, FAKE, FAKE, 100, None) == SHARD
        assert lib.logp_partials_ex(dtype, 1.0, FAKE, 159744, 4, 151936, 159744, 100, 159744,
                                    FAKE, None, -100, FAKE, 39, None) == SHARD


def test_check_targets_host_validation():
    lib = dst.library()
    assert lib.logp_check_targets(FAKE, None, -1, 10, -100, FAKE, None) == SHAPE
    assert lib.logp_check_targets(FAKE, None, 5, 0, -100, FAKE, None) == SHAPE
    assert lib.logp_check_targets(FAKE, None, 5, 10, -100, None, None) == NULL
    assert lib.logp_check_targets(None, None, 5, 10, -100, FAKE, None) == NULL


def test_binding_rejects_cpu_tensors_without_calling_the_library():
    import torch
    x = torch.zeros((2, 8), dtype=torch.bfloat16)
    y = torch.zeros(2, dtype=torch.int64)
    with pytest.raises(ValueError, match="GPU tensor"):
        dst.logp_forward(x, y)
    with pytest.raises(TypeError):
        dst.logp_forward(x.float(), y)


def test_binding_rejects_partials_too_narrow_for_the_shard():
    """The C side sees the shard's first partials slot and the row stride only, so the
    binding must check that the shard's last tile still has a slot in the row: [20T, 39T)
    into a buffer of 30 tiles per row would write row t's tiles 30..38 over row t + 1."""
    import torch
    n = 2
    x = torch.zeros((n, 19 * T), dtype=torch.bfloat16)
    y = torch.zeros(n, dtype=torch.int64)
    for width in (30, 38):
        with pytest.raises(ValueError, match="run past"):
            dst.logp_partials(x, y, 39 * T, 39 * T, 20 * T, 39 * T,
                              torch.zeros((n, width, 3)))
    with pytest.raises(ValueError, match="run past"):  # a ragged last tile needs its slot too
        dst.logp_partials_ex(x[:, :T + 5], y, 21 * T + 5, 21 * T + 5, 20 * T, 21 * T + 5,
                             torch.zeros((n, 21, 3)))
    # wide enough: the shape checks pass and the next check (device memory) fails
    with pytest.raises(ValueError, match="GPU tensor"):
        dst.logp_partials(x, y, 39 * T, 39 * T, 20 * T, 39 * T, torch.zeros((n, 39, 3)))
    with pytest.raises(ValueError, match="GPU tensor"):
        dst.logp_partials_ex(x[:, :T + 5], y, 21 * T + 5, 21 * T + 5, 20 * T, 21 * T + 5,
                             torch.zeros((n, 22, 3)))


def test_product_path_never_imports_the_oracle():
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, flags=re.M), f
                assert "logp_oracle" not in text and "grpo_oracle" not in text, f
    for h in HEADERS:
        assert "oracle" not in open(h).read().lower(), h


def test_import_fails_loudly_without_the_library():
    tmp = tempfile.mkdtemp(prefix="nolib_")
    try:
        dst_pkg = os.path.join(tmp, "deterministic_selected_token_amd")
        os.makedirs(dst_pkg)
        shutil.copy(os.path.join(PKG, "__init__.py"), dst_pkg)
        r = subprocess.run([sys.executable, "-c", "import deterministic_selected_token_amd"],
                           cwd=tmp, capture_output=True, text=True,
                           env={k: v for k, v in dict(os.environ, PYTHONPATH=tmp).items()
                                if k != "DST_AMD_LIB"})
        assert r.returncode != 0 and "is missing: build it first" in r.stderr
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
