"""Host-side validation of the GRPO-loss entry points (no GPU: every case fails before any
HIP call), and the layout of the structs the binding shares with include/grpo_loss.h."""

from __future__ import annotations

import ctypes
import os
import re

import pytest

from deterministic_selected_token_amd import grpo

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "grpo_loss.h")
OK, NULL, SHAPE, SHARD, ARG = 0, 1, 2, 3, 8
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced
lib = grpo._lib


def P(**kw):
    return ctypes.byref(grpo.params(**kw))


def test_header_constants_and_struct_layout():
    text = open(HEADER).read()
    assert re.search(r"#define GRPO_TOKEN_TILE (\d+)", text).group(1) == str(grpo.TOKEN_TILE)
    assert grpo.MAX_SEQ_LEN == grpo.TOKEN_TILE * 4096
    for name, code in grpo.MODES.items():
        assert re.search(rf"GRPO_{name.upper()}\s*=\s*{code}\b", text), name
    assert ctypes.sizeof(grpo.GrpoParams) == 32
    assert grpo.GrpoParams.norm_tokens.offset == 16


def loss_call(**over):
    a = dict(logp=FAKE, old=FAKE, ref=None, adv=FAKE, mask=None, n=4, T=100, ld=100,
             params=P(), seq_stats=FAKE, loss=FAKE, dlogp=None)
    a.update(over)
    return lib.grpo_loss(a["logp"], a["old"], a["ref"], a["adv"], a["mask"], a["n"], a["T"],
                         a["ld"], a["params"], a["seq_stats"], a["loss"], a["dlogp"], None)


@pytest.mark.parametrize("over,want", [
    (dict(logp=None), NULL), (dict(old=None), NULL), (dict(adv=None), NULL),
    (dict(seq_stats=None), NULL), (dict(loss=None), NULL), (dict(params=None), NULL),
    (dict(n=-1), SHAPE), (dict(T=-1), SHAPE), (dict(ld=99), SHAPE),
    (dict(T=grpo.MAX_SEQ_LEN + 1, ld=grpo.MAX_SEQ_LEN + 1), SHAPE),
    (dict(params=P(mode="token_mean", eps_low=-0.1)), ARG),
    (dict(params=P(eps_low=1.5)), ARG), (dict(params=P(eps_high=float("inf"))), ARG),
    (dict(params=P(beta=float("nan"))), ARG), (dict(params=P(beta=-1.0)), ARG),
    (dict(params=P(norm_tokens=-3)), ARG), (dict(params=P(norm_seqs=-1)), ARG),
], ids=lambda v: str(v))
def test_grpo_loss_host_validation(over, want):
    assert loss_call(**over) == want


def test_bad_mode_is_rejected():
    p = grpo.params()
    p.mode = 7
    assert loss_call(params=ctypes.byref(p)) == ARG


def partials_call(**over):
    a = dict(logp=FAKE, old=FAKE, ref=None, adv=FAKE, mask=None, n=4, T=1000, ld=1000,
             t0=0, t1=512, seq_tokens=None, params=P(norm_tokens=10), partials=FAKE, ldp=4,
             dlogp=None)
    a.update(over)
    return lib.grpo_loss_partials(a["logp"], a["old"], a["ref"], a["adv"], a["mask"], a["n"],
                                  a["T"], a["ld"], a["t0"], a["t1"], a["seq_tokens"],
                                  a["params"], a["partials"], a["ldp"], a["dlogp"], None)


@pytest.mark.parametrize("over,want", [
    (dict(partials=None), NULL), (dict(t0=100), SHARD), (dict(t1=300), SHARD),
    (dict(t0=512, t1=256), SHARD), (dict(t1=1001), SHARD), (dict(ldp=3), SHAPE),
    # missing normalizer metadata for the gradient fails loudly
    (dict(dlogp=FAKE, params=P(mode="token_mean")), ARG),
    (dict(dlogp=FAKE, params=P(mode="seq_mean", norm_seqs=4)), ARG),
    (dict(dlogp=FAKE, params=P(mode="seq_mean"), seq_tokens=FAKE), ARG),
    (dict(dlogp=FAKE, params=P(mode="seq_sum_token_mean")), ARG),
], ids=lambda v: str(v))
def test_grpo_partials_host_validation(over, want):
    assert partials_call(**over) == want


def test_other_entry_points_validate():
    assert lib.grpo_advantages(FAKE, 10, 3, 1e-6, 1, FAKE, None) == SHAPE
    assert lib.grpo_advantages(FAKE, 9, 0, 1e-6, 1, FAKE, None) == SHAPE
    assert lib.grpo_advantages(FAKE, 9, 3, -1.0, 1, FAKE, None) == ARG
    assert lib.grpo_advantages(None, 9, 3, 1e-6, 1, FAKE, None) == NULL
    assert lib.grpo_advantages(FAKE, 0, 3, 1e-6, 1, FAKE, None) == OK  # empty: no launch
    assert lib.grpo_token_counts(FAKE, 4, 100, 100, 0, 101, FAKE, None) == SHAPE
    assert lib.grpo_token_counts(FAKE, 4, 100, 100, 50, 40, FAKE, None) == SHAPE
    assert lib.grpo_token_counts(FAKE, 4, 100, 100, 0, 100, None, None) == NULL
    assert lib.grpo_loss_merge(FAKE, 3, 4, 4, FAKE, None) == SHAPE
    assert lib.grpo_loss_merge(None, 4, 4, 4, FAKE, None) == NULL
    assert lib.grpo_loss_merge(None, 4, 0, 4, None, None) == OK
    assert lib.grpo_token_counts(None, 0, 100, 100, 0, 100, None, None) == OK
    assert lib.grpo_advantages(None, 0, 3, 1e-6, 1, None, None) == OK
    assert lib.grpo_loss_merge(FAKE, 4, 0, 4, FAKE, None) == OK
    assert lib.grpo_loss_reduce(FAKE, -1, P(), FAKE, None) == SHAPE
    assert lib.grpo_loss_reduce(FAKE, 4, None, FAKE, None) == NULL
    assert lib.grpo_loss_reduce(FAKE, 4, P(), None, None) == NULL
    assert lib.grpo_loss_reduce(None, 4, P(), FAKE, None) == NULL


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros((2, 8))
    with pytest.raises(ValueError, match="GPU tensor"):
        grpo.grpo_loss(x, x, torch.zeros(2))
