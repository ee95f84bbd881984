"""GRPO loss on the GPU against the FP64 oracle, and its bitwise contract.

Tolerances (float32 kernels against the float64 oracle):
  * per-token gradient: |gpu - oracle| <= 2^-19 (|d pg| + beta |d kl|) * s + 1e-30, s the
    token's normalizer weight; tokens whose float32 ratio lies within two spacings of a clip
    bound may take either branch (a last-bit difference in exp moves them across), so for
    them either branch's gradient is accepted.
  * sums (per-sequence pg_sum / kl_sum, the reduced losses): 4e-6 of the sum of absolute
    terms, plus 1e-30 (float32 sums of up to a few thousand terms, each within ~2^-21; the
    KL term is formed without cancellation for small |d|, so this holds for it too).
  * token counts exact; clipped counts within the number of ambiguous tokens; clip_frac
    within that count over the tokens plus its own float32 rounding (2^-24 of its value).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import deterministic_selected_token_amd as dst
from deterministic_selected_token_amd import grpo

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(msg: str):
    print(f"[gpu] {msg}", flush=True)


def make_batch(n, T, seed, spread=0.3, mask_frac=0.15, empty_rows=(), ld=None, adv_zero=0.1):
    g = torch.Generator().manual_seed(seed)
    ld = T if ld is None else ld
    lp = torch.randn((n, ld), generator=g) * 1.5 - 2.0
    old = lp + torch.randn((n, ld), generator=g) * spread
    ref = lp + torch.randn((n, ld), generator=g) * spread
    adv = torch.randn(n, generator=g)
    adv[torch.rand(n, generator=g) < adv_zero] = 0.0
    mask = (torch.rand((n, ld), generator=g) >= mask_frac).to(torch.uint8)
    for r in empty_rows:
        mask[r] = 0
    return {k: v.to(DEV) for k, v in dict(lp=lp, old=old, ref=ref, adv=adv, mask=mask).items()}


def host(t, T):
    return t[:, :T].cpu().numpy()


def check_against_oracle(b, T, mode, beta, eps_low=0.2, eps_high=0.28, use_ref=True,
                         use_mask=True, norm_tokens=0, norm_seqs=0):
    from oracle import grpo_oracle as O
    lp, old = b["lp"][:, :T], b["old"][:, :T]
    ref = b["ref"][:, :T] if use_ref else None
    mask = b["mask"][:, :T] if use_mask else None
    loss, st, d = grpo.grpo_loss(lp, old, b["adv"], ref_logp=ref, mask=mask, mode=mode,
                                 eps_low=eps_low, eps_high=eps_high, beta=beta,
                                 norm_tokens=norm_tokens, norm_seqs=norm_seqs)
    torch.cuda.synchronize()
    L = grpo.loss_fields(loss)
    S = {k: v.cpu().numpy() for k, v in grpo.partial_fields(st).items()}
    ref_np = host(b["ref"], T) if use_ref else None
    mask_np = host(b["mask"], T) if use_mask else None
    o = O.loss(host(b["lp"], T), host(b["old"], T), ref_np, b["adv"].cpu().numpy(), mask_np,
               mode=mode, eps_low=eps_low, eps_high=eps_high, beta=beta,
               norm_tokens=norm_tokens, norm_seqs=norm_seqs)
    amb = o["ambiguous"]
    n_amb = int(amb.sum())
    beta_eff = float(np.float32(beta)) if use_ref else 0.0
    # counts
    assert np.array_equal(S["tokens"], o["seq_tokens"])
    assert np.all(np.abs(S["clipped"] - o["seq_clipped"]) <= amb.sum(1))
    assert L["tokens"] == o["tokens"] and L["sequences"] == o["sequences"]
    assert abs(L["clipped"] - o["clipped"]) <= n_amb
    # per-sequence sums
    t = o["terms"]
    pg_abs = np.abs(t["pg"]).sum(1)
    kl_abs = np.abs(t["kl"]).sum(1)
    assert np.all(np.abs(S["pg_sum"] - o["seq_pg_sum"]) <= 4e-6 * pg_abs + 1e-30 +
                  (amb * np.abs(t["pg"])).sum(1) * 1e-6)
    kl_bound = 4e-6 * kl_abs
    assert np.all(np.abs(S["kl_sum"] - o["seq_kl_sum"]) <= kl_bound + 1e-30)
    # reduced losses
    n_i = np.maximum(o["seq_tokens"], 1)
    if mode == "token_mean":
        D = o["tokens"] if norm_tokens == 0 else norm_tokens
        pg_scale, kl_tol = pg_abs.sum() / max(D, 1), kl_bound.sum() / max(D, 1)
    else:
        D = (o["sequences"] if norm_seqs == 0 else norm_seqs) if mode == "seq_mean" else 1
        pg_scale = (pg_abs / n_i).sum() / max(D, 1)
        kl_tol = (kl_bound / n_i).sum() / max(D, 1)
    assert L["norm"] == D
    assert abs(L["pg_loss"] - o["pg_loss"]) <= 4e-6 * pg_scale + 1e-30
    assert abs(L["kl_loss"] - o["kl_loss"]) <= kl_tol + 1e-30
    assert abs(L["loss"] - o["loss"]) <= 4e-6 * pg_scale + beta_eff * kl_tol + 1e-30
    assert abs(L["clip_frac"] - o["clip_frac"]) <= \
        (n_amb + 1e-3) / max(o["tokens"], 1) + 2.0 ** -24 * o["clip_frac"]
    # gradient: each token's normalizer weight s, then either branch for ambiguous tokens
    g = host(d, T).astype(np.float64)
    t = o["terms"]
    act = t["active"]
    n_seq = o["seq_tokens"].astype(np.float64)
    if mode == "token_mean":
        s_row = np.full(len(n_seq), 1.0 / D if D > 0 else 0.0)
    elif mode == "seq_mean":
        s_row = np.where(n_seq > 0, 1.0 / (np.maximum(n_seq, 1) * max(D, 1)), 0.0)
    else:
        s_row = np.where(n_seq > 0, 1.0 / np.maximum(n_seq, 1), 0.0)
    s_tok = np.where(act, s_row[:, None], 0.0)
    A = np.broadcast_to(b["adv"].cpu().numpy().astype(np.float64)[:, None], act.shape)
    kl_part = beta_eff * t["dkl"]
    cand_c = kl_part * s_tok                          # clipped branch
    cand_u = (-A * t["ratio"] + kl_part) * s_tok      # unclipped branch
    tol = 2.0 ** -19 * (np.abs(A * t["ratio"]) + np.abs(kl_part)) * s_tok + 1e-30
    err = np.abs(g - o["dlogp"])
    ok = (err <= tol) | (amb & ((np.abs(g - cand_c) <= tol) | (np.abs(g - cand_u) <= tol)))
    assert ok.all(), (mode, np.argwhere(~ok)[:5], err[~ok][:5], tol[~ok][:5])
    assert np.all(g[~act] == 0.0)
    return L, o


SHAPES = [(1, 1), (3, 63), (5, 256), (7, 257), (4, 1000), (9, 3000), (2, 8192), (33, 300)]


@pytest.mark.parametrize("n,T", SHAPES, ids=[f"n{n}_T{T}" for n, T in SHAPES])
@pytest.mark.parametrize("mode", list(grpo.MODES))
def test_grpo_parity(n, T, mode):
    b = make_batch(n, T, seed=n * 31 + T, empty_rows=(1,) if n > 2 else ())
    say(f"grpo parity n={n} T={T} {mode}")
    for beta, use_ref, use_mask in ((0.04, True, True), (0.0, False, False), (0.3, True, False)):
        L, o = check_against_oracle(b, T, mode, beta, use_ref=use_ref, use_mask=use_mask)
    say(f"n={n} T={T} {mode}: loss {L['loss']:.6g} vs {o['loss']:.6g}")


@pytest.mark.parametrize("mode", list(grpo.MODES))
def test_grpo_parity_global_normalizers_and_row_stride(mode):
    b = make_batch(6, 700, seed=5, ld=777, empty_rows=(2,))
    say(f"global normalizers, ld=777, {mode}")
    check_against_oracle(b, 700, mode, 0.1, eps_low=0.1, eps_high=0.4, norm_tokens=5000,
                         norm_seqs=16)


def test_grpo_large_ratios_and_clip_edges():
    """Spread 2.0 puts most ratios outside the clip interval on both sides."""
    b = make_batch(8, 2000, seed=9, spread=2.0)
    say("wide ratios")
    for mode in grpo.MODES:
        L, o = check_against_oracle(b, 2000, mode, 0.04)
        assert 0.3 < o["clip_frac"] < 0.9


def test_kl_term_small_differences():
    """One token per sequence with ref - logp = d from 0.49 down to 1e-7: each sequence's KL
    sum is the token's exp(d) - d - 1 to within 4 float32 units relative (expm1(d) - d in
    float32 would be off by about 2^-23 / |d| relative: 1e-2 at d = 1e-5).  The oracle's
    float64 expm1(d) - d is itself within 2^-52 / |d| relative, 2e-9 at the smallest d."""
    from oracle import grpo_oracle as O
    d = np.array([0.49, -0.49, 0.1, -0.1, 1e-2, -1e-2, 1e-3, -1e-3, 1e-5, -1e-5, 1e-7, -1e-7,
                  0.7, -0.7, 3.0, 0.0], dtype=np.float32)
    n = d.size
    lp = np.full((n, 1), -2.0, dtype=np.float32)
    ref = (lp + d[:, None]).astype(np.float32)
    e = ref.astype(np.float64) - lp  # exact: the float32 difference the kernel forms
    adv = np.linspace(-1.0, 1.0, n).astype(np.float32)
    t = {k: torch.from_numpy(v).to(DEV) for k, v in dict(lp=lp, ref=ref, adv=adv).items()}
    say("KL term at small ref - logp")
    _, st, _ = grpo.grpo_loss(t["lp"], t["lp"], t["adv"], ref_logp=t["ref"],
                              mode="seq_sum_token_mean", beta=0.1)
    torch.cuda.synchronize()
    got = grpo.partial_fields(st)["kl_sum"].cpu().numpy().astype(np.float64)
    o = O.loss(lp, lp, ref, adv, None, mode="seq_sum_token_mean", beta=0.1)
    want = o["seq_kl_sum"]
    assert np.allclose(want, np.expm1(e[:, 0]) - e[:, 0], rtol=0, atol=0)
    rel = np.abs(got - want) / np.where(want > 0, want, 1.0)
    assert got[-1] == 0.0 and np.all(got >= 0)
    assert np.all(rel <= 4 * 2.0 ** -24 + 2.0 ** -52 / np.maximum(np.abs(e[:, 0]), 1e-300)), \
        list(zip(d.tolist(), rel.tolist()))
    say(f"KL relative errors: max {rel.max():.3e}")


def expected_identity_grad(adv, mask, mode):
    """d loss / d logp at logp == old_logp == ref_logp: fl32(-A) * fl32(1 / den)."""
    act = mask != 0
    n_i = act.sum(1).astype(np.float64)
    if mode == "token_mean":
        den = np.full(len(n_i), act.sum(), dtype=np.float64)
    elif mode == "seq_mean":
        den = n_i * (n_i > 0).sum()
    else:
        den = n_i
    s = np.where(den > 0, (1.0 / np.where(den > 0, den, 1.0)), 0.0).astype(np.float32)
    g = (-adv.astype(np.float32))[:, None] * s[:, None]
    return np.where(act, g, np.float32(0)).astype(np.float32)


@pytest.mark.parametrize("mode", list(grpo.MODES))
def test_kl_zero_identity_bitwise(mode):
    """logp == old_logp == ref_logp: ratio 1, kl 0, no clipping, and d loss / d logp is
    bitwise fl32(-A) * fl32(1/den) -- the gradient of -A logp under the same reduction."""
    b = make_batch(12, 1500, seed=13, empty_rows=(4,))
    lp = b["lp"]
    say(f"KL=0 identity {mode}")
    loss, st, d = grpo.grpo_loss(lp, lp, b["adv"], ref_logp=lp, mask=b["mask"], mode=mode,
                                 beta=0.04)
    L = grpo.loss_fields(loss)
    want = expected_identity_grad(b["adv"].cpu().numpy(), b["mask"].cpu().numpy(), mode)
    got = d.cpu().numpy()
    assert np.array_equal(got, want)  # every value equal (A = 0 tokens: +0 vs -0 compare equal)
    S = grpo.partial_fields(st)
    assert L["clipped"] == 0 and L["kl_loss"] == 0.0
    assert torch.all(S["kl_sum"] == 0) and torch.all(S["clipped"] == 0)
    # pg per sequence: the sum of n_i copies of -A_i, in float32
    a = b["adv"].cpu().numpy().astype(np.float64)
    n_i = S["tokens"].cpu().numpy()
    assert np.allclose(S["pg_sum"].cpu().numpy(), -a * n_i, rtol=1e-6, atol=0)


def test_run_to_run_bitwise():
    b = make_batch(16, 4000, seed=17)
    say("run to run")
    outs = [grpo.grpo_loss(b["lp"], b["old"], b["adv"], ref_logp=b["ref"], mask=b["mask"],
                           mode="seq_mean", beta=0.04) for _ in range(3)]
    for o in outs[1:]:
        for u, w in zip(outs[0], o):
            assert torch.equal(u, w)


def test_side_stream_is_bitwise():
    """The loss's kernels (counts, normalizer, per-sequence pass, reduce) all run on the stream
    they are given: a side stream reproduces the default stream's bits while the default
    stream is kept busy."""
    b = make_batch(40, 3000, seed=41, empty_rows=(3,))
    say("grpo on a side stream")

    def run():
        loss, st, d = grpo.grpo_loss(b["lp"], b["old"], b["adv"], ref_logp=b["ref"],
                                     mask=b["mask"], mode="seq_mean", beta=0.04)
        return loss, st, d

    ref = run()
    torch.cuda.synchronize()
    busy = torch.randn((4096, 4096), device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    for _ in range(8):
        busy = torch.tanh(busy @ busy.t() * 1e-3)  # keeps the default stream occupied
    with torch.cuda.stream(s):
        got = run()
    s.synchronize()
    torch.cuda.synchronize()
    for u, w in zip(ref, got):
        assert torch.equal(u.contiguous().view(torch.int32) if u.dtype == torch.float32 else u,
                           w.contiguous().view(torch.int32) if w.dtype == torch.float32 else w)


@pytest.mark.parametrize("mode", list(grpo.MODES))
def test_data_parallel_split_is_bitwise(mode):
    """Sequences split over 'ranks' with the global normalizers: the concatenated per-sequence
    sums and gradients, and the reduced loss, equal one call over the whole batch."""
    n, T = 40, 1200
    b = make_batch(n, T, seed=19, empty_rows=(7, 30))
    say(f"data-parallel split {mode}")
    kw = dict(ref_logp=b["ref"], mask=b["mask"], mode=mode, beta=0.04)
    loss, st, d = grpo.grpo_loss(b["lp"], b["old"], b["adv"], **kw)
    L = grpo.loss_fields(loss)
    for bounds in ([0, 13, 27, 40], [0, 1, 39, 40], [0, 20, 40]):
        sts, ds = [], []
        for r0, r1 in zip(bounds[:-1], bounds[1:]):
            s = slice(r0, r1)
            kw_r = dict(ref_logp=b["ref"][s], mask=b["mask"][s], mode=mode, beta=0.04,
                        norm_tokens=L["tokens"], norm_seqs=L["sequences"])
            _, st_r, d_r = grpo.grpo_loss(b["lp"][s], b["old"][s], b["adv"][s], **kw_r)
            sts.append(st_r)
            ds.append(d_r)
        cat = torch.cat(sts)
        assert torch.equal(cat, st)
        assert torch.equal(torch.cat(ds), d)
        red = grpo.grpo_loss_reduce(cat, mode=mode, beta=0.04, norm_tokens=L["tokens"],
                                    norm_seqs=L["sequences"])
        assert torch.equal(red, loss), bounds


@pytest.mark.parametrize("mode", list(grpo.MODES))
def test_context_parallel_split_is_bitwise(mode):
    """Each sequence split at token-tile boundaries: per-shard counts add up, shard partials
    merge to the whole-sequence sums, shard gradients equal the whole-sequence ones."""
    n, T = 10, 2500  # 10 tiles, the last one ragged
    b = make_batch(n, T, seed=23, empty_rows=(3,))
    say(f"context-parallel split {mode}")
    loss, st, d = grpo.grpo_loss(b["lp"], b["old"], b["adv"], ref_logp=b["ref"],
                                 mask=b["mask"], mode=mode, beta=0.04)
    L = grpo.loss_fields(loss)
    L_tiles = -(-T // grpo.TOKEN_TILE)
    for cuts in ([0, 2500], [0, 1280, 2500], [0, 512, 768, 2048, 2500], [0, 256 * 9, 2500]):
        counts = torch.zeros(n, dtype=torch.int32, device=DEV)
        for t0, t1 in zip(cuts[:-1], cuts[1:]):
            counts += grpo.grpo_token_counts(b["mask"], t0, t1)
        assert torch.equal(counts, grpo.partial_fields(st)["tokens"])
        partials = torch.full((n, L_tiles, 4), -1, dtype=torch.int32, device=DEV)
        dl = torch.full((n, T), float("nan"), device=DEV)
        for t0, t1 in zip(cuts[:-1], cuts[1:]):
            c = slice(t0, t1)
            grpo.grpo_loss_partials(b["lp"][:, c], b["old"][:, c], b["adv"], T, t0, partials,
                                    ref_logp=b["ref"][:, c], mask=b["mask"][:, c],
                                    seq_tokens=counts, dlogp=dl[:, c], mode=mode, beta=0.04,
                                    norm_tokens=L["tokens"], norm_seqs=L["sequences"])
        st2 = grpo.grpo_loss_merge(partials, L_tiles)
        assert torch.equal(st2, st), cuts
        assert torch.equal(dl, d), cuts
        red = grpo.grpo_loss_reduce(st2, mode=mode, beta=0.04, norm_tokens=L["tokens"],
                                    norm_seqs=L["sequences"])
        assert torch.equal(red, loss)


@pytest.mark.parametrize("G", [1, 2, 5, 8, 64, 100])
def test_advantages(G):
    from oracle import grpo_oracle as O
    n = G * 37
    r = (torch.randn(n, generator=torch.Generator().manual_seed(G)) * 3 + 1).to(DEV)
    say(f"advantages G={G}")
    for sbs in (True, False):
        a = grpo.grpo_advantages(r, G, eps=1e-6, scale_by_std=sbs)
        want = O.advantages(r.cpu().numpy(), G, eps=1e-6, scale_by_std=sbs)
        spread = np.abs(r.cpu().numpy()).reshape(-1, G).max(1).repeat(G)
        den = 1.0
        if sbs and G > 1:
            g = r.cpu().numpy().astype(np.float64).reshape(-1, G)
            den = (g.std(1, ddof=1) + 1e-6).repeat(G)
        assert np.all(np.abs(a.cpu().numpy() - want) <= 1e-5 * spread / den + 1e-30)
    # in place
    r2 = r.clone()
    grpo.grpo_advantages(r2, G, adv=r2)
    assert torch.equal(r2, grpo.grpo_advantages(r, G))


def test_empty_batch_and_no_active_tokens():
    say("empty inputs")
    e = torch.empty((0, 10), device=DEV)
    loss, st, d = grpo.grpo_loss(e, e, torch.empty(0, device=DEV))
    L = grpo.loss_fields(loss)
    assert L["tokens"] == 0 and L["loss"] == 0.0 and L["norm"] == 0
    b = make_batch(3, 100, seed=29, empty_rows=(0, 1, 2))
    for mode in grpo.MODES:
        loss, st, d = grpo.grpo_loss(b["lp"], b["old"], b["adv"], ref_logp=b["ref"],
                                     mask=b["mask"], mode=mode, beta=0.1)
        L = grpo.loss_fields(loss)
        assert L["tokens"] == 0 and L["sequences"] == 0 and L["loss"] == 0.0
        assert torch.all(d == 0)


def test_grpo_step_chain_logits_to_dlogits():
    """logp_forward -> grpo_loss -> logp_backward: logp [B*T] viewed as [B, T], dlogp fed back
    as the upstream gradient, each stage checked against the oracle on its own inputs."""
    import oracle
    from oracle import grpo_oracle as O
    from parity_checks import BackwardTally, host_values
    B, T, V = 4, 300, 5000
    gen = torch.Generator().manual_seed(31)
    x = (torch.randn((B * T, V), generator=gen) * 2).to(torch.bfloat16).to(DEV)
    y = torch.randint(0, V, (B * T,), generator=gen).to(DEV)
    say("grpo step chain")
    logp, lse, stats = dst.logp_forward(x, y)
    lp = logp.view(B, T)
    old = (lp + 0.05 * torch.randn((B, T), device=DEV)).contiguous()
    adv = grpo.grpo_advantages(torch.randn(B, device=DEV), 2)
    loss, st, d = grpo.grpo_loss(lp, old, adv, ref_logp=old, mode="seq_mean", beta=0.04)
    dlogits = dst.logp_backward(x, y, d.reshape(-1), stats)
    torch.cuda.synchronize()
    xo = x.cpu()
    ref_f = oracle.forward(xo, y.cpu().numpy(), V)
    assert np.abs(logp.cpu().numpy() - ref_f["logp"]).max() <= 1e-4
    o = O.loss(lp.cpu().numpy(), old.cpu().numpy(), old.cpu().numpy(), adv.cpu().numpy(),
               None, mode="seq_mean", beta=0.04)
    assert abs(grpo.loss_fields(loss)["loss"] - o["loss"]) <= 1e-5 * (1 + abs(o["loss"]))
    t = BackwardTally()
    t.add_block(xo, y.cpu().numpy(), d.reshape(-1).cpu().numpy(), V, V, None, -100,
                host_values(dlogits), "grpo chain")
    t.finish("grpo chain")
