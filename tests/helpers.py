"""Shared test helpers: run the HIP path on a seeded workload and compare it
with the oracle under the stated tolerance."""

from __future__ import annotations

import contextlib
import sys

import numpy as np

# Output tolerance on bf16 outputs against the unrounded fp64 oracle, per
# element: |gpu - ref| <= ATOL + RTOL * |ref| (max-abs 1e-2, max-rel 2e-2).
ATOL = 1e-2
RTOL = 2e-2
# LSE is a diagnostic of the softmax normaliser, held to an absolute bound
# plus a part relative to its size: the matrix-core fp8 dot products that
# produce the logits accumulate with a relative error near 2^-13 of the sum
# of |products| (measured on the hardware), which shifts large logits (K
# outlier channels) by a few 1e-3.
LSE_ATOL = 2e-3
LSE_RTOL = 2e-4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def compare_out(out_gpu, O_ref, what=""):
    g = out_gpu.float().cpu().numpy().astype(np.float64)
    ok = ~np.isnan(O_ref)
    assert ok.any()
    diff = np.abs(g - O_ref)[ok]
    ref = np.abs(O_ref)[ok]
    bad = diff > ATOL + RTOL * ref
    stats = dict(max_abs=float(diff.max()), max_rel=float((diff / np.maximum(ref, 1e-3)).max()),
                 n_bad=int(bad.sum()), n=int(ok.sum()))
    say(f"  {what} out: max_abs={stats['max_abs']:.3e} max_rel(|ref|>=1e-3)={stats['max_rel']:.3e} "
        f"bad={stats['n_bad']}/{stats['n']}")
    assert np.all(np.isfinite(g[ok])), f"{what}: non-finite outputs"
    assert stats["n_bad"] == 0, f"{what}: {stats}"
    return stats


def compare_lse(lse_gpu, LSE_ref, what=""):
    g = lse_gpu.cpu().numpy().astype(np.float64)
    ok = ~np.isnan(LSE_ref)
    fin = ok & np.isfinite(LSE_ref)
    assert np.array_equal(np.isneginf(g[ok]), np.isneginf(LSE_ref[ok])), f"{what}: -inf LSE rows differ"
    if fin.any():
        d = np.abs(g[fin] - LSE_ref[fin])
        say(f"  {what} lse: max_abs={d.max():.3e}")
        assert np.all(d <= LSE_ATOL + LSE_RTOL * np.abs(LSE_ref[fin])), f"{what}: lse max_abs {d.max()}"


def oracle_step(wl, seqs=None, heads=None, quantize=True):
    """Run the oracle on a workload (optionally on a subset of sequences /
    KV heads).  Returns O, LSE for the full batch shape (NaN where skipped)."""
    from oracle.attention import decode_step

    s = wl.spec
    seqs = list(range(s.b)) if seqs is None else list(seqs)
    heads = list(range(s.h_k)) if heads is None else list(heads)
    h = wl.host(seqs)
    O_sub, L_sub = decode_step(h, q_len=s.q_len, h_q=s.h_q, h_k=s.h_k, d=s.d, page_size=s.page_size,
                               kv_format=s.kv_format, causal=s.causal, quantize=quantize,
                               pairs=[(r, g) for r in range(len(seqs)) for g in heads])
    O = np.full((s.b * s.q_len, s.h_q, s.d), np.nan)
    LSE = np.full((s.b * s.q_len, s.h_q), np.nan)
    for r, i in enumerate(seqs):
        O[i * s.q_len:(i + 1) * s.q_len] = O_sub[r * s.q_len:(r + 1) * s.q_len]
        LSE[i * s.q_len:(i + 1) * s.q_len] = L_sub[r * s.q_len:(r + 1) * s.q_len]
    return O, LSE


@contextlib.contextmanager
def step_overrides(**kw):
    """Config fields (kernel selection: decode_kernel, kv_cache_policy,
    step_merge) that every DecodeStep built inside the block takes unless its
    caller passes them: the A/B and every-kernel tests run one test body on
    each kernel.  Test-side only; the library keeps no such state."""
    from paged_fp8_decode_amd import runner

    orig = runner.DecodeStep.__init__

    def init(self, **a):
        orig(self, **{**kw, **a})

    runner.DecodeStep.__init__ = init
    try:
        yield
    finally:
        runner.DecodeStep.__init__ = orig
