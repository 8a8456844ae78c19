"""Pins of the attention oracle: dense reduction against torch's
scaled_dot_product_attention in fp64, physical-page permutation invariance,
split-count invariance of the LSE merge, softmax row sums, closed-form special
cases, the fp6 scale folding identity and HND/NHD equivalence."""

import math

import numpy as np
import pytest
import torch

import synth
from oracle import attention as A
from oracle.formats import e2m1_decode, e2m3_decode, e3m2_decode, e4m3_decode, unpack_4bit, unpack_6bit


def _ref_sdpa(qrows, K, V, allowed, scale):
    """Library route: torch SDPA in fp64 on the CPU with an explicit boolean mask."""
    q = torch.from_numpy(qrows)[None, None]
    k = torch.from_numpy(K)[None, None]
    v = torch.from_numpy(V)[None, None]
    m = torch.from_numpy(allowed)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=m, scale=scale)[0, 0].numpy()


def _small(key, **kw):
    wl = synth.build(synth.spec_for(key, small=True, **kw))
    return wl, wl.host()


def _args(wl):
    s = wl.spec
    return dict(q_len=s.q_len, h_q=s.h_q, h_k=s.h_k, d=s.d, page_size=s.page_size, kv_format=s.kv_format)


@pytest.mark.parametrize("key", ["cfg1", "cfg2", "cfg4c", "cfg4n", "cfg5", "cfg5_e3m2", "cfg5_e2m1", "cfg5_nvfp4",
                                 "cfg3_nvfp4", "cfg3_e2m3", "cfg3_e2m1"])
def test_matches_sdpa_per_head(key):
    wl, h = _small(key)
    s = wl.spec
    from oracle.qquant import quantize_q
    codes, qd = quantize_q(h["q"], s.b, s.q_len, s.h_k, h["q_mul"])
    O, LSE = A.decode_step(h, causal=s.causal, **_args(wl))
    for i in range(s.b):
        for g in range(s.h_k):
            qrows, K, V = A.head_inputs(h, i, g, q_codes=codes, q_descale=qd, **_args(wl))
            allowed = A.visible(K.shape[0], s.q_len, s.h_r, s.causal)
            ref = _ref_sdpa(qrows, K, V, allowed, h["softmax_scale"]).reshape(s.q_len, s.h_r, s.d)
            if h["o_mul"] is not None:
                ref = ref * h["o_mul"][g * s.h_r:(g + 1) * s.h_r][None]
            got = O[i * s.q_len:(i + 1) * s.q_len, g * s.h_r:(g + 1) * s.h_r]
            assert np.max(np.abs(got - ref)) < 1e-12
            # LSE against a direct logsumexp of the visible logits
            sc = h["softmax_scale"] * qrows @ K.T
            lse = np.array([np.log(np.sum(np.exp(sc[r][allowed[r]] - sc[r][allowed[r]].max())))
                            + sc[r][allowed[r]].max() for r in range(sc.shape[0])])
            assert np.max(np.abs(LSE[i * s.q_len:(i + 1) * s.q_len, g * s.h_r:(g + 1) * s.h_r].reshape(-1)
                                 - lse)) < 1e-12


@pytest.mark.parametrize("key", ["cfg1", "cfg2", "cfg4c", "cfg4n", "cfg5_nvfp4"])
def test_unquantized_q_matches_sdpa(key):
    """The bf16-Q reading (Q used as given, no quantization): each (sequence,
    KV head) equals torch SDPA in fp64 on Q rows gathered here by query head
    and token, the dequantized K/V and the step's mask."""
    wl, h = _small(key)
    s = wl.spec
    O, LSE = A.decode_step(h, causal=s.causal, quantize=False, **_args(wl))
    q = wl.q.float().numpy().astype(np.float64).reshape(s.b, s.q_len, s.h_q, s.d)
    for i in range(s.b):
        for g in range(s.h_k):
            _, K, V = A.head_inputs(h, i, g, quantize=False, **_args(wl))
            L = K.shape[0]
            for t in range(s.q_len):
                for r in range(s.h_r):
                    seen = L if not (s.causal and s.q_len > 1) else L - s.q_len + t + 1
                    allowed = np.zeros((1, L), bool)
                    allowed[0, :max(seen, 0)] = True
                    h_idx = g * s.h_r + r
                    got = O[i * s.q_len + t, h_idx]
                    if seen <= 0:
                        assert np.all(got == 0) and np.isneginf(LSE[i * s.q_len + t, h_idx])
                        continue
                    ref = _ref_sdpa(q[i, t, h_idx][None], K, V, allowed, h["softmax_scale"])[0]
                    assert np.max(np.abs(got - ref)) < 1e-12
                    sc = h["softmax_scale"] * (K[:seen] @ q[i, t, h_idx])
                    lse = sc.max() + math.log(np.sum(np.exp(sc - sc.max())))
                    assert abs(LSE[i * s.q_len + t, h_idx] - lse) < 1e-12


def test_gather_identity_table_is_dense_slice():
    # one page holding the whole sequence, identity block table: the gather is a plain slice
    rng = np.random.default_rng(0)
    L, h_k, row = 48, 3, 128
    pool = rng.integers(0, 256, size=(2, h_k, L, row), dtype=np.uint8)  # HND, page size L
    flat = pool.reshape(-1)
    st = (pool.strides[0], pool.strides[2], pool.strides[1])
    for g in range(h_k):
        got = A.gather_codes(flat, st, L, np.array([1]), L, g, row)
        assert np.array_equal(got, pool[1, g])


def test_physical_page_permutation_is_exactly_invariant():
    wl, h = _small("cfg2")
    s = wl.spec
    O1, L1 = A.decode_step(h, causal=True, **_args(wl))
    # move every page to a new physical slot and rewrite the block table to match
    kp = h["k_pool"].reshape(-1, h["k_strides"][0])
    vp = h["v_pool"].reshape(-1, h["v_strides"][0])
    perm = np.random.default_rng(1).permutation(kp.shape[0])
    inv = np.argsort(perm)
    h2 = dict(h, k_pool=kp[perm].reshape(-1), v_pool=vp[perm].reshape(-1), block_table=inv[h["block_table"]])
    O2, L2 = A.decode_step(h2, causal=True, **_args(wl))
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


@pytest.mark.parametrize("key", ["cfg2", "cfg4c", "cfg3_nvfp4"])
def test_split_merge_invariance(key):
    wl, h = _small(key)
    s = wl.spec
    rng = np.random.default_rng(2)
    from oracle.qquant import quantize_q
    codes, qd = quantize_q(h["q"], s.b, s.q_len, s.h_k)
    for i in range(s.b):
        qrows, K, V = A.head_inputs(h, i, 1, q_codes=codes, q_descale=qd, **_args(wl))
        allowed = A.visible(K.shape[0], s.q_len, s.h_r, s.causal)
        O, lse, P = A.attend(qrows, K, V, allowed, h["softmax_scale"])
        assert np.max(np.abs(P.sum(axis=1) - 1.0)) < 1e-12  # softmax rows sum to 1
        for nsplit in (1, 2, 3, 7, 16):
            cuts = np.sort(rng.choice(np.arange(1, K.shape[0]), size=nsplit - 1, replace=False)) if nsplit > 1 else []
            bounds = [0, *cuts.tolist(), K.shape[0]] if nsplit > 1 else [0, K.shape[0]]
            parts = [A.partial(qrows, K, V, allowed, h["softmax_scale"], a, b) for a, b in zip(bounds, bounds[1:])]
            Om, lm = A.merge(parts)
            assert np.max(np.abs(Om - O)) < 1e-12
            assert np.max(np.abs(lm - lse)) < 1e-12


def test_special_cases():
    rng = np.random.default_rng(4)
    d, n = 128, 6
    qrows = rng.standard_normal((n, d))
    K = rng.standard_normal((37, d))
    V = rng.standard_normal((37, d))
    allowed = np.ones((n, 37), dtype=bool)
    # constant V -> O = V
    Vc = np.tile(rng.standard_normal(d), (37, 1))
    O, _, _ = A.attend(qrows, K, Vc, allowed, 0.1)
    assert np.max(np.abs(O - Vc[0])) < 1e-12
    # L = 1 -> O = V_0, LSE = the single logit
    O, lse, _ = A.attend(qrows, K[:1], V[:1], allowed[:, :1], 0.1)
    assert np.max(np.abs(O - V[0])) < 1e-15
    assert np.max(np.abs(lse - 0.1 * qrows @ K[0])) < 1e-12
    # all-zero K -> uniform weights -> mean of V over the visible keys, LSE = ln(count)
    vis = A.visible(37, 3, 2, True)
    O, lse, _ = A.attend(qrows, np.zeros_like(K), V, vis, 0.1)
    for r in range(n):
        assert np.max(np.abs(O[r] - V[vis[r]].mean(axis=0))) < 1e-12
        assert abs(lse[r] - math.log(vis[r].sum())) < 1e-12
    # q_len == 1: causal and non-causal masks agree; causal last token == non-causal
    assert np.array_equal(A.visible(50, 1, 4, True), A.visible(50, 1, 4, False))
    c, nc = A.visible(50, 4, 2, True), A.visible(50, 4, 2, False)
    assert np.array_equal(c[-2:], nc[-2:])
    assert c[0].sum() == 47 and c[2].sum() == 48
    # no visible key -> O = 0, LSE = -inf
    O, lse, _ = A.attend(qrows, K[:0], V[:0], allowed[:, :0], 0.1)
    assert np.all(O == 0) and np.all(np.isneginf(lse))


def test_empty_sequence_in_a_batch():
    wl, h = _small("cfg2", lens=(0, 300, 129, 1))
    O, LSE = A.decode_step(h, causal=True, **_args(wl))
    assert np.all(O[0] == 0) and np.all(np.isneginf(LSE[0]))
    assert np.all(np.isfinite(O[1:]))


@pytest.mark.parametrize("key", ["cfg5", "cfg5_e3m2", "cfg5_e2m1"])
def test_fp6_folding_identity(key):
    """Channel scales folded into Q and O equal attention on explicitly
    dequantized K/V (the identities in mjolnir/backend.py, _install_fp6_scales)."""
    wl, h = _small(key)
    s = wl.spec
    O, _ = A.decode_step(h, causal=True, quantize=False, **_args(wl))
    ks = wl.k_channel_scale.numpy().astype(np.float64)
    vs = wl.v_channel_scale.numpy().astype(np.float64)
    for i in range(s.b):
        for g in (0, s.h_k - 1):
            L = int(h["seq_lens"][i])
            kc = A.gather_codes(h["k_pool"], h["k_strides"], s.page_size, h["block_table"][i], L, g, s.row_bytes)
            vc = A.gather_codes(h["v_pool"], h["v_strides"], s.page_size, h["block_table"][i], L, g, s.row_bytes)
            unpack = (lambda r: unpack_4bit(r, 128)) if s.kv_format == "e2m1" else (lambda r: unpack_6bit(r, 128))
            dec = {"e2m3": e2m3_decode, "e3m2": e3m2_decode, "e2m1": e2m1_decode}[s.kv_format]
            K = dec(unpack(kc)) * ks[g]
            V = dec(unpack(vc)) * vs[g]
            q = h["q"][i, g * s.h_r:(g + 1) * s.h_r].astype(np.float64)
            ref = _ref_sdpa(q, K, V, np.ones((s.h_r, L), bool), h["softmax_scale"])
            assert np.max(np.abs(O[i, g * s.h_r:(g + 1) * s.h_r] - ref)) < 1e-12


def test_hnd_and_nhd_layouts_agree():
    wl, h = _small("cfg2")
    s = wl.spec
    # rebuild the same logical cache in the token-major layout
    kp = wl.k_pool.permute(0, 2, 1, 3).contiguous()
    vp = wl.v_pool.permute(0, 2, 1, 3).contiguous()
    h2 = dict(h, k_pool=kp.numpy().reshape(-1), v_pool=vp.numpy().reshape(-1),
              k_strides=(kp.stride(0), kp.stride(1), kp.stride(2)),
              v_strides=(vp.stride(0), vp.stride(1), vp.stride(2)))
    O1, L1 = A.decode_step(h, causal=True, **_args(wl))
    O2, L2 = A.decode_step(h2, causal=True, **_args(wl))
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_descale_kinds_scale_linearly():
    wl, h = _small("cfg4c")
    s = wl.spec
    O, _ = A.decode_step(h, causal=True, **_args(wl))
    h2 = dict(h, v_descale=h["v_descale"] * 2.0)
    O2, _ = A.decode_step(h2, causal=True, **_args(wl))
    assert np.max(np.abs(O2 - 2.0 * O)) < 1e-12


@pytest.mark.parametrize("G", [2, 3, 8])
def test_context_parallel_combine_is_full_attention(G):
    """Attention over contiguous slices of the context, each normalized with
    its own LSE, combined by the LSE merge, equals attention over the whole
    context (slices may be empty; the last slice holds the causal tail)."""
    wl, h = _small("cfg4c")
    s = wl.spec
    from oracle.qquant import quantize_q
    codes, qd = quantize_q(h["q"], s.b, s.q_len, s.h_k, h["q_mul"])
    for i in range(s.b):
        for g in range(s.h_k):
            qrows, K, V = A.head_inputs(h, i, g, q_codes=codes, q_descale=qd, **_args(wl))
            L = K.shape[0]
            allowed = A.visible(L, s.q_len, s.h_r, s.causal)
            O, LSE, _ = A.attend(qrows, K, V, allowed, h["softmax_scale"])
            cuts = np.linspace(0, L - s.q_len, G).astype(int).tolist() + [L]  # last slice: the q_len tail and more
            cuts[0] = 0
            parts = []
            for a, b in zip(cuts[:-1], cuts[1:]):
                o, lse, _ = A.attend(qrows, K[a:b], V[a:b], allowed[:, a:b], h["softmax_scale"])
                parts.append((o, lse))
            Oc, LSEc = A.combine(parts)
            assert np.max(np.abs(Oc - O)) < 1e-12
            assert np.max(np.abs(LSEc - LSE)) < 1e-12
    # a row no slice saw: O = 0, LSE = -inf
    e = np.zeros((2, 128))
    Oc, LSEc = A.combine([(e, np.array([-np.inf, 0.0])), (e + 1.0, np.array([-np.inf, -np.inf]))])
    assert np.all(Oc[0] == 0) and LSEc[0] == -np.inf and np.all(Oc[1] == 0) and LSEc[1] == 0.0


def _descale_case(kind, seed=23):
    """Three sequences of two KV heads (b != h_k, so a transposed index
    reads another pair), two query heads each, q_len 2, HND pages of 16
    through a permuted block table.  Each (sequence, KV head) pair's true K
    and V are e4m3 values times that pair's own scale: per tensor one scale (0.625),
    per head 0.75*(g+1), per (sequence, head) 2^i * 3^g / 8, all distinct and
    exact in fp32 (V: times 1.25).
    The descale array is filled from those scales in the layout of its kind;
    the reference below never reads it."""
    rng = np.random.default_rng(seed)
    b, h_k, h_r, q_len, d, P = 3, 2, 2, 2, 128, 16
    lens = [37, 20, 50]
    finite = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)

    def scale(i, g, side):
        base = {"tensor": 0.625, "head": 0.75 * (g + 1), "seq_head": 2.0 ** i * 3.0 ** g / 8}[kind]
        return base * (1.0 if side == 0 else 1.25)

    pages = [-(-L // P) for L in lens]
    perm = rng.permutation(sum(pages) + 3)
    bt = np.zeros((b, max(pages)), dtype=np.int32)
    k = 0
    for i, n in enumerate(pages):
        bt[i, :n] = perm[k:k + n]
        k += n
    n_pages = len(perm)
    pools = [np.zeros((n_pages, h_k, P, d), dtype=np.uint8) for _ in range(2)]
    true = {}  # (i, g, side) -> fp64 values
    for i, L in enumerate(lens):
        for g in range(h_k):
            for side in range(2):
                codes = rng.choice(finite, size=(L, d))
                vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
                true[i, g, side] = vals * scale(i, g, side)
                for j in range(L):
                    pools[side][bt[i, j // P], g, j % P] = codes[j]
    if kind == "tensor":
        kd, vd = np.array([scale(0, 0, 0)]), np.array([scale(0, 0, 1)])
    elif kind == "head":
        kd = np.array([scale(0, g, 0) for g in range(h_k)])
        vd = np.array([scale(0, g, 1) for g in range(h_k)])
    else:
        kd = np.array([[scale(i, g, 0) for g in range(h_k)] for i in range(b)])
        vd = np.array([[scale(i, g, 1) for g in range(h_k)] for i in range(b)])
    q = torch.randn(b * q_len, h_k * h_r, d, generator=torch.Generator().manual_seed(seed)).to(torch.bfloat16)
    st = (h_k * P * d, d, P * d)
    h = dict(q=q.float().numpy(), k_pool=pools[0].reshape(-1), v_pool=pools[1].reshape(-1), k_strides=st,
             v_strides=st, block_table=bt, seq_lens=np.array(lens), k_descale=kd.astype(np.float32),
             v_descale=vd.astype(np.float32), descale_kind=kind, softmax_scale=1 / math.sqrt(d), q_mul=None,
             o_mul=None)
    args = dict(q_len=q_len, h_q=h_k * h_r, h_k=h_k, d=d, page_size=P, kv_format="e4m3")
    return h, args, true, q


def _descale_reference(h, args, true, q):
    """torch SDPA in fp64 on the pairs' true K and V, Q as given, the causal
    block's mask built here."""
    q_len, h_q, h_k, d = args["q_len"], args["h_q"], args["h_k"], args["d"]
    h_r = h_q // h_k
    b = len(h["seq_lens"])
    O = np.zeros((b * q_len, h_q, d))
    qq = q.float().numpy().astype(np.float64)
    for i, L in enumerate(h["seq_lens"]):
        for g in range(h_k):
            for t in range(q_len):
                allowed = np.zeros((h_r, L), bool)
                allowed[:, :L - q_len + t + 1] = True
                rows = qq[i * q_len + t, g * h_r:(g + 1) * h_r]
                O[i * q_len + t, g * h_r:(g + 1) * h_r] = _ref_sdpa(rows, true[i, g, 0], true[i, g, 1], allowed,
                                                                    h["softmax_scale"])
    return O


@pytest.mark.parametrize("kind", ["tensor", "head", "seq_head"])
def test_descale_kinds_against_true_values(kind):
    h, args, true, q = _descale_case(kind)
    O, _ = A.decode_step(h, causal=True, quantize=False, **args)
    assert np.max(np.abs(O - _descale_reference(h, args, true, q))) < 1e-12


@pytest.mark.parametrize("wrong", ["transposed", "head_by_seq", "seq_head_by_head"])
def test_descale_pin_catches_wrong_indexing(wrong, monkeypatch):
    """Mistakes planted in the oracle (on the CPU): each one changes the
    result, so the pin above would fail on it."""
    real = A.descale

    def planted(values, kind, i, g):
        v = np.asarray(values, dtype=np.float64)
        if wrong == "transposed" and kind == "seq_head":
            return float(v.reshape(-1)[g * v.shape[0] + i])  # the (b, h_k) array read as (h_k, b)
        if wrong == "head_by_seq" and kind == "head":
            return float(v.reshape(-1)[i % v.size])
        if wrong == "seq_head_by_head" and kind == "seq_head":
            return float(v.reshape(-1)[g])
        return real(values, kind, i, g)

    kind = "head" if wrong == "head_by_seq" else "seq_head"
    h, args, true, q = _descale_case(kind)
    monkeypatch.setattr(A, "descale", planted)
    O, _ = A.decode_step(h, causal=True, quantize=False, **args)
    assert np.max(np.abs(O - _descale_reference(h, args, true, q))) > 1e-3
