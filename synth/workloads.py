"""Seeded workload builder: Q, a paged e4m3 / packed-e2m3 KV cache, block tables.

The five workloads follow the decode shapes the mjolnir-kernel pages describe
(PyPI project page, "What it does" and "fp6 (e2m3) KV in vLLM"; wheel listing
mjolnir/runner.py, ``T5DecodeRunner.run`` for the Q/K/V/scale shapes):

* Q is bf16 drawn from N(0, 1), token-major ``(b*q_len, h_q, d)``.
* K and V are drawn from N(0, 1); selected K channels can be multiplied by 20
  before quantization (outlier channels).
* e4m3 caches use one fp32 scale ``amax / 448`` per tensor, per KV head or per
  (sequence, KV head), computed over the pages that group owns, and torch's
  own float8_e4m3fn cast.
* The sub-byte caches (e2m3, e3m2, e2m1) use static per-(KV head, channel)
  scales ``amax_c / max`` (7.5, 28, 6) from a separate seeded calibration
  draw; 6-bit codes are packed four per three bytes and 4-bit codes two per
  byte, as little-endian bitstreams.
* nvfp4 caches: a per-tensor or per-KV-head fp32 scale ``amax / (6 * 448)``
  (as the e4m3 caches), then per 16-channel block of each row an e4m3 block
  scale (torch's float8_e4m3fn cast of ``amax_block / 6``) and e2m1 codes of
  the values over it; the 8 scale bytes of a row sit in a second pool paged
  like the codes.
* Physical pages are consecutive slices of one seeded permutation of the pool.
  Unused block-table entries and the unused tail slots of each sequence's last
  page hold a poison page (codes of value 448, or 7.5 for e2m3) so that any
  stray read changes the result; unused pool pages hold random bytes.

Bulk values are drawn with ``torch.Generator`` on the target device (so large
workloads never pass through host memory); structure (lengths, permutations,
outlier channels) comes from NumPy's PCG64 so it is identical on every device.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch

E4M3_MAX = 448.0
E2M3_MAX = 7.5
E3M2_MAX = 28.0
E2M1_MAX = 6.0
HEAD_DIM = 128
OUTLIER_GAIN = 20.0
CALIB_TOKENS = 8192

# poison codes: the largest finite magnitude of each format
POISON_E4M3 = 0x7E
POISON_E2M3 = 0x1F
POISON_E3M2 = 0x1F
POISON_E2M1 = 0x7


@dataclass(frozen=True)
class Spec:
    name: str
    b: int
    q_len: int
    h_q: int
    h_k: int
    page_size: int
    layout: str  # "HND" | "NHD"
    kv_format: str  # "e4m3" | "e2m3" | "e3m2" | "e2m1" | "nvfp4"
    scale_kind: str  # "tensor" | "head" | "seq_head" | "channel" (fp6 / e2m1 only)
    lens: tuple = ()  # explicit context lengths (tokens, including the q_len new ones)
    lens_loguniform: tuple = ()  # (lo, hi): draw b lengths floor(exp(U(ln lo, ln hi)))
    k_outliers: int = 0  # outlier K channels per KV head (x20 before quantization)
    causal: bool = True
    slots_override: int = 0  # 0 = automatic split planning
    pool_pages: int = 0  # 0 = round_up(2 * pages needed, 1024)
    extra_bt_cols: int = 2  # block-table columns beyond the longest sequence (poison)
    q_extra_heads: int = 0  # >0: Q is a strided view into a wider (fused-QKV-like) buffer
    tail_nan: bool = False  # unused tail slots of each last page hold NaN codes (e4m3, nvfp4 scales), not poison
    seed: int = 1000
    d: int = HEAD_DIM

    @property
    def h_r(self) -> int:
        return self.h_q // self.h_k

    @property
    def n_q(self) -> int:
        return self.q_len * self.h_r

    @property
    def row_bytes(self) -> int:
        bits = {"e4m3": 8, "e2m3": 6, "e3m2": 6, "e2m1": 4, "nvfp4": 4}[self.kv_format]
        return self.d * bits // 8

    @property
    def scale_row_bytes(self) -> int:
        """Block-scale bytes per row (nvfp4: one e4m3 per 16 channels)."""
        return self.d // 16 if self.kv_format == "nvfp4" else 0


# The five workloads (full size) and the 32k-context target point.
SPECS = {
    "cfg1": Spec("cfg1_b1_L512_p16_hnd_e4m3", b=1, q_len=1, h_q=8, h_k=2, page_size=16, layout="HND",
                 kv_format="e4m3", scale_kind="tensor", lens=(512,), pool_pages=64, extra_bt_cols=0, seed=1001),
    "cfg2": Spec("cfg2_b32_L4096_p16_hnd_e4m3_head", b=32, q_len=1, h_q=32, h_k=8, page_size=16, layout="HND",
                 kv_format="e4m3", scale_kind="head", lens=(4096,) * 32, k_outliers=4, pool_pages=16384, seed=1002),
    "cfg3": Spec("cfg3_b64_ragged1k-32k_p64_nhd_e4m3", b=64, q_len=1, h_q=32, h_k=8, page_size=64, layout="NHD",
                 kv_format="e4m3", scale_kind="tensor", lens_loguniform=(1024, 32768), slots_override=256,
                 seed=1003),
    "cfg4c": Spec("cfg4_b16_q4_L8192_p32_hnd_causal", b=16, q_len=4, h_q=64, h_k=8, page_size=32, layout="HND",
                  kv_format="e4m3", scale_kind="seq_head", lens=(8192,) * 16, causal=True, pool_pages=8192,
                  seed=1004),
    "cfg4n": Spec("cfg4_b16_q4_L8192_p32_hnd_noncausal", b=16, q_len=4, h_q=64, h_k=8, page_size=32, layout="HND",
                  kv_format="e4m3", scale_kind="seq_head", lens=(8192,) * 16, causal=False, pool_pages=8192,
                  seed=1004),
    "cfg5": Spec("cfg5_b4_L131072_p128_hnd_e2m3", b=4, q_len=1, h_q=32, h_k=8, page_size=128, layout="HND",
                 kv_format="e2m3", scale_kind="channel", lens=(131072,) * 4, k_outliers=4, pool_pages=8192,
                 seed=1005),
    "32k": Spec("b64_L32768_p64_nhd_e4m3", b=64, q_len=1, h_q=32, h_k=8, page_size=64, layout="NHD",
                kv_format="e4m3", scale_kind="tensor", lens=(32768,) * 64, seed=1006),
    # the 32k point at batch 16: the split path (several splits per sequence)
    "32k_b16": Spec("b16_L32768_p64_nhd_e4m3", b=16, q_len=1, h_q=32, h_k=8, page_size=64, layout="NHD",
                    kv_format="e4m3", scale_kind="tensor", lens=(32768,) * 16, seed=1007),
    # the fp6 long-context point in the harness's other sub-byte formats
    "cfg5_e3m2": Spec("b4_L131072_p128_hnd_e3m2", b=4, q_len=1, h_q=32, h_k=8, page_size=128, layout="HND",
                      kv_format="e3m2", scale_kind="channel", lens=(131072,) * 4, k_outliers=4, pool_pages=8192,
                      seed=1008),
    "cfg5_e2m1": Spec("b4_L131072_p128_hnd_e2m1", b=4, q_len=1, h_q=32, h_k=8, page_size=128, layout="HND",
                      kv_format="e2m1", scale_kind="channel", lens=(131072,) * 4, k_outliers=4, pool_pages=8192,
                      seed=1009),
    # block-scaled fp4 at the long-context point and at the ragged token-major point
    "cfg5_nvfp4": Spec("b4_L131072_p128_hnd_nvfp4", b=4, q_len=1, h_q=32, h_k=8, page_size=128, layout="HND",
                       kv_format="nvfp4", scale_kind="head", lens=(131072,) * 4, k_outliers=4, pool_pages=8192,
                       seed=1010),
    "cfg3_nvfp4": Spec("b64_ragged1k-32k_p64_nhd_nvfp4", b=64, q_len=1, h_q=32, h_k=8, page_size=64, layout="NHD",
                       kv_format="nvfp4", scale_kind="tensor", lens_loguniform=(1024, 32768), slots_override=256,
                       seed=1011),
    # the packed fp6 and fp4 caches at the ragged token-major point
    "cfg3_e2m3": Spec("b64_ragged1k-32k_p64_nhd_e2m3", b=64, q_len=1, h_q=32, h_k=8, page_size=64, layout="NHD",
                      kv_format="e2m3", scale_kind="channel", lens_loguniform=(1024, 32768), slots_override=256,
                      seed=1012),
    "cfg3_e2m1": Spec("b64_ragged1k-32k_p64_nhd_e2m1", b=64, q_len=1, h_q=32, h_k=8, page_size=64, layout="NHD",
                      kv_format="e2m1", scale_kind="channel", lens_loguniform=(1024, 32768), slots_override=256,
                      seed=1013),
}

# Reduced sizes with the same heads, page size, layout, format and scales: the
# oracle checks every output of these in seconds.  Lengths span several
# 128-token tiles and end in ragged tails.
SMALL = {
    "cfg1": {},
    "cfg2": dict(b=4, lens=(1000, 2048, 777, 1391), pool_pages=0),
    "cfg3": dict(b=6, lens=(), lens_loguniform=(100, 3000), slots_override=24),
    "cfg4c": dict(b=3, lens=(1031, 517, 2000), pool_pages=0),
    "cfg4n": dict(b=3, lens=(1031, 517, 2000), pool_pages=0),
    "cfg5": dict(b=2, lens=(3001, 1290), pool_pages=0),
    "32k": dict(b=3, lens=(2048, 1985, 64), pool_pages=0),
    "32k_b16": dict(b=2, lens=(4096, 3000), pool_pages=0),
    "cfg5_e3m2": dict(b=2, lens=(3001, 1290), pool_pages=0),
    "cfg5_e2m1": dict(b=2, lens=(3001, 1290), pool_pages=0),
    "cfg5_nvfp4": dict(b=2, lens=(3001, 1290), pool_pages=0),
    "cfg3_nvfp4": dict(b=6, lens=(), lens_loguniform=(100, 3000), slots_override=24),
    "cfg3_e2m3": dict(b=6, lens=(), lens_loguniform=(100, 3000), slots_override=24),
    "cfg3_e2m1": dict(b=6, lens=(), lens_loguniform=(100, 3000), slots_override=24),
}


def spec_for(key: str, small: bool = False, **overrides) -> Spec:
    s = SPECS[key]
    if small:
        s = replace(s, name=s.name + "_small", **SMALL[key])
    if overrides:
        s = replace(s, **overrides)
    return s


@dataclass
class Workload:
    spec: Spec
    seq_lens: list  # host ints
    seq_lens_dev: torch.Tensor  # (b,) int32
    block_table: torch.Tensor  # (b, max_blocks) int32
    poison_page: int
    q: torch.Tensor  # (b*q_len, h_q, d) bf16, possibly a strided view
    k_pool: torch.Tensor  # uint8, HND (pages, h_k, P, row) or NHD (pages, P, h_k, row)
    v_pool: torch.Tensor
    k_descale: torch.Tensor  # fp32: (1,), (h_k,) or (b, h_k)
    v_descale: torch.Tensor
    descale_kind: str  # "tensor" | "head" | "seq_head"
    q_mul: torch.Tensor | None  # (h_q, d) fp32
    o_mul: torch.Tensor | None
    k_channel_scale: torch.Tensor | None = None  # (h_k, d) for e2m3
    v_channel_scale: torch.Tensor | None = None
    k_bs_pool: torch.Tensor | None = None  # nvfp4: uint8 block scales, laid out like k_pool with 8-byte rows
    v_bs_pool: torch.Tensor | None = None
    softmax_scale: float = 1.0 / math.sqrt(HEAD_DIM)
    extra: dict = field(default_factory=dict)

    @property
    def num_pages(self) -> int:
        return self.k_pool.shape[0]

    def kv_strides(self):
        """Byte strides (page, slot, head) of the K and V pools."""
        def st(p):
            if self.spec.layout == "HND":
                return (p.stride(0), p.stride(2), p.stride(1))
            return (p.stride(0), p.stride(1), p.stride(2))
        return st(self.k_pool), st(self.v_pool)

    def bs_strides(self):
        """Byte strides (page, slot, head) of the K and V block-scale pools."""
        def st(p):
            if self.spec.layout == "HND":
                return (p.stride(0), p.stride(2), p.stride(1))
            return (p.stride(0), p.stride(1), p.stride(2))
        return st(self.k_bs_pool), st(self.v_bs_pool)

    def kv_bytes(self) -> int:
        """K and V bytes one decode step must read: sum_i L_i * h_k * 2 * row
        (row = codes plus block scales)."""
        s = self.spec
        return int(sum(self.seq_lens)) * s.h_k * 2 * (s.row_bytes + s.scale_row_bytes)

    def host(self, seqs=None) -> dict:
        """NumPy copies for the oracle.  ``seqs`` restricts the copy to the
        pages those sequences use (compact pool, remapped block table), which
        keeps full-size workloads cheap to check on samples."""
        s = self.spec
        bt = self.block_table.cpu().numpy()
        lens = np.asarray(self.seq_lens, dtype=np.int64)
        seqs = list(range(s.b)) if seqs is None else list(seqs)
        nv = self.k_bs_pool is not None
        kbp = vbp = None
        if len(seqs) == s.b and self.num_pages * self.k_pool[0].numel() <= (1 << 30):
            kp, vp, bt_sub = self.k_pool.cpu().numpy(), self.v_pool.cpu().numpy(), bt
            if nv:
                kbp, vbp = self.k_bs_pool.cpu().numpy(), self.v_bs_pool.cpu().numpy()
            bt_sub = bt_sub[seqs]
        else:
            used = []
            for i in seqs:
                used.extend(bt[i, : max(1, -(-int(lens[i]) // s.page_size))].tolist())
            uniq = sorted(set(used))
            remap = {p: j for j, p in enumerate(uniq)}
            idx = torch.tensor(uniq, dtype=torch.long, device=self.k_pool.device)
            kp = self.k_pool.index_select(0, idx).cpu().numpy()
            vp = self.v_pool.index_select(0, idx).cpu().numpy()
            if nv:
                kbp = self.k_bs_pool.index_select(0, idx).cpu().numpy()
                vbp = self.v_bs_pool.index_select(0, idx).cpu().numpy()
            bt_sub = np.zeros((len(seqs), bt.shape[1]), dtype=np.int32)
            for r, i in enumerate(seqs):
                n = max(1, -(-int(lens[i]) // s.page_size))
                bt_sub[r, :n] = [remap[p] for p in bt[i, :n]]
        qd = self.q.float().cpu().numpy().reshape(s.b, s.q_len, s.h_q, s.d)[seqs].reshape(-1, s.h_q, s.d)

        def strides(p):
            st = np.array(p.strides)  # numpy strides of a uint8 array are bytes
            return (st[0], st[2], st[1]) if s.layout == "HND" else (st[0], st[1], st[2])

        kd = self.k_descale.cpu().numpy()
        vd = self.v_descale.cpu().numpy()
        if self.descale_kind == "seq_head":
            kd, vd = kd[seqs], vd[seqs]
        extra = {}
        if nv:
            extra = dict(k_bs_pool=np.ascontiguousarray(kbp).reshape(-1), v_bs_pool=np.ascontiguousarray(vbp).reshape(-1),
                         k_bs_strides=strides(np.ascontiguousarray(kbp)),
                         v_bs_strides=strides(np.ascontiguousarray(vbp)))
        return dict(
            **extra,
            q=np.ascontiguousarray(qd),
            k_pool=np.ascontiguousarray(kp).reshape(-1),
            v_pool=np.ascontiguousarray(vp).reshape(-1),
            k_strides=strides(np.ascontiguousarray(kp)),
            v_strides=strides(np.ascontiguousarray(vp)),
            block_table=np.ascontiguousarray(bt_sub),
            seq_lens=lens[seqs],
            k_descale=kd,
            v_descale=vd,
            descale_kind=self.descale_kind,
            q_mul=None if self.q_mul is None else self.q_mul.cpu().numpy(),
            o_mul=None if self.o_mul is None else self.o_mul.cpu().numpy(),
            softmax_scale=self.softmax_scale,
        )


# ----------------------------------------------------------------------------
# e2m3 cache-write helpers (input preparation only)
# ----------------------------------------------------------------------------
def e2m3_magnitudes() -> list:
    """The 32 non-negative e2m3 values in code order (OCP MX FP6 E2M3)."""
    out = []
    for m in range(32):
        e, man = m >> 3, m & 7
        out.append(man / 8.0 if e == 0 else (1.0 + man / 8.0) * 2.0 ** (e - 1))
    return out


def e3m2_magnitudes() -> list:
    """The 32 non-negative e3m2 values in code order (OCP MX FP6 E3M2)."""
    out = []
    for m in range(32):
        e, man = m >> 2, m & 3
        out.append(man / 4.0 * 0.25 if e == 0 else (1.0 + man / 4.0) * 2.0 ** (e - 3))
    return out


def e2m1_magnitudes() -> list:
    """The 8 non-negative e2m1 values in code order (OCP MX FP4 E2M1)."""
    out = []
    for m in range(8):
        e, man = m >> 1, m & 1
        out.append(man / 2.0 if e == 0 else (1.0 + man / 2.0) * 2.0 ** (e - 1))
    return out


def _encode_table(x: torch.Tensor, mags_list: list, sign_bit: int) -> torch.Tensor:
    """Nearest code of each value of a small sign-magnitude format (clamped to
    its largest magnitude), ties to the even code."""
    mags = torch.tensor(mags_list, dtype=torch.float32, device=x.device)
    n = len(mags_list)
    mids = (mags[1:] + mags[:-1]) * 0.5  # exact in fp32
    a = x.abs().clamp_max(mags_list[-1])
    idx = torch.bucketize(a, mids)  # mids[idx-1] < a <= mids[idx]
    tie = (idx < n - 1) & (a == mids[idx.clamp_max(n - 2)])
    idx = torch.where(tie & (idx % 2 == 1), idx + 1, idx)
    sign = (x < 0) | ((x == 0) & torch.signbit(x))
    return (idx | (sign.to(idx.dtype) << sign_bit)).to(torch.uint8)


def e2m3_encode_table(x: torch.Tensor) -> torch.Tensor:
    """Nearest e2m3 code of each value (clamped to +-7.5), ties to the even code."""
    return _encode_table(x, e2m3_magnitudes(), 5)


def e3m2_encode_table(x: torch.Tensor) -> torch.Tensor:
    return _encode_table(x, e3m2_magnitudes(), 5)


def e2m1_encode_table(x: torch.Tensor) -> torch.Tensor:
    return _encode_table(x, e2m1_magnitudes(), 3)


def pack_codes_4bit(codes: torch.Tensor) -> torch.Tensor:
    """(..., n) 4-bit codes -> (..., n/2) bytes: code 2k in the low nibble of
    byte k, code 2k + 1 in its high nibble (little-endian bitstream)."""
    c = codes.to(torch.int32).reshape(*codes.shape[:-1], codes.shape[-1] // 2, 2)
    return (c[..., 0] | (c[..., 1] << 4)).to(torch.uint8)


# per sub-byte format: (largest magnitude, encoder, packer, poison code)
SUBBYTE = {
    "e2m3": (E2M3_MAX, e2m3_encode_table, lambda c: pack_codes_6bit(c), POISON_E2M3),
    "e3m2": (E3M2_MAX, e3m2_encode_table, lambda c: pack_codes_6bit(c), POISON_E3M2),
    "e2m1": (E2M1_MAX, e2m1_encode_table, lambda c: pack_codes_4bit(c), POISON_E2M1),
}


def nvfp4_encode_blocks(y: torch.Tensor):
    """(..., d) fp32 -> ((..., d/2) e2m1 code bytes, (..., d/16) e4m3 block
    scales): per 16 values, scale = e4m3(min(amax / 6, 448)) by torch's cast,
    codes the nearest e2m1 of y / scale (zero codes under a zero scale)."""
    blk = y.reshape(*y.shape[:-1], y.shape[-1] // 16, 16)
    sc8 = (blk.abs().amax(dim=-1) / 6.0).clamp_max(E4M3_MAX).to(torch.float8_e4m3fn)  # the cast does not saturate
    sv = sc8.to(torch.float32).unsqueeze(-1)
    codes = e2m1_encode_table(torch.where(sv > 0, blk / torch.where(sv > 0, sv, 1.0), 0.0))
    return pack_codes_4bit(codes.reshape(y.shape)), sc8.view(torch.uint8)


def pack_codes_6bit(codes: torch.Tensor) -> torch.Tensor:
    """(..., n) 6-bit codes -> (..., 3n/4) bytes: code k occupies stream bits
    [6k, 6k+6), stream bit 8B+j being bit j of byte B (little-endian)."""
    c = codes.to(torch.int32).reshape(*codes.shape[:-1], codes.shape[-1] // 4, 4)
    w = c[..., 0] | (c[..., 1] << 6) | (c[..., 2] << 12) | (c[..., 3] << 18)
    b = torch.stack([w & 255, (w >> 8) & 255, (w >> 16) & 255], dim=-1)
    return b.to(torch.uint8).reshape(*codes.shape[:-1], codes.shape[-1] * 3 // 4)


# ----------------------------------------------------------------------------
# builder
# ----------------------------------------------------------------------------
def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & 0x7FFFFFFFFFFFFFFF)
    return g


def _randn(shape, device, seed) -> torch.Tensor:
    return torch.randn(shape, generator=_gen(device, seed), device=device, dtype=torch.float32)


def _lens(spec: Spec, rng: np.random.Generator) -> list:
    if spec.lens:
        assert len(spec.lens) == spec.b
        return [int(x) for x in spec.lens]
    lo, hi = spec.lens_loguniform
    u = rng.uniform(math.log(lo), math.log(hi), size=spec.b)
    return [int(max(lo, min(hi, math.floor(math.exp(v))))) for v in u]


def build(spec: Spec, device="cpu") -> Workload:
    device = torch.device(device)
    rng = np.random.default_rng(spec.seed)
    s = spec
    P, h_k, d, row = s.page_size, s.h_k, s.d, s.row_bytes
    lens = _lens(s, rng)
    pages = [max(1, -(-L // P)) for L in lens]
    need = sum(pages)
    gran = 1024 if need >= 1024 else 64
    pool = s.pool_pages or int(math.ceil(2 * need / gran) * gran)
    assert pool >= need + 1, "pool must hold every sequence's pages plus the poison page"
    perm = rng.permutation(pool).astype(np.int64)
    poison = int(perm[need])
    max_blocks = max(pages) + s.extra_bt_cols
    bt = np.full((s.b, max_blocks), poison, dtype=np.int32)
    off = 0
    for i, n in enumerate(pages):
        bt[i, :n] = perm[off: off + n]
        off += n

    # outlier K channels, per KV head
    gain = np.ones((h_k, d), dtype=np.float32)
    for g in range(h_k):
        if s.k_outliers:
            gain[g, rng.choice(d, size=s.k_outliers, replace=False)] = OUTLIER_GAIN
    gain_t = torch.from_numpy(gain).to(device)

    def draw(i: int, side: str) -> torch.Tensor:
        x = _randn((lens[i], h_k, d), device, s.seed * 1_000_003 + 2 * i + (side == "v"))
        return x * gain_t if side == "k" else x

    # pools: random bytes, then the poison page, then each sequence's pages
    shape = (pool, h_k, P, row) if s.layout == "HND" else (pool, P, h_k, row)
    k_pool = torch.randint(0, 256, shape, generator=_gen(device, s.seed + 11), device=device, dtype=torch.uint8)
    v_pool = torch.randint(0, 256, shape, generator=_gen(device, s.seed + 12), device=device, dtype=torch.uint8)
    k_bs = v_bs = None
    srow = s.scale_row_bytes
    if s.kv_format == "e4m3":
        k_pool[poison] = POISON_E4M3
        v_pool[poison] = POISON_E4M3
        # tail slots: the poison code, or e4m3's NaN code S.1111.111
        poison_row = torch.full((row,), 0x7F if s.tail_nan else POISON_E4M3, dtype=torch.uint8, device=device)
    elif s.kv_format == "nvfp4":
        # poison: codes of 6 under scales of 448
        bshape = shape[:-1] + (srow,)
        k_bs = torch.randint(0, 256, bshape, generator=_gen(device, s.seed + 13), device=device, dtype=torch.uint8)
        v_bs = torch.randint(0, 256, bshape, generator=_gen(device, s.seed + 14), device=device, dtype=torch.uint8)
        poison_row = torch.full((row,), POISON_E2M1 * 0x11, dtype=torch.uint8, device=device)
        poison_srow = torch.full((srow,), POISON_E4M3, dtype=torch.uint8, device=device)
        for pool_t, bs_t in ((k_pool, k_bs), (v_pool, v_bs)):
            pool_t[poison] = poison_row
            bs_t[poison] = poison_srow
        if s.tail_nan:  # NaN block scales (S.1111.111) in the tail slots
            poison_srow = torch.full((srow,), 0x7F, dtype=torch.uint8, device=device)
    else:
        fmax, enc_fn, pack_fn, pcode = SUBBYTE[s.kv_format]
        poison_row = pack_fn(torch.full((d,), pcode, dtype=torch.uint8, device=device))
        k_pool[poison] = poison_row
        v_pool[poison] = poison_row

    q_mul = o_mul = kcs = vcs = None
    if s.kv_format in ("e4m3", "nvfp4"):
        # pass 1: amax per (sequence, KV head); nvfp4's second-level scale
        # leaves room for e2m1's 6 times e4m3's 448
        top = E4M3_MAX if s.kv_format == "e4m3" else E2M1_MAX * E4M3_MAX
        amax = torch.zeros(2, s.b, h_k, dtype=torch.float32, device=device)
        for i in range(s.b):
            for j, side in enumerate("kv"):
                if lens[i] > 0:
                    amax[j, i] = draw(i, side).abs().amax(dim=(0, 2))
        if s.scale_kind == "tensor":
            sc = amax.amax(dim=(1, 2)).reshape(2, 1) / top
        elif s.scale_kind == "head":
            sc = amax.amax(dim=1) / top
        elif s.scale_kind == "seq_head":
            sc = torch.where(amax > 0, amax, torch.ones_like(amax)) / top
        else:
            raise ValueError(s.scale_kind)
        k_desc, v_desc = sc[0].contiguous(), sc[1].contiguous()
        kind = s.scale_kind

        def encode(i, side, x):
            scl = k_desc if side == "k" else v_desc
            if kind == "tensor":
                y = x / scl
            elif kind == "head":
                y = x / scl.view(1, h_k, 1)
            else:
                y = x / scl[i].view(1, h_k, 1)
            if s.kv_format == "e4m3":
                return y.to(torch.float8_e4m3fn).view(torch.uint8)
            return nvfp4_encode_blocks(y)
    else:
        assert s.scale_kind == "channel"
        # calibration pass: a separate seeded draw, same outlier channels
        ck = _randn((CALIB_TOKENS, h_k, d), device, s.seed + 1) * gain_t
        cv = _randn((CALIB_TOKENS, h_k, d), device, s.seed + 2)
        kcs = (ck.abs().amax(dim=0) / fmax).contiguous()  # (h_k, d)
        vcs = (cv.abs().amax(dim=0) / fmax).contiguous()
        del ck, cv
        q_mul = kcs.repeat_interleave(s.h_r, dim=0).contiguous()  # (h_q, d)
        o_mul = vcs.repeat_interleave(s.h_r, dim=0).contiguous()
        k_desc = torch.ones(1, dtype=torch.float32, device=device)
        v_desc = torch.ones(1, dtype=torch.float32, device=device)
        kind = "tensor"

        def encode(i, side, x):
            scl = kcs if side == "k" else vcs
            return pack_fn(enc_fn(x / scl.view(1, h_k, d)))

    bt_t = torch.from_numpy(bt).to(device)
    for i in range(s.b):
        n = pages[i]
        idx = bt_t[i, :n].long()
        for side, pool_t in (("k", k_pool), ("v", v_pool)):
            codes = encode(i, side, draw(i, side))  # (L, h_k, row)
            scales = None
            if s.kv_format == "nvfp4":
                codes, scales = codes
            padded = poison_row.view(1, 1, row).expand(n * P, h_k, row).clone()
            padded[: lens[i]] = codes
            paged = padded.view(n, P, h_k, row)
            if s.layout == "HND":
                paged = paged.permute(0, 2, 1, 3)
            pool_t[idx] = paged.contiguous()
            if scales is not None:
                bs_t = k_bs if side == "k" else v_bs
                padded = poison_srow.view(1, 1, srow).expand(n * P, h_k, srow).clone()
                padded[: lens[i]] = scales
                paged = padded.view(n, P, h_k, srow)
                if s.layout == "HND":
                    paged = paged.permute(0, 2, 1, 3)
                bs_t[idx] = paged.contiguous()

    # Q: bf16 N(0,1); optionally a strided view into a wider per-token buffer
    tokens = s.b * s.q_len
    width = s.h_q + s.q_extra_heads
    qfull = _randn((tokens, width, d), device, s.seed + 3).to(torch.bfloat16)
    q = qfull[:, : s.h_q, :]

    return Workload(
        spec=s,
        seq_lens=lens,
        seq_lens_dev=torch.tensor(lens, dtype=torch.int32, device=device),
        block_table=bt_t,
        poison_page=poison,
        q=q,
        k_pool=k_pool,
        v_pool=v_pool,
        k_descale=k_desc,
        v_descale=v_desc,
        descale_kind=kind,
        q_mul=q_mul,
        o_mul=o_mul,
        k_channel_scale=kcs,
        v_channel_scale=vcs,
        k_bs_pool=k_bs,
        v_bs_pool=v_bs,
    )
