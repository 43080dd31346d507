"""Seeded synthetic inputs for MLA flash attention over the latent KV cache.

This module produces the exact bytes that both the HIP path and the CPU oracle
receive.  It holds none of the attention arithmetic: it draws normal values,
rounds them to the storage formats (f16, bf16, Q8_0 blocks) and builds f16
additive masks.  Nothing here imports the oracle or the HIP library.

Storage formats (what the pages fix):
  * a latent cache row is kv_lora_rank 512 + RoPE 64 = 576 values, and with flash
    attention on it is a K-only cache whose first 512 columns serve as V
    ("ik_llama.cpp -mla flag deep-dive", sections "what MLA is" and "the four
    -mla levels");
  * `-ctk q8_0` quantises that cache row to Q8_0 blocks: per 32 values one f16
    scale followed by 32 int8 codes, 34 bytes per block, 18 blocks = 612 bytes a
    row (same page, recommended DeepSeek command combinations);
  * the flash-attention mask is f16, with -inf marking cells that are not kept
    ("baguaai Flash Attention tag page", digest on the f16 FA mask PR).

Recipe: numpy Generator(PCG64(seed*1000 + stream)),
stream 0 = Q, 1 = cache, 2 = mask; values standard_normal(float32), rounded to
nearest-even into f16/bf16, or quantised to Q8_0 with d = amax/127.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

DK = 576           # latent 512 + RoPE 64
DV = 512           # V = first 512 columns of the latent row
QK8_0 = 32         # values per Q8_0 block
Q8_0_BLOCK_BYTES = 34
F16_NEG_INF = 0xFC00

TYPE_F16 = 1
TYPE_BF16 = 2
TYPE_Q8_0 = 3
TYPE_NAMES = {TYPE_F16: "f16", TYPE_BF16: "bf16", TYPE_Q8_0: "q8_0"}
TYPE_IDS = {v: k for k, v in TYPE_NAMES.items()}


def q8_0_row_bytes(dk: int = DK) -> int:
    assert dk % QK8_0 == 0
    return dk // QK8_0 * Q8_0_BLOCK_BYTES


def rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed * 1000 + stream))


# ---------------------------------------------------------------- rounding
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to IEEE binary16 (numpy rounds to nearest even)."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def round_bits(x: np.ndarray, type_id: int) -> np.ndarray:
    if type_id == TYPE_F16:
        return f32_to_f16_bits(x)
    if type_id == TYPE_BF16:
        return f32_to_bf16_bits(x)
    raise ValueError(type_id)


def quantize_q8_0(x: np.ndarray) -> np.ndarray:
    """Quantise rows of float32 values (last axis a multiple of 32) to Q8_0 bytes.

    Per 32-value block: d = amax/127 in fp32, codes q = round-half-away(x * (1/d))
    with the reciprocal in fp32, d stored as f16 (nearest even); d == 0 gives
    all-zero codes.  Both sides read the bytes this returns, so the rounding rule
    here cannot move parity; it only has to be deterministic.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    lead = x.shape[:-1]
    d_model = x.shape[-1]
    assert d_model % QK8_0 == 0
    nb = d_model // QK8_0
    blocks = x.reshape(-1, nb, QK8_0)
    amax = np.max(np.abs(blocks), axis=-1)                     # fp32
    d = (amax / np.float32(127.0)).astype(np.float32)
    with np.errstate(divide="ignore"):
        inv = np.where(d != 0, np.float32(1.0) / d, np.float32(0.0)).astype(np.float32)
    v = (blocks * inv[..., None]).astype(np.float32)
    qv = np.trunc(v.astype(np.float64) + np.copysign(0.5, v.astype(np.float64)))
    qv = np.clip(qv, -127, 127).astype(np.int8)
    out = np.empty((blocks.shape[0], nb, Q8_0_BLOCK_BYTES), dtype=np.uint8)
    out[:, :, 0:2] = f32_to_f16_bits(d).reshape(blocks.shape[0], nb, 1).view(np.uint8)
    out[:, :, 2:] = qv.view(np.uint8)
    return out.reshape(*lead, nb * Q8_0_BLOCK_BYTES)


# ---------------------------------------------------------------- masks
def sparse_runs_mask(n_kv: int, g: np.random.Generator, max_gap: int = 2312,
                     max_run: int = 256) -> np.ndarray:
    """f16 mask bits [n_kv]: alternating gaps of -inf (length U{0..max_gap}) and
    kept runs of 0.0 (length U{1..max_run}); about 10% kept at the defaults."""
    bits = np.full(n_kv, F16_NEG_INF, dtype=np.uint16)
    pos = 0
    while pos < n_kv:
        pos += int(g.integers(0, max_gap + 1))
        run = int(g.integers(1, max_run + 1))
        if pos >= n_kv:
            break
        bits[pos:min(n_kv, pos + run)] = 0
        pos += run
    return bits


# ---------------------------------------------------------------- problems
@dataclasses.dataclass
class Problem:
    """One attention problem, as host bytes.

    q    : uint16 [n_seq][n_tok][n_head][576] (f16 or bf16 bits)
    kv   : uint16 [n_seq or 1][n_kv][576], or uint8 [n_seq or 1][n_kv][612] (Q8_0)
    mask : uint16 [n_seq][n_tok][n_kv] f16 bits, or None
    """
    name: str
    kind: str              # "decode" | "prefill" | "sparse"
    q: np.ndarray
    q_type: int
    kv: np.ndarray
    kv_type: int
    n_seq: int
    n_tok: int
    n_head: int
    n_kv: int
    scale: np.float32
    causal: bool = False
    mask: np.ndarray | None = None
    kv_len: np.ndarray | None = None      # int32 [n_seq] valid cells per sequence
    alibi: np.ndarray | None = None       # float32 [n_head] per-head mask slopes
    sinks: np.ndarray | None = None       # float32 [n_head] per-head sink logits
    softcap: float = 0.0                  # 0 = off

    @property
    def shared_kv(self) -> bool:
        return self.kv.shape[0] == 1 and self.n_seq >= 1 and self.kind == "prefill"

    @property
    def kv_row_bytes(self) -> int:
        return self.kv.shape[-1] * self.kv.itemsize


DEFAULT_SCALE = np.float32(1.0 / math.sqrt(192.0))

# The five workloads: DeepSeek-V2-Lite (16 heads) and V3 (128 heads) head counts,
# 576-wide latent rows, contexts up to 128k cells.
CONFIGS = {
    1: dict(name="C1 decode 1x1x16h n_kv=1024 f16", kind="decode", n_seq=1, n_tok=1,
            n_head=16, n_kv=1024, q_type=TYPE_F16, kv_type=TYPE_F16),
    2: dict(name="C2 decode 4x1x128h n_kv=32768 bf16 split-KV", kind="decode", n_seq=4,
            n_tok=1, n_head=128, n_kv=32768, q_type=TYPE_BF16, kv_type=TYPE_BF16),
    3: dict(name="C3 causal prefill 2048 tok x128h n_kv=4096 bf16", kind="prefill",
            n_seq=1, n_tok=2048, n_head=128, n_kv=4096, q_type=TYPE_BF16,
            kv_type=TYPE_BF16, causal=True),
    4: dict(name="C4 decode 4x1x128h n_kv=65536 Q8_0", kind="decode", n_seq=4, n_tok=1,
            n_head=128, n_kv=65536, q_type=TYPE_BF16, kv_type=TYPE_Q8_0),
    5: dict(name="C5 sparse decode 1x1x128h 131072 cells ~10% kept bf16", kind="sparse",
            n_seq=1, n_tok=1, n_head=128, n_kv=131072, q_type=TYPE_BF16,
            kv_type=TYPE_BF16, sparse=True),
}


def make_problem(kind: str = "decode", n_seq: int = 1, n_tok: int = 1, n_head: int = 16,
                 n_kv: int = 1024, q_type: int = TYPE_BF16, kv_type: int = TYPE_BF16,
                 seed: int = 0, causal: bool = False, sparse: bool = False,
                 mask_kind: str | None = None, q_gain: float = 1.0,
                 scale: float | None = None, name: str = "", dk: int = DK,
                 ragged: bool = False, alibi: bool = False, sinks: bool = False,
                 softcap: float = 0.0) -> Problem:
    """Draw one problem.  `mask_kind`: None, "runs" (sparse runs of kept cells),
    "runs_bias" (runs with finite random biases on kept cells), "random" (iid 50%
    kept with finite biases), "none_kept" (every cell -inf), "distance" (minus the
    distance |pos_t - j| of each cell to the query position, as ALiBi masks carry).
    ragged: valid cells per sequence drawn from U{n_tok..n_kv} (stream 3); alibi:
    per-head slopes 2^(-8(h+1)/n_head); sinks: per-head sink logits 2*N(0,1) (stream 4)."""
    gq, gk, gm = rng(seed, 0), rng(seed, 1), rng(seed, 2)
    qf = gq.standard_normal((n_seq, n_tok, n_head, dk), dtype=np.float32)
    if q_gain != 1.0:
        qf = qf * np.float32(q_gain)
    n_kv_seqs = 1 if kind == "prefill" else n_seq
    kf = gk.standard_normal((n_kv_seqs, n_kv, dk), dtype=np.float32)
    q_bits = round_bits(qf, q_type)
    kv = quantize_q8_0(kf) if kv_type == TYPE_Q8_0 else round_bits(kf, kv_type)
    if (sparse or kind == "sparse") and mask_kind is None:
        mask_kind = "runs"
    kv_len = None
    if ragged:
        kv_len = rng(seed, 3).integers(n_tok, n_kv + 1, n_seq).astype(np.int32)
    if mask_kind == "distance":
        mask = np.empty((n_seq, n_tok, n_kv), dtype=np.uint16)
        for s_ in range(n_seq):
            length = n_kv if kv_len is None else int(kv_len[s_])
            for t in range(n_tok):
                pos = length - n_tok + t
                mask[s_, t] = f32_to_f16_bits(-np.abs(pos - np.arange(n_kv, dtype=np.float32)))
    else:
        mask = make_mask(mask_kind, n_seq, n_tok, n_kv, gm)
    slopes = None
    if alibi:
        slopes = np.exp2(-8.0 * (np.arange(n_head, dtype=np.float64) + 1) / n_head).astype(np.float32)
    sink = None
    if sinks:
        sink = (2.0 * rng(seed, 4).standard_normal(n_head)).astype(np.float32)
    return Problem(name=name or f"{kind} s{n_seq} t{n_tok} h{n_head} kv{n_kv}", kind=kind,
                   q=q_bits, q_type=q_type, kv=kv, kv_type=kv_type, n_seq=n_seq,
                   n_tok=n_tok, n_head=n_head, n_kv=n_kv,
                   scale=np.float32(DEFAULT_SCALE if scale is None else scale),
                   causal=causal, mask=mask, kv_len=kv_len, alibi=slopes, sinks=sink,
                   softcap=float(np.float32(softcap)))


def make_mask(mask_kind: str | None, n_seq: int, n_tok: int, n_kv: int,
              g: np.random.Generator) -> np.ndarray | None:
    if mask_kind is None:
        return None
    out = np.empty((n_seq, n_tok, n_kv), dtype=np.uint16)
    for s in range(n_seq):
        for t in range(n_tok):
            if mask_kind in ("runs", "runs_bias"):
                row = sparse_runs_mask(n_kv, g)
                if mask_kind == "runs_bias":
                    keep = row == 0
                    bias = f32_to_f16_bits(g.uniform(-2.0, 2.0, n_kv).astype(np.float32))
                    row = np.where(keep, bias, row).astype(np.uint16)
            elif mask_kind == "random":
                keep = g.random(n_kv) < 0.5
                bias = f32_to_f16_bits(g.uniform(-3.0, 3.0, n_kv).astype(np.float32))
                row = np.where(keep, bias, np.uint16(F16_NEG_INF)).astype(np.uint16)
            elif mask_kind == "none_kept":
                row = np.full(n_kv, F16_NEG_INF, dtype=np.uint16)
            else:
                raise ValueError(mask_kind)
            out[s, t] = row
    return out


def make_config(cfg_id: int, seed: int | None = None, **overrides) -> Problem:
    """Workload `cfg_id` (1..5) at full size, seed defaults to the config id."""
    spec = dict(CONFIGS[cfg_id])
    spec.update(overrides)
    return make_problem(seed=cfg_id if seed is None else seed, **spec)


# ---------------------------------------------------------------- per-head (non-absorbed) shape
MHA_DK = 192       # 128 per-head dims + 64 RoPE
MHA_DV = 128


@dataclasses.dataclass
class MhaProblem:
    """Per-head attention with separate K and V (bits): q [n_tok][n_head][192],
    k [n_kv][n_head][192], v [n_kv][n_head][128]; mask [n_tok][n_kv] f16 bits or None."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    q_type: int
    kv_type: int
    n_tok: int
    n_head: int
    n_kv: int
    scale: np.float32
    causal: bool = True
    mask: np.ndarray | None = None


def make_mha_problem(n_tok: int, n_head: int, n_kv: int, q_type: int = TYPE_BF16, kv_type: int = TYPE_BF16,
                     seed: int = 0, causal: bool = True, mask_kind: str | None = None,
                     scale: float | None = None) -> MhaProblem:
    """Streams: 0 = Q, 1 = K, 5 = V, 2 = mask; N(0,1) values rounded to the storage type;
    scale defaults to 1/sqrt(192) in fp32."""
    q = round_bits(rng(seed, 0).standard_normal((n_tok, n_head, MHA_DK), dtype=np.float32), q_type)
    k = round_bits(rng(seed, 1).standard_normal((n_kv, n_head, MHA_DK), dtype=np.float32), kv_type)
    v = round_bits(rng(seed, 5).standard_normal((n_kv, n_head, MHA_DV), dtype=np.float32), kv_type)
    mask = None if mask_kind is None else make_mask(mask_kind, 1, n_tok, n_kv, rng(seed, 2))[0]
    return MhaProblem(q=q, k=k, v=v, q_type=q_type, kv_type=kv_type, n_tok=n_tok, n_head=n_head, n_kv=n_kv,
                      scale=np.float32(DEFAULT_SCALE if scale is None else scale), causal=causal, mask=mask)


# ---------------------------------------------------------------- absorbed projections
QK_NOPE = 128      # per-head query/key dims without RoPE
QK_ROPE = 64       # RoPE dims (shared key part in the cache row)
V_HEAD = 128       # per-head value dims


@dataclasses.dataclass
class AbsorbedProblem:
    """Latent attention with the per-head projections either side (bits):
    q_nope [n_seq][n_tok][n_head][128], q_pe [..][64], w_uk [n_head][512][128] (latent from
    key dims), w_uv [n_head][128][512] (value dims from latent), cache as in Problem."""
    q_nope: np.ndarray
    q_pe: np.ndarray
    w_uk: np.ndarray
    w_uv: np.ndarray
    q_type: int
    kv: np.ndarray
    kv_type: int
    n_seq: int
    n_tok: int
    n_head: int
    n_kv: int
    scale: np.float32
    causal: bool = False
    mask: np.ndarray | None = None
    kv_len: np.ndarray | None = None


def make_absorbed_problem(n_seq: int, n_tok: int, n_head: int, n_kv: int, q_type: int = TYPE_BF16,
                          kv_type: int = TYPE_BF16, seed: int = 0, causal: bool = False,
                          mask_kind: str | None = None, ragged: bool = False,
                          scale: float | None = None) -> AbsorbedProblem:
    """Cache, mask and lengths as make_problem (streams 1, 2, 3); q_nope stream 6, q_pe
    stream 7, W_UK stream 8 (N(0, 1/128): latent queries of unit variance), W_UV stream 9
    (N(0, 1/512)); all rounded to q_type.  Scale defaults to 1/sqrt(192), the per-head
    key width the projections stand for."""
    base = make_problem(kind="decode", n_seq=n_seq, n_tok=n_tok, n_head=n_head, n_kv=n_kv, q_type=q_type,
                        kv_type=kv_type, seed=seed, causal=causal, mask_kind=mask_kind, ragged=ragged)
    qn = rng(seed, 6).standard_normal((n_seq, n_tok, n_head, QK_NOPE), dtype=np.float32)
    qp = rng(seed, 7).standard_normal((n_seq, n_tok, n_head, QK_ROPE), dtype=np.float32)
    wk = rng(seed, 8).standard_normal((n_head, DV, QK_NOPE), dtype=np.float32) * np.float32(1 / np.sqrt(QK_NOPE))
    wv = rng(seed, 9).standard_normal((n_head, V_HEAD, DV), dtype=np.float32) * np.float32(1 / np.sqrt(DV))
    return AbsorbedProblem(q_nope=round_bits(qn, q_type), q_pe=round_bits(qp, q_type), w_uk=round_bits(wk, q_type),
                           w_uv=round_bits(wv, q_type), q_type=q_type, kv=base.kv, kv_type=kv_type, n_seq=n_seq,
                           n_tok=n_tok, n_head=n_head, n_kv=n_kv,
                           scale=np.float32(1 / np.sqrt(QK_NOPE + QK_ROPE) if scale is None else scale),
                           causal=causal, mask=base.mask, kv_len=base.kv_len)
