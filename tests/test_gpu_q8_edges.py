"""GPU parity for Q8_0 caches at the edges of the block format and of the f16 range.

A Q8_0 block is an f16 scale d and 32 int8 codes, value = code * d ("ik_llama.cpp -mla
flag deep-dive", recommended DeepSeek command combinations: `-ctk q8_0`).  The GPU
computes Q8_0 attention with f16 MFMA operands: each value is f16(code * d), rounded
once and saturated to +-65504, and a bf16 query is converted to f16 with the same
saturation.  These cases put every corner of that contract in front of the whole-output
comparison with the exact fp64 oracle:
  * all-zero blocks (d = 0, codes 0) and d = 0 with nonzero codes;
  * codes -128 and +127 (the quantiser never writes -128);
  * f16-subnormal scales;
  * the largest scale whose values stay finite in f16 (511.75: -128 * 511.75 = -65504);
  * scales past it (516, 1000, 65504), whose values the GPU saturates, placed where
    they cannot move the exact result: in dims where every query is zero (so they never
    enter a score; a key and its value are the same row, so a large value in a scored dim
    would decide the softmax by itself), and there only in cells the mask drops or
    biases to a negligible weight;
  * bf16 queries past the f16 range (1e5, 3e38) and below it (1e-8), in dims where every
    key is zero.
An unsaturated conversion turns each of the large cases into inf * 0 = NaN or inf - inf,
which the finiteness check catches; the rest must meet the usual bar (whole-output
relative L2 <= 5e-3, max |error| <= 2e-2)."""
import numpy as np
import pytest

import oracle
from mla_flash_attention_amd import synth
from tests.gpu_common import assert_parity, run_decode

pytestmark = pytest.mark.gpu

BF16, F16, Q8 = synth.TYPE_BF16, synth.TYPE_F16, synth.TYPE_Q8_0
NB = synth.DK // 32            # 18 blocks per row: 0..15 latent (also V), 16..17 RoPE


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    from mla_flash_attention_amd import binding
    binding.lib()


def _f16(x):
    return int(np.float16(x).view(np.uint16))


def set_block(kv_row, b, d_bits, codes):
    """Write block b of one Q8_0 row (uint8 [612]): d as f16 bits, then 32 int8 codes."""
    kv_row[34 * b:34 * b + 2] = np.array([d_bits], np.uint16).view(np.uint8)
    kv_row[34 * b + 2:34 * b + 34] = np.asarray(codes, np.int8).view(np.uint8)


def edge_problem(q_type, seed):
    p = synth.make_problem(kind="decode", n_seq=2, n_head=128, n_kv=3000, q_type=q_type, kv_type=Q8,
                           seed=seed, mask_kind="runs_bias")
    g = np.random.default_rng(seed)
    kv = p.kv
    n_kv = p.n_kv
    extreme = [_f16(516.0), _f16(1000.0), 0x7BFF]          # |code * d| can pass 65504
    scored = [b for b in range(NB) if b not in (15, 17)]    # blocks 15 and 17 are set below
    for s in range(p.n_seq):
        mask = p.mask[s, 0]
        for j in range(n_kv):
            row = kv[s, j]
            # block 15 (dims 480..511) is zero in every row, so the query may hold
            # anything there; blocks 14 (dims 448..479, also V) and 17 (dims 544..575)
            # of the query are zeroed below, so the keys never score them
            set_block(row, 15, 0, np.zeros(32))
            set_block(row, 17, int(g.choice(extreme)), g.choice([-128, 127, -127, 1, 0], 32))
            kind = j % 7
            if kind == 0:                                     # all-zero block
                set_block(row, int(g.integers(0, 15)), 0, np.zeros(32))
            elif kind == 1:                                   # d = 0, codes nonzero
                set_block(row, int(g.integers(0, 15)), 0, g.integers(-128, 128, 32))
            elif kind == 2:                                   # codes -128 / +127, d normal
                set_block(row, int(g.choice(scored)), _f16(0.02), g.choice([-128, 127], 32))
            elif kind == 3:                                   # f16-subnormal scales
                for b in g.choice(scored, 4, replace=False):
                    set_block(row, int(b), int(g.integers(1, 0x400)), g.integers(-128, 128, 32))
            elif kind == 4:
                # largest finite scale: -128 * 511.75 = -65504 exactly.  In the unscored
                # RoPE block 17; and in one cell per sequence also in the unscored V block
                # 14, kept with a bias of -6, so that ~65504 e^-10 / sum of weights reaches
                # the output on both sides.  (One cell only: f16 probabilities carry 2^-11
                # relative and 2^-25 absolute error, which values of 65504 amplify.)
                set_block(row, 17, 0x5FFF, g.choice([-128, 127], 32))
                if j == 4:
                    set_block(row, 14, 0x5FFF, g.choice([-128, 127], 32))
                    mask[j] = _f16(-6.0)
            elif kind == 5 and mask[j] == synth.F16_NEG_INF:
                # values past the f16 range in every V dim of a dropped cell
                for b in range(15):
                    set_block(row, b, int(g.choice(extreme)), g.choice([-128, 127], 32))
            elif kind == 6:
                # values past the f16 range in the unscored V block of a kept cell whose
                # weight is e^-30 relative: the exact contribution (< 1e-8) is far below the
                # tolerance, while an overflow would give inf or NaN
                set_block(row, 14, int(g.choice(extreme)), g.choice([-128, 127], 32))
                mask[j] = _f16(-30.0)
    # the query: zero in block 17; block 15 holds values past f16's range either way
    qf = np.zeros(32, np.float32)
    qf[:] = g.choice([1e5, -1e5, 3e38, -3e38, 7e4, -65504.0, 1e-8, -3e-8], 32)
    if q_type == F16:
        qf = np.clip(qf, -65504, 65504)
    p.q[..., 480:512] = synth.round_bits(qf, q_type)
    p.q[..., 448:480] = 0
    p.q[..., 544:576] = 0
    return p


@pytest.mark.parametrize("q_type", [BF16, F16])
@pytest.mark.parametrize("sparse", [False, True])
def test_q8_0_edge_blocks(q_type, sparse):
    p = edge_problem(q_type, seed=90 + q_type)
    ref = oracle.attention_problem(p)
    assert np.all(np.isfinite(ref))
    for n_split in (0, 1):
        got, _ = run_decode(p, n_split=n_split, via_compaction=sparse)
        assert_parity(got, ref, f"q8_0 edges q{q_type} sparse={sparse} split{n_split}")


def test_q8_0_saturation_is_the_documented_one():
    """Each Q8_0 value is computed as f16(code * d), rounded once and saturated to
    +-65504: with a single kept cell the output is that cell's V row, so the GPU must
    return exactly those values (and the oracle the exact ones)."""
    p = synth.make_problem(kind="decode", n_seq=1, n_head=16, n_kv=64, q_type=BF16, kv_type=Q8, seed=93,
                           mask_kind="none_kept")
    p.mask[0, 0, 37] = 0
    row = p.kv[0, 37]
    codes = np.tile(np.array([127, -128, 1, -1], np.int8), 8)
    set_block(row, 3, _f16(516.0), codes)                  # 127 * 516 = 65532 -> 65504
    set_block(row, 4, 0x5FFF, codes)                       # exact: -128 * 511.75 = -65504
    got, _ = run_decode(p, n_split=1)
    got = got.reshape(16, 512)

    def f16_saturated(x):          # f16(x) rounded to nearest even, then clamped to +-65504
        with np.errstate(over="ignore"):
            return np.clip(np.asarray(x, np.float64).astype(np.float16).astype(np.float64), -65504, 65504)
    exp3 = f16_saturated(codes.astype(np.float64) * 516.0)
    exp4 = f16_saturated(codes.astype(np.float64) * 511.75)
    assert exp3[0] == 65504 and exp3[1] == -65504 and exp4[1] == -65504
    for h in range(16):
        assert np.array_equal(got[h, 96:128], exp3)
        assert np.array_equal(got[h, 128:160], exp4)
    ref = oracle.attention_problem(p).reshape(16, 512)
    assert np.array_equal(ref[0, 96:128], codes.astype(np.float64) * 516.0)
