// attn.hip -- fused MLA flash attention over the latent cache for gfx950 (CDNA4).
//
// One kernel family serves dense decode, split-KV decode, sparse (indexed) decode and
// causal chunked prefill.  What it computes follows the pages:
//   * scores are built key-tile by key-tile with an online softmax: a running max m
//     and running sum l per query head; when a tile raises m, everything accumulated
//     before is corrected by exp(m_old - m_new) ("Vulkan backend fused Flash
//     Attention: DeepSeek MLA local inference", sections 2.1-2.2);
//   * the cache row is 512 latent + 64 RoPE values; V is the first 512 columns of the
//     same row and one latent head serves every query head ("ik_llama.cpp -mla flag
//     deep-dive", sections "what MLA is" and "the four -mla levels");
//   * the f16 mask is additive and -inf drops a cell ("baguaai Flash Attention tag
//     page", f16 mask digest); the sparse path attends only to the compacted rows
//     ("llama.cpp Vulkan backend adds sparse Flash Attention for quantized K/V");
//   * `-ctk q8_0` caches are dequantised in the kernel ("ik_llama.cpp -mla flag
//     deep-dive", recommended command combinations).
//
// Design (gfx950-specific, not from the pages):
//   * 64-key tiles of 576-wide rows are copied HBM -> LDS with global_load_lds_dwordx4
//     (no VGPR staging), double-buffered.  A tile is stored as two areas: the 1024
//     latent bytes of each row at a 1120-byte pitch, and the 128 RoPE bytes of each row
//     packed 8 rows per KiB with an XOR swizzle.  Every copy then moves one contiguous
//     KiB of LDS with all 64 lanes, and both LDS read patterns below are bank-conflict
//     free.  Q8_0 tiles are DMA'd raw and dequantised LDS -> LDS to f16.
//   * Q.K^T runs as S^T = K.Q^T on v_mfma_f32_16x16x32_{bf16,f16}: A = 16 keys from
//     LDS, B = 16 heads of Q held in VGPRs for the whole kernel.  The accumulator
//     layout (lane = head, 4 keys per lane) is exactly the A-operand layout P.V needs
//     with heads as M, so P never round-trips through LDS.
//   * P.V takes its B operand straight from the row-major tile with
//     ds_read_b64_tr_b16 (LDS transpose read), so no transposed copy of V exists.
//   * Lazy rescale: m only moves when a tile's max exceeds it by more than 2^8, so
//     the 512-wide O accumulators are rarely touched by the softmax.
//   * A workgroup is NW waves = (NW/WK) head sets x WK key halves; key halves merge
//     their (m, l, O) through LDS at the end, which halves split-KV partial traffic.
//     Each wave of a pair merges and writes half of the 512 output columns.
#include <type_traits>

#include "mla_fa_internal.h"

namespace mlafa {
namespace {

#include "device_common.h"

constexpr int kSub = 32;                                  // keys per compute sub-tile
// LDS tile layout.  Latent area: row r's bytes 0..1023 (dims 0..511, also V) at
// r * kVRow.  The pitch 1120 (= 96 mod 256) keeps the S^T reads (16 rows, one 16-byte
// column) and the transpose reads (4 rows x 32 bytes per 16 lanes) bank-conflict free
// on gfx950 (measured: 1088 or 1072 halves both rates, and the unpadded 1152-byte row
// quarters the S^T rate).  RoPE area: row r's bytes 1024..1151 (dims 512..575), 16-byte
// chunk c stored at kRopeOff + 128 r + 16 (c ^ ((r >> 1) & 7)); 16 consecutive rows
// reading one chunk then hit 16 distinct 16-byte bank groups.
constexpr int kVRow = 1120;
constexpr int kRopeOff = kTileKeys * kVRow;               // 71,680
constexpr int kTileBytes = kRopeOff + kTileKeys * 128;    // 79,872
__device__ __forceinline__ int rope_slot(int r, int c) { return 128 * r + 16 * (c ^ ((r >> 1) & 7)); }
constexpr int kQ8TileBytes = kTileKeys * kQ8RowBytes;     // 39,168
constexpr float kRescaleThresh = 8.0f;                    // log2 units

// An index-list entry clamped into [0, n_kv): a list with entries out of range gives an
// unspecified result but never a read outside the cache.
__device__ __forceinline__ int clamp_row(int v, int64_t n_kv) {
    const int hi = (int)(n_kv - 1);
    return v < 0 ? 0 : (v > hi ? hi : v);
}

// ---------------------------------------------------------------------------------
// Length-proportional split plan (Ragged with budget > 0).  One whole wave computes it,
// lane l holding rows l + 64 i: wave 0 of every attention workgroup, from the same
// lengths, so no workgroup waits for another; the merge reads the row table the first
// workgroup leaves in the workspace.
constexpr int kRaggedPer = kRaggedRows / 64;

// End of row r's range (keys, or index-list positions), clamped as the row clamps it.
__device__ __forceinline__ int64_t ragged_extent(const Ragged &g, int r) {
    int64_t e;
    if (g.count) {
        e = g.count[r];
    } else {
        int64_t len = g.kv_len[r / g.n_tok];
        len = len < 0 ? 0 : (len > g.n_kv ? g.n_kv : len);
        e = g.causal ? len - g.n_tok + r % g.n_tok + 1 : len;
    }
    return e < 0 ? 0 : (e > g.n_kv ? g.n_kv : e);
}

struct RaggedPlan {
    int pieces[kRaggedPer];    // pieces of rows lane + 64 i
    int chunk;                 // tiles per piece (C), wave-uniform
    int nper;                  // row blocks of 64 in use, wave-uniform
};

// Sum over the 64 lanes, in every lane: DPP rotations within each 16-lane row, then the
// two cross-row swaps (VALU only; no LDS round trip).
__device__ __forceinline__ int wave_sum_i32(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, false);   // row_ror:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x124, 0xF, 0xF, false);   // row_ror:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x122, 0xF, 0xF, false);   // row_ror:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x121, 0xF, 0xF, false);   // row_ror:1
    auto s32 = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    x = (int)s32[0] + (int)s32[1];
    auto s16 = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return (int)s16[0] + (int)s16[1];
}
__device__ __forceinline__ int wave_max_i32(int x) {
    x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, false));
    x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x124, 0xF, 0xF, false));
    x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x122, 0xF, 0xF, false));
    x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x121, 0xF, 0xF, false));
    auto s32 = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    x = max((int)s32[0], (int)s32[1]);
    auto s16 = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return max((int)s16[0], (int)s16[1]);
}

// ceil(t / d) for 0 <= t, d < 2^26 with rd = 1 / d in double: the rounded quotient is
// within 2^-26 of t / d, so its ceiling is exact except where t / d is an integer k and
// the product lands just above k; the one check corrects that.
__device__ __forceinline__ int ceil_div_small(int t, int d, double rd) {
    const int q = (int)__builtin_ceil((double)t * rd);
    return q > 0 && (q - 1) * d >= t ? q - 1 : q;
}

// C = the smallest chunk (in tiles) with sum_r ceil(tiles_r / C) <= budget.  It lies in
// [ceil(T / B), ceil(T / (B - n))] (T tiles in all, n non-empty rows, B the budget: each
// ceil adds less than one piece per row), and C = the longest row always fits (B >= rows),
// so a bisection over that range, a few steps in practice, finds it.
__device__ RaggedPlan ragged_plan(const Ragged &g) {
    const int lane = threadIdx.x & 63;
    RaggedPlan p;
    p.nper = (g.rows + 63) >> 6;
    int t[kRaggedPer];
    int thi = 0, tlo = 0, nz = 0, mx = 0;      // the tile total as 2^16 thi + tlo (no overflow)
#pragma unroll
    for (int i = 0; i < kRaggedPer; ++i) {
        const int r = lane + 64 * i;
        t[i] = i < p.nper && r < g.rows ? (int)((ragged_extent(g, r) + kTileKeys - 1) / kTileKeys) : 0;
        thi += t[i] >> 16;
        tlo += t[i] & 0xFFFF;
        nz += t[i] > 0;
        mx = t[i] > mx ? t[i] : mx;
    }
    const long long tot = ((long long)__builtin_amdgcn_readfirstlane(wave_sum_i32(thi)) << 16) +
                          __builtin_amdgcn_readfirstlane(wave_sum_i32(tlo));
    nz = __builtin_amdgcn_readfirstlane(wave_sum_i32(nz));
    mx = __builtin_amdgcn_readfirstlane(wave_max_i32(mx));
    int lo = 1, hi = 1;
    if (tot > 0) {
        const long long b = g.budget;
        lo = (int)((tot + b - 1) / b);
        hi = mx;
        if (b > nz) {
            const long long h2 = (tot + (b - nz) - 1) / (b - nz);
            if (h2 < hi) hi = (int)h2;
        } else {
            lo = mx;                                  // one piece per non-empty row
        }
        lo = lo < 1 ? 1 : (lo > hi ? hi : lo);
    }
    while (lo < hi) {                                 // (lo, hi wave-uniform)
        const int mid = (lo + hi) >> 1;
        const double rd = 1.0 / mid;
        int c = 0;
#pragma unroll
        for (int i = 0; i < kRaggedPer; ++i)
            if (i < p.nper) c += ceil_div_small(t[i], mid, rd);
        if (__builtin_amdgcn_readfirstlane(wave_sum_i32(c)) <= g.budget) hi = mid;
        else lo = mid + 1;
    }
    p.chunk = lo;
    const double rd = 1.0 / lo;
#pragma unroll
    for (int i = 0; i < kRaggedPer; ++i) p.pieces[i] = i < p.nper ? ceil_div_small(t[i], lo, rd) : 0;
    return p;
}

// Inclusive sum of x over lanes 0 .. lane.
__device__ __forceinline__ int wave_incl_scan(int x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    return x;
}

// Row and piece of the plan's piece number k; row = -1 when k is past the last piece.
__device__ __forceinline__ void ragged_find(const RaggedPlan &p, int k, int &row, int &piece) {
    int carry = 0;
    row = -1;
    piece = 0;
#pragma unroll
    for (int i = 0; i < kRaggedPer; ++i) {
        if (i >= p.nper) break;
        const int incl = wave_incl_scan(p.pieces[i]) + carry;
        const int excl = incl - p.pieces[i];
        const unsigned long long hit = __builtin_amdgcn_ballot_w64(k >= excl && k < incl);
        if (hit) {
            const int l = __builtin_ctzll(hit);
            row = 64 * i + l;
            piece = k - __builtin_amdgcn_readlane(excl, l);
            break;
        }
        carry = __builtin_amdgcn_readlane(incl, 63);
    }
}

// The plan's row table (ragged_table_off) lives in the workspace's tail after the
// partials; the first workgroup of the attention launch writes it and the merges read it.
__device__ __forceinline__ void ragged_write_table(const RaggedPlan &p, int32_t *tab, int rows) {
    const int lane = threadIdx.x & 63;
    int carry = 0;
#pragma unroll
    for (int i = 0; i < kRaggedPer; ++i) {
        if (i >= p.nper) break;
        const int incl = wave_incl_scan(p.pieces[i]) + carry;
        const int r = lane + 64 * i;
        if (r < rows) tab[r] = (incl - p.pieces[i]) | (p.pieces[i] << 16);
        carry = __builtin_amdgcn_readlane(incl, 63);
    }
}

// ---------------------------------------------------------------------------------
// The attention kernel.  NW waves, each owning MB blocks of 16 heads; WK waves share
// one head set and split every 64-key tile between them (WK = 2: keys 0..31 /
// 32..63).  Heads per workgroup = NW / WK * 16 * MB.  IDX: sparse path (rows gathered
// through the index list).  At MB = 2 a wave holds Q (144 VGPRs) and O (256) for 32
// heads, so the kernel runs one wave per SIMD.
template <int MB, int NW, int WK, int KIND, bool IDX>
__global__ void __launch_bounds__(NW * 64, 1) attn_kernel(AttnArgs a) {
    constexpr int kHS = NW / WK;                     // head sets per workgroup
    constexpr int kHPW = kHS * 16 * MB;              // heads per workgroup
    constexpr bool kQ8 = KIND == KV_Q8;
    // A copy stage holds one tile's rows, then the tile's 64 f16 mask values, then the 64
    // index-list entries of the tile after it.  LDS copies of 2-byte elements land in
    // 4-byte slots (value zero-extended), so the mask area is 256 B as well.  16-bit
    // caches copy straight into two such stages; Q8_0 copies raw rows into two stages
    // and dequantises into one f16 tile.
    constexpr int kRowArea = kQ8 ? kQ8TileBytes : kTileBytes;
    constexpr int kMaskOff = kRowArea, kIdxOff = kRowArea + 256;
    constexpr int kStageBytes = kRowArea + 256 + 256;
    constexpr int kF16Off = 2 * kStageBytes;                       // Q8_0 only
    constexpr int kLdsBytes = 2 * kStageBytes + (kQ8 ? kTileBytes : 0);
    static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
    static_assert(kTileKeys % NW == 0 && 8 % NW == 0, "copy split over waves");
    // key-half exchange area per head set and 16-head block: [2 waves][16 blocks][64 lanes]
    // f32x4 of O, then m[2][16] and l[2][16]
    constexpr int kXfer = 2 * 16 * 64 * 4 + 64;   // floats
    static_assert(WK == 1 || kHS * MB * kXfer * 4 <= kLdsBytes, "key-half merge fits in LDS");
    __shared__ __attribute__((aligned(1024))) unsigned char lds[kLdsBytes];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hs = wave / WK;                         // head block of this wave
    const int kp = wave % WK;                         // key half of this wave
    const int g = lane >> 4;                          // 16-lane group
    const int l16 = lane & 15;

    // ---- which (row, split, head group) this workgroup owns.  Workgroups x and x+8 are
    // dispatched to the same XCD (round-robin over 8): they get one key range and
    // different head groups, so they share its L2.
    int hg, split, row;
    int64_t slot;                                     // partial slot of (split, row)
    int64_t kend, chunk = a.split_chunk;
    const int n_rows = a.n_seq * a.n_tok;
    {
        const int x = blockIdx.x;
        int xr = x;                                   // key range number
        hg = 0;
        if (a.head_groups > 1) {
            hg = (x >> 3) % a.head_groups;
            xr = (x & 7) + 8 * (x / (8 * a.head_groups));
        }
        if (a.ragged.budget) {
            // length-proportional plan: key range xr is the plan's piece number xr, which
            // is also its partial slot.  Wave 0 computes the plan and hands (row, piece,
            // chunk) over in stage 1's index area, which no copy reaches before the main
            // loop's first barrier; the first workgroup also writes the merge's row table.
            int *hand = reinterpret_cast<int *>(lds + kStageBytes + kIdxOff);
            if (wave == 0) {
                const RaggedPlan p = ragged_plan(a.ragged);
                int r, j;
                ragged_find(p, xr, r, j);
                if (lane == 0) {
                    hand[0] = r;
                    hand[1] = j;
                    hand[2] = p.chunk;
                }
                if (x == 0)
                    ragged_write_table(p, reinterpret_cast<int32_t *>(a.ws + ragged_table_off(a.n_split, n_rows, a.n_head)),
                                       a.ragged.rows);
            }
            __syncthreads();
            row = hand[0];
            split = hand[1];
            chunk = (int64_t)hand[2] * kTileKeys;
            if (row < 0) return;
            kend = ragged_extent(a.ragged, row);
            slot = xr;
        } else {
            split = xr;
            if (split >= a.n_split) return;
            const int row_lin = (int)blockIdx.y + a.row_base;
            const int t = a.n_tok - 1 - row_lin % a.n_tok;   // longest causal rows first
            row = row_lin / a.n_tok * a.n_tok + t;
            slot = (int64_t)split * n_rows + row;
        }
    }
    const int s_idx = row / a.n_tok;
    const int t_idx = row % a.n_tok;
    const uint8_t *kvs = a.kv + (int64_t)s_idx * a.kv_seq_stride;
    const uint16_t *mrow = a.mask ? a.mask + (int64_t)s_idx * a.mask_seq_stride +
                                        (int64_t)t_idx * a.mask_tok_stride
                                  : nullptr;
    const int32_t *irow = IDX ? a.kv_idx + (int64_t)s_idx * a.idx_seq_stride + (int64_t)t_idx * a.idx_tok_stride
                              : nullptr;
    if (a.ragged.budget) {
        // kend and chunk come from the plan
    } else if constexpr (IDX) {
        const int64_t c = a.kv_idx_count[row];          // one count per (sequence, token) row
        kend = c < 0 ? 0 : (c > a.n_kv ? a.n_kv : c);
        chunk = (kend + a.n_split - 1) / a.n_split;
        chunk = (chunk + kTileKeys - 1) / kTileKeys * kTileKeys;
        if (chunk == 0) chunk = kTileKeys;
    } else if (a.kv_len) {
        // per-sequence valid length; the split chunk follows the row's own range
        int64_t len = a.kv_len[s_idx];
        len = len < 0 ? 0 : (len > a.n_kv ? a.n_kv : len);
        kend = a.causal ? len - a.n_tok + t_idx + 1 : len;
        if (kend < 0) kend = 0;
        chunk = (kend + a.n_split - 1) / a.n_split;
        chunk = (chunk + kTileKeys - 1) / kTileKeys * kTileKeys;
        if (chunk == 0) chunk = kTileKeys;
    } else {
        kend = a.causal ? a.n_kv - a.n_tok + t_idx + 1 : a.n_kv;
    }
    const int64_t k0 = (int64_t)split * chunk;
    const int64_t k1 = k0 + chunk < kend ? k0 + chunk : kend;
    const int n_tiles = k1 > k0 ? (int)((k1 - k0 + kTileKeys - 1) / kTileKeys) : 0;

    // ---- Q of this wave's heads, resident in VGPRs: B operand of S^T = K.Q^T.  With two
    // key-half waves per head set (WK = 2) both need the same Q: the workgroup copies its
    // heads' Q rows once into LDS (the area the second tile lands in later; for Q8_0 the
    // f16 tile) and each wave reads its rows at the first iteration.  Otherwise each wave
    // loads its rows directly.
    const int h_base = hg * kHPW + hs * 16 * MB;
    constexpr bool kQviaLds = WK == 2 && MB == 1 && !kQ8;   // (Q8_0: the extra live range spills)
    constexpr int kQOff = kQ8 ? kF16Off : kStageBytes;
    static_assert(!kQviaLds || (kHPW * kRowBytes16 <= (kQ8 ? kTileBytes : kStageBytes) &&
                                (kHPW * kRowBytes16) % (1024 * NW) == 0), "Q staging area");
    u32x4 qreg[MB][18];
    auto q_fix = [&](u32x4 v, bool ok) __attribute__((always_inline)) {
        if (!ok) v = u32x4{0, 0, 0, 0};
        if constexpr (kQ8) {
            if (a.q_bf16) {   // bf16 -> f16 for the f16 MFMA, saturated to the f16 range
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    v[e] = pack_f16x2(sat_f16(bf16_bits_to_f32(v[e] & 0xFFFFu)), sat_f16(bf16_bits_to_f32(v[e] >> 16)));
            }
        }
        return v;
    };
    if constexpr (kQviaLds) {
        if (n_tiles > 0) {
            // rows of heads hg*kHPW .. +kHPW-1, contiguous in Q; absent heads re-read the last
            // row (and are zeroed when read back)
            const int h0 = hg * kHPW;
            const int nh = a.n_head - h0 < kHPW ? a.n_head - h0 : kHPW;
            const uint8_t *qb = reinterpret_cast<const uint8_t *>(a.q + ((int64_t)row * a.n_head + h0) * kDK);
#pragma unroll
            for (int j = 0; j < kHPW * kRowBytes16 / (1024 * NW); ++j) {
                const int chunk = wave + j * NW;
                const int o = chunk * 1024 + lane * 16;
                int hl = o / kRowBytes16;
                const int inrow = o - hl * kRowBytes16;
                hl = hl < nh ? hl : nh - 1;
                __builtin_amdgcn_global_load_lds((const void *)(qb + hl * kRowBytes16 + inrow),
                                                 (LDS_PTR(void))(lds + kQOff + chunk * 1024), 16, 0, 0);
            }
        }
    } else {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int head = h_base + mb * 16 + l16;
            const bool ok = head < a.n_head;
            const u32x4 *qp = reinterpret_cast<const u32x4 *>(
                a.q + ((int64_t)row * a.n_head + (ok ? head : a.n_head - 1)) * kDK + 8 * g);
#pragma unroll
            for (int s = 0; s < 18; ++s) qreg[mb][s] = q_fix(qp[4 * s], ok);
        }
    }

    // ---- online-softmax state, per 16-head block mb (per lane: head l16);
    // o[mb][nb]: heads 4g..4g+3 of block mb, dv columns 16nb + l16
    float m_run[MB], l_run[MB];
    f32x4 o[MB][32];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        m_run[mb] = -INFINITY;
        l_run[mb] = 0.f;
#pragma unroll
        for (int nb = 0; nb < 32; ++nb) o[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // ALiBi slope of this lane's head (scaled to log2 units), per 16-head block
    float slope_l2[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int head = h_base + mb * 16 + l16;
        slope_l2[mb] = a.alibi && head < a.n_head ? a.alibi[head] * kLog2e : kLog2e;
    }

    // ---- per-lane LDS read offsets (relative to a sub-tile), tile-invariant
    // S^T A operand: key row (kb*16 + l16), dims 32*s + 8*g .. +7 (byte 64*s + 16*g);
    // steps s = 16, 17 (RoPE dims) read chunk 4*(s-16) + g of the swizzled RoPE area
    // (the swizzle depends on the row only through bits 1..3, which kb*16 and the
    // sub-tile's 32-row offset leave unchanged).
    const int qk_off = l16 * kVRow + 16 * g;
    const int rope_off0 = rope_slot(l16, g), rope_off1 = rope_slot(l16, 4 + g);
    // P.V B operand via transpose read: lane 16G + j reads row 4G + j/4 (+16 for the
    // upper 16 keys), columns 16*nb + 4*(j%4) .. +3 (byte 32*nb + 8*(j%4)).
    const int tr_off = (4 * g + (l16 >> 2)) * kVRow + 8 * (lane & 3);

    // ---- first tile's index entries (later tiles' entries arrive by LDS copy)
    int idx0 = 0;
    if constexpr (IDX) {
        int64_t pos = k0 + lane;
        if (pos >= k1) pos = k1 - 1;
        if (n_tiles > 0) idx0 = clamp_row(irow[pos], a.n_kv);
    }

    // Copy tile `it` into stage `dst` (HBM -> LDS; raw bytes for Q8_0) together with its
    // mask values, and the index entries of tile `it + 1` after it.  Index entries of
    // tile `it` come from `idx_src` (the previous stage's index area, or idx0 for the
    // first tile).  Every copy is an LDS-DMA load: the loop holds no register results of
    // global loads, so the only memory wait is the explicit one at the top of the loop.
    auto issue_tile = [&](int it, unsigned char *__restrict__ dst, const unsigned char *__restrict__ idx_src)
        __attribute__((always_inline)) {
        const int64_t kt = k0 + (int64_t)it * kTileKeys;
        const int last = (int)((k1 - kt) < kTileKeys ? (k1 - kt) : kTileKeys) - 1;  // last valid row
        int ln = lane;
        asm volatile("" : "+v"(ln));
        int my_idx = 0;                                    // cache row of list position kt + lane
        if constexpr (IDX)
            my_idx = it == 0 ? idx0 : clamp_row(reinterpret_cast<const int *>(idx_src + kIdxOff)[ln], a.n_kv);
        if (mrow) {
            const int r = ln < last ? ln : last;
            const int64_t col = IDX ? (int64_t)shfl_int(my_idx, r) : kt + r;
            __builtin_amdgcn_global_load_lds((const void *)(mrow + col), (LDS_PTR(void))(dst + kMaskOff), 2, 0, 0);
        }
        const uint8_t *tbase = IDX ? kvs : kvs + kt * a.kv_row_stride;
        if constexpr (!kQ8) {
            // Latent copies: one per row, lane l moving bytes 16 l .. 16 l + 15 of the
            // row; the row address is wave-uniform, so a copy costs scalar work only.
            // RoPE copies: copy q fills the RoPE slots of rows 8q .. 8q + 7 (lane l: row
            // 8q + l/8, slot l%8 holding chunk (l%8) ^ swizzle).  Rows past the range
            // re-read the last valid row.
            const int voff = ln * 16;
            // A full tile of a packed cache (row stride 1152) needs no clamping and only
            // 32-bit offsets; other tiles clamp rows past the range and scale by the stride.
            const bool contiguous = !IDX && a.kv_row_stride == kRowBytes16 && last == kTileKeys - 1;
            if (contiguous) {
#pragma unroll
                for (int j = 0; j < kTileKeys / NW; ++j) {
                    const int r = wave + j * NW;
                    __builtin_amdgcn_global_load_lds((const void *)(tbase + (uint32_t)(r * kRowBytes16 + voff)),
                                                     (LDS_PTR(void))(dst + r * kVRow), 16, 0, 0);
                }
#pragma unroll
                for (int j = 0; j < 8 / NW; ++j) {
                    const int q = wave + j * NW;
                    const int r = 8 * q + (ln >> 3);
                    const int chunk = (ln & 7) ^ ((r >> 1) & 7);
                    __builtin_amdgcn_global_load_lds(
                        (const void *)(tbase + (uint32_t)(r * kRowBytes16 + 1024 + 16 * chunk)),
                        (LDS_PTR(void))(dst + kRopeOff + q * 1024), 16, 0, 0);
                }
            } else {
#pragma unroll
            for (int j = 0; j < kTileKeys / NW; ++j) {
                const int r = wave + j * NW;                   // tile row (wave-uniform)
                const int rc = r < last ? r : last;
                const uint8_t *rowp;
                if constexpr (IDX)
                    rowp = tbase + (int64_t)__builtin_amdgcn_readlane(my_idx, rc) * a.kv_row_stride;
                else
                    rowp = tbase + (int64_t)rc * a.kv_row_stride;
                __builtin_amdgcn_global_load_lds((const void *)(rowp + voff), (LDS_PTR(void))(dst + r * kVRow),
                                                 16, 0, 0);
            }
#pragma unroll
            for (int j = 0; j < 8 / NW; ++j) {
                const int q = wave + j * NW;
                const int r = 8 * q + (ln >> 3);
                const int rc = r < last ? r : last;
                const int chunk = (ln & 7) ^ ((r >> 1) & 7);
                const uint8_t *src;
                if constexpr (IDX)
                    src = tbase + (int64_t)shfl_int(my_idx, rc) * a.kv_row_stride;
                else
                    src = tbase + (int64_t)rc * a.kv_row_stride;
                __builtin_amdgcn_global_load_lds((const void *)(src + 1024 + 16 * chunk),
                                                 (LDS_PTR(void))(dst + kRopeOff + q * 1024), 16, 0, 0);
            }
            }
        } else {
            // raw Q8_0 rows of 612 bytes, packed back to back (153 dwords each)
            constexpr int kDw = kQ8TileBytes / 4;              // 9792 = 153 * 64
            constexpr int kBlocks = kDw / 64;                  // 153 wave-wide 256 B copies
            // A full tile of a packed cache (row stride 612) is one contiguous block in
            // memory too: copy it without splitting dwords into (row, column).
            const bool contiguous = !IDX && a.kv_row_stride == kQ8RowBytes && last == kTileKeys - 1;
            if (contiguous && (reinterpret_cast<uintptr_t>(tbase) & 15) == 0) {
                // 16-byte copies: 38 KiB blocks and one 256-byte tail, a quarter of the
                // copy instructions of the 4-byte form below
                constexpr int kKiB = kQ8TileBytes / 1024;
                static_assert(kQ8TileBytes - kKiB * 1024 == 256, "one 256-byte tail");
#pragma unroll
                for (int j = 0; j < (kKiB + NW - 1) / NW; ++j) {
                    const int blk = wave + j * NW;
                    if (blk < kKiB)
                        __builtin_amdgcn_global_load_lds((const void *)(tbase + (uint32_t)(blk * 1024 + ln * 16)),
                                                         (LDS_PTR(void))(dst + blk * 1024), 16, 0, 0);
                }
                if (wave == NW - 1)
                    __builtin_amdgcn_global_load_lds((const void *)(tbase + (uint32_t)(kKiB * 1024 + ln * 4)),
                                                     (LDS_PTR(void))(dst + kKiB * 1024), 4, 0, 0);
            } else if (contiguous) {
#pragma unroll
                for (int j = 0; j < (kBlocks + NW - 1) / NW; ++j) {
                    const int blk = wave + j * NW;
                    if (blk < kBlocks)
                        __builtin_amdgcn_global_load_lds((const void *)(tbase + (uint32_t)(blk * 256 + ln * 4)),
                                                         (LDS_PTR(void))(dst + blk * 256), 4, 0, 0);
                }
            } else
#pragma unroll
            for (int j = 0; j < (kBlocks + NW - 1) / NW; ++j) {
                const int blk = wave + j * NW;
                if (blk < kBlocks) {
                    const int dw = blk * 64 + ln;
                    int r = dw / (kQ8RowBytes / 4);
                    const int c = dw - r * (kQ8RowBytes / 4);
                    r = r < last ? r : last;
                    const uint8_t *src;
                    if constexpr (IDX)
                        src = tbase + (int64_t)shfl_int(my_idx, r) * a.kv_row_stride + c * 4;
                    else
                        // 32-bit offset within the tile: the host bounds the row stride
                        // by 2^26 bytes, so 63 rows + one row never wrap
                        src = tbase + (uint32_t)(r * (uint32_t)a.kv_row_stride + c * 4);
                    __builtin_amdgcn_global_load_lds((const void *)src, (LDS_PTR(void))(dst + blk * 256), 4, 0, 0);
                }
            }
        }
        if constexpr (IDX) {                               // index entries of tile it + 1
            int64_t pos = kt + kTileKeys + ln;
            if (pos >= k1) pos = k1 - 1;
            __builtin_amdgcn_global_load_lds((const void *)(irow + pos), (LDS_PTR(void))(dst + kIdxOff), 4, 0, 0);
        }
    };

    // The same copies of a 16-bit tile, issued one at a time: with eight waves the copies
    // of tile it+1 are spread over the Q.K^T steps of tile it instead of issued as one
    // burst at the top of the step.  LDS-DMA copies pass the memory pipeline at ~30
    // cycles per KiB, so a burst of a whole tile (72 copies per CU) held the second wave
    // of every SIMD at its copy issue for ~2k cycles while its MFMAs waited.  Copy j of a
    // wave: latent row wave + NW j (j < kTileKeys / NW), else the RoPE slots of rows
    // 8q .. 8q + 7, q = wave + NW (j - kTileKeys / NW).  Row addresses are clamped as in
    // issue_tile (a no-op for full tiles) and computed in scalar registers.
    constexpr int kCopies = (kTileKeys + 8) / NW;          // copies per wave and tile
    struct TileSrc {
        const uint8_t *base;
        int64_t kt;
        int last, my_idx;
    };
    auto tile_src = [&](int it, const unsigned char *idx_src) __attribute__((always_inline)) {
        TileSrc t;
        t.kt = k0 + (int64_t)it * kTileKeys;
        t.last = (int)((k1 - t.kt) < kTileKeys ? (k1 - t.kt) : kTileKeys) - 1;
        t.my_idx = 0;
        if constexpr (IDX)
            t.my_idx = it == 0 ? idx0 : clamp_row(reinterpret_cast<const int *>(idx_src + kIdxOff)[lane], a.n_kv);
        t.base = IDX ? kvs : kvs + t.kt * a.kv_row_stride;
        return t;
    };
    auto copy_aux = [&](const TileSrc &t, unsigned char *__restrict__ dst) __attribute__((always_inline)) {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        if (mrow) {
            const int r = ln < t.last ? ln : t.last;
            const int64_t col = IDX ? (int64_t)shfl_int(t.my_idx, r) : t.kt + r;
            __builtin_amdgcn_global_load_lds((const void *)(mrow + col), (LDS_PTR(void))(dst + kMaskOff), 2, 0, 0);
        }
        if constexpr (IDX) {                               // index entries of the tile after it
            int64_t pos = t.kt + kTileKeys + ln;
            if (pos >= k1) pos = k1 - 1;
            __builtin_amdgcn_global_load_lds((const void *)(irow + pos), (LDS_PTR(void))(dst + kIdxOff), 4, 0, 0);
        }
    };
    auto copy_one = [&](const TileSrc &t, int j, unsigned char *__restrict__ dst) __attribute__((always_inline)) {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        if (j < kTileKeys / NW) {
            const int r = wave + j * NW;
            const int rc = r < t.last ? r : t.last;
            const int64_t ri = IDX ? (int64_t)__builtin_amdgcn_readlane(t.my_idx, rc) : (int64_t)rc;
            const uint8_t *rowp = t.base + ri * a.kv_row_stride;
            __builtin_amdgcn_global_load_lds((const void *)(rowp + (uint32_t)(ln * 16)),
                                             (LDS_PTR(void))(dst + r * kVRow), 16, 0, 0);
        } else {
            const int q = wave + (j - kTileKeys / NW) * NW;
            const int r = 8 * q + (ln >> 3);
            const int rc = r < t.last ? r : t.last;
            const int chunk = (ln & 7) ^ ((r >> 1) & 7);
            const int64_t ri = IDX ? (int64_t)shfl_int(t.my_idx, rc) : (int64_t)rc;
            __builtin_amdgcn_global_load_lds((const void *)(t.base + ri * a.kv_row_stride + 1024 + 16 * chunk),
                                             (LDS_PTR(void))(dst + kRopeOff + q * 1024), 16, 0, 0);
        }
    };

    // Dequantise a raw Q8_0 stage into the f16 tile (the 16-bit tile layout).  One task
    // = one 34-byte block of one row: f16 scale d at byte 0, 32 int8 codes after it;
    // value = code * d, computed exactly in fp32 (8-bit code x 11-bit d) and rounded
    // once to f16.  Blocks are 2-byte aligned; 9 dwords cover one at either phase
    // (the last block of the last row ends exactly at the end of the raw stage).
    auto dequant_tile = [&](const unsigned char *raw, unsigned char *f16tile) __attribute__((always_inline)) {
        // Lane l converts row l, wave w blocks w, w + NW, ...: the lanes of one read are a
        // row (612 B = 153 dwords, odd mod 64 banks) apart, so every read is conflict-free.
        // A code c becomes u = c + 128 (flip the sign bit); one v_perm builds the f16 pair
        // (1024 + u0, 1024 + u1), and (x - 1152) * d in packed f16 gives (c0 d, c1 d): the
        // subtraction is exact and the product is rounded once, as code * d to f16 is.
        // |code * d| <= 128 * 511.75 = 65504 whenever |d| < 512, so only blocks with a
        // larger scale can leave the f16 range; those (rare) lanes saturate their values
        // to +-65504 instead of becoming infinite.
#pragma clang fp contract(off)
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        const unsigned *rw = reinterpret_cast<const unsigned *>(raw);
        const int r = threadIdx.x & 63;
        // (Issuing the reads of two blocks before converting either measured 4% slower on
        // the Q8_0 decode: the second block's registers spill.)
#pragma unroll 1
        for (int b = threadIdx.x >> 6; b < 18; b += NW) {                // (wave-uniform)
            unsigned w[9];
            const int dw0 = (r * kQ8RowBytes + 34 * b) >> 2;
#pragma unroll
            for (int i = 0; i < 9; ++i) w[i] = rw[dw0 + i];
            const bool odd = (b & 1) != 0;          // block starts mid-dword (34 b = 2 mod 4)
            const unsigned dbits = odd ? (w[0] >> 16) : (w[0] & 0xFFFFu);
            const h2 dd = __builtin_bit_cast(h2, dbits | (dbits << 16));
            const h2 off = h2{(_Float16)1152.f, (_Float16)1152.f};
            // |d| >= 512 (or not finite) in any lane of the wave: the saturating form (a
            // wave-uniform choice between two copies of the conversion)
            auto convert = [&](auto satc) __attribute__((always_inline)) {
                constexpr bool kSat = decltype(satc)::value;
#pragma unroll
                for (int c = 0; c < 4; ++c) {                        // 8 values -> 16 B chunk
                    unsigned pk[4];
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int i = 2 * c + h;                     // code dword i of the block
                        const unsigned code = odd ? w[i + 1] : __builtin_amdgcn_alignbyte(w[i + 1], w[i], 2);
                        const unsigned u = code ^ 0x80808080u;       // code + 128 per byte
                        const h2 x01 = __builtin_bit_cast(h2, __builtin_amdgcn_perm(u, 0x64646464u, 0x00050004u));
                        const h2 x23 = __builtin_bit_cast(h2, __builtin_amdgcn_perm(u, 0x64646464u, 0x00070006u));
                        h2 v01 = (x01 - off) * dd, v23 = (x23 - off) * dd;
                        if constexpr (kSat) {
                            v01 = sat_f16x2(v01);
                            v23 = sat_f16x2(v23);
                        }
                        pk[2 * h] = __builtin_bit_cast(unsigned, v01);
                        pk[2 * h + 1] = __builtin_bit_cast(unsigned, v23);
                    }
                    const int lc = 4 * b + c;                        // 16-byte chunk of the row
                    unsigned char *dp = lc < 64 ? f16tile + r * kVRow + 16 * lc
                                                : f16tile + kRopeOff + rope_slot(r, lc - 64);
                    *reinterpret_cast<u32x4 *>(dp) = u32x4{pk[0], pk[1], pk[2], pk[3]};
                }
            };
            if (__builtin_amdgcn_ballot_w64((dbits & 0x7FFFu) >= 0x6000u)) convert(std::true_type{});
            else convert(std::false_type{});
        }
    };

    // One 32-key sub-tile: keys sub0..sub0+31 of the tile that starts at key kt.
    // LDS operands are loaded kQkD / kPvD steps ahead of the MFMAs that use them, and a
    // scheduling fence closes every step, so at most a few operands are in flight.
    constexpr int kQkD = 2, kPvD = 3;
    // hook(s) runs after the MFMAs of Q.K^T step s (copies placed among the steps).
    auto compute_sub = [&](const unsigned char *stage, const unsigned char *mask_lds, int64_t kt, int sub0,
                           auto &&hook) __attribute__((always_inline)) {
        const unsigned char *sb = stage + sub0 * kVRow;
        const unsigned char *rb = stage + kRopeOff + sub0 * 128;
        // S^T = K . Q^T: A = 16 keys x 32 dims from LDS (two 16-key blocks), B = Q
        f32x4 sacc[2][MB];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) sacc[kb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
        u32x4 ka[kQkD + 1][2];
        auto load_k = [&](int s, u32x4 *dst) __attribute__((always_inline)) {
            if (s < 16) {
                const int off = qk_off + 64 * s;
                dst[0] = *reinterpret_cast<const u32x4 *>(sb + off);
                dst[1] = *reinterpret_cast<const u32x4 *>(sb + off + 16 * kVRow);
            } else {
                const int off = s == 16 ? rope_off0 : rope_off1;
                dst[0] = *reinterpret_cast<const u32x4 *>(rb + off);
                dst[1] = *reinterpret_cast<const u32x4 *>(rb + off + 16 * 128);
            }
        };
#pragma unroll
        for (int s = 0; s < kQkD; ++s) load_k(s, ka[s]);
#pragma unroll
        for (int s = 0; s < 18; ++s) {
            if (s + kQkD < 18) load_k(s + kQkD, ka[(s + kQkD) % (kQkD + 1)]);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    sacc[kb][mb] = mfma16x16x32<KIND>(ka[s % (kQkD + 1)][kb], qreg[mb][s], sacc[kb][mb]);
            hook(s);
            __builtin_amdgcn_sched_barrier(0);
        }
        // Scores in log2 units for this lane's 8 keys: i < 4: key sub0 + 4g + i; i >= 4: key
        // sub0 + 16 + 4g + (i - 4).  The mask bias and the range check are applied only when
        // present (uniform branches: most sub-tiles have neither).
        const int64_t rem64 = k1 - kt - sub0;              // keys of this sub-tile in range
        u32x4 pa[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            float tv[8];
            if (a.cap_in != 0.f) {
                // logit softcap: cap * tanh(scale * dot / cap), tanh(y) = 1 - 2 / (e^(2y) + 1)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float e2y = __builtin_amdgcn_exp2f(sacc[i >> 2][mb][i & 3] * a.cap_in * (2.f * kLog2e));
                    tv[i] = a.cap_out * (1.f - 2.f * __builtin_amdgcn_rcpf(e2y + 1.f));
                }
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) tv[i] = sacc[i >> 2][mb][i & 3] * a.scale_log2;
            }
            if (mrow) {
                const unsigned *mls = reinterpret_cast<const unsigned *>(mask_lds);
                const u32x4 mk[2] = {*reinterpret_cast<const u32x4 *>(mls + sub0 + 4 * g),
                                     *reinterpret_cast<const u32x4 *>(mls + sub0 + 16 + 4 * g)};
                if (a.alibi) {   // slope * mask value for kept cells; -inf stays -inf
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const unsigned short mbits = (unsigned short)(mk[i >> 2][i & 3] & 0xFFFFu);
                        tv[i] += mbits == 0xFC00u ? -INFINITY : f16_bits_to_f32(mbits) * slope_l2[mb];
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i)   // key k's mask: low half of dword k
                        tv[i] += f16_bits_to_f32((unsigned short)(mk[i >> 2][i & 3] & 0xFFFFu)) * kLog2e;
                }
            }
            if (rem64 < kSub) {
                const int rem = (int)rem64;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    if (16 * (i >> 2) + 4 * g + (i & 3) >= rem) tv[i] = -INFINITY;
            }
            float mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < 8; ++i) mx = fmaxf(mx, tv[i]);
            mx = wave_max_groups(mx);
            const bool need = mx > m_run[mb] + kRescaleThresh;
            if (__builtin_amdgcn_ballot_w64(need)) {
                const float alpha = need ? __builtin_amdgcn_exp2f(m_run[mb] - mx) : 1.f;
                if (need) m_run[mb] = mx;
                l_run[mb] *= alpha;
                float ar[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) ar[r] = shfl_f(alpha, 4 * g + r);
#pragma unroll
                for (int nb = 0; nb < 32; ++nb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[mb][nb][r] *= ar[r];
            }
            const float m_use = m_run[mb] == -INFINITY ? 0.f : m_run[mb];
            float p[8], ps = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                p[i] = __builtin_amdgcn_exp2f(tv[i] - m_use);
                ps += p[i];
            }
            l_run[mb] += ps;
            pa[mb] = u32x4{pack_p<KIND>(p[0], p[1]), pack_p<KIND>(p[2], p[3]),
                           pack_p<KIND>(p[4], p[5]), pack_p<KIND>(p[6], p[7])};
        }
        // O += P . V, V = columns 0..511 of the same rows, transposed on the LDS read
        u32x4 vb[kPvD + 1];
        auto load_v = [&](int nb) __attribute__((always_inline)) -> u32x4 {
            const int off = tr_off + 32 * nb;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_PTR(s16x4))(sb + off));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_PTR(s16x4))(sb + off + 16 * kVRow));
            const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
            return u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
        };
#pragma unroll
        for (int nb = 0; nb < kPvD; ++nb) vb[nb] = load_v(nb);
#pragma unroll
        for (int nb = 0; nb < 32; ++nb) {
            if (nb + kPvD < 32) vb[(nb + kPvD) % (kPvD + 1)] = load_v(nb + kPvD);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) o[mb][nb] = mfma16x16x32<KIND>(pa[mb], vb[nb % (kPvD + 1)], o[mb][nb]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // One loop step: start copying tile `it + 1` into `next`, then compute tile `it`
    // from `cur`.  The pointers are restrict-qualified: within a step the copy targets
    // and the stage being read never overlap, which lets the compiler keep the copies
    // in flight across the LDS reads (without it, every LDS transpose read would wait
    // for all outstanding copies).  Ordering between steps is explicit: wait for this
    // wave's copies, then a barrier, at the top of every iteration.
    auto step16 = [&](int it, unsigned char *__restrict__ next, const unsigned char *__restrict__ cur)
        __attribute__((always_inline)) {
        // With eight waves in key halves, the copies of tile it+1 ride on the Q.K^T steps
        // (measured on decode: kernel -3 to -7%).  The 128-head prefill shape keeps the
        // burst: spread there it ran 2.7% slower.
        constexpr bool kSpread = NW == 8 && WK == 2;
        static_assert(!kSpread || 2 * kCopies <= 18, "one copy every other Q.K^T step");
        const bool spread = kSpread && it >= 0 && it + 1 < n_tiles;
        if (it + 1 < n_tiles && !spread) issue_tile(it + 1, next, cur);
        if (it < 0) return;
        const int64_t kt = k0 + (int64_t)it * kTileKeys;
        const TileSrc t = tile_src(spread ? it + 1 : it, cur);
        if (spread) copy_aux(t, next);
#pragma unroll 1
        for (int sub = kp; sub < 2; sub += WK)
            compute_sub(cur, cur + kMaskOff, kt, sub * kSub, [&](int s) __attribute__((always_inline)) {
                if (spread && sub == kp && (s & 1) && (s >> 1) < kCopies) copy_one(t, s >> 1, next);
            });
    };
    auto stepq8 = [&](int it, unsigned char *__restrict__ next, const unsigned char *__restrict__ cur,
                      unsigned char *__restrict__ f16tile) __attribute__((always_inline)) {
        // (The Q8_0 copies stay one burst: spread over the Q.K^T steps they made the
        // compiler spill a Q register inside the loop, and the kernel ran 6% slower.)
        if (it + 1 < n_tiles) issue_tile(it + 1, next, cur);
        if (it < 0) return;
        dequant_tile(cur, f16tile);
        // publish the f16 tile: this wave's LDS writes done, then a plain barrier (a full
        // __syncthreads would also wait for the next tile's copy, which is still in flight)
        __builtin_amdgcn_s_waitcnt(0xC07F);            // lgkmcnt(0), vmcnt/expcnt untouched
        __builtin_amdgcn_s_barrier();
        const int64_t kt = k0 + (int64_t)it * kTileKeys;
#pragma unroll 1
        for (int sub = kp; sub < 2; sub += WK) compute_sub(f16tile, cur + kMaskOff, kt, sub * kSub, [](int) {});
    };

    // ---- main loop: one barrier per tile for 16-bit caches (it publishes tile `it`
    // and frees the other stage), two for Q8_0 (raw copy landed / f16 tile written).
    // Iteration -1 only issues tile 0, so that every copy comes from the same inlined
    // step (one set of alias scopes for the compiler to reason about).
    for (int it = -1; it < n_tiles; ++it) {
        if (it >= 0) {
            wait_vm0();
            __syncthreads();
        }
        if constexpr (kQviaLds) {
            if (it == 0) {   // Q landed with tile 0: read this wave's rows before tile 1 overwrites them
                const int hl = hs * 16 + l16;
                const bool ok = h_base + l16 < a.n_head;
                const unsigned char *qr = lds + kQOff + hl * kRowBytes16 + 16 * g;
#pragma unroll
                for (int s = 0; s < 18; ++s) qreg[0][s] = q_fix(*reinterpret_cast<const u32x4 *>(qr + 64 * s), ok);
                lds_barrier();
            }
        }
        // one inlined copy of the step with computed stage pointers (two copies
        // selected by parity would double the register footprint)
        unsigned char *next = lds + ((it + 1) & 1) * kStageBytes;
        const unsigned char *cur = lds + (it & 1) * kStageBytes;
        if constexpr (kQ8) stepq8(it, next, cur, lds + kF16Off);
        else step16(it, next, cur);
    }

#pragma unroll
    for (int mb = 0; mb < MB; ++mb) l_run[mb] = wave_sum_groups(l_run[mb]);   // lane groups' sums

    // ---- merge the two key halves of each head set through LDS.  Wave kp keeps dv column
    // blocks 16 kp .. 16 kp + 15: it hands the partner's 16 blocks over (16-byte LDS writes),
    // takes the partner's copy of its own 16, and both waves write half of the output.
    // (The register array O is only ever indexed with constants: the half is a template
    // argument of the merge step, selected by a wave-uniform branch.)
    if constexpr (WK == 2) {
        __syncthreads();                                   // tiles no longer needed
        float *xs = reinterpret_cast<float *>(lds) + hs * MB * kXfer;
        auto merge_half = [&](auto kpc) __attribute__((always_inline)) {
            constexpr int K = decltype(kpc)::value, P = 1 - K;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                f32x4 *xo = reinterpret_cast<f32x4 *>(xs + mb * kXfer);
                float *xm = xs + mb * kXfer + 2 * 16 * 64 * 4;
#pragma unroll
                for (int j = 0; j < 16; ++j) xo[(K * 16 + j) * 64 + lane] = o[mb][16 * P + j];
                if (lane < 16) {
                    xm[K * 16 + lane] = m_run[mb];
                    xm[32 + K * 16 + lane] = l_run[mb];
                }
            }
            __syncthreads();
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const f32x4 *xo = reinterpret_cast<const f32x4 *>(xs + mb * kXfer);
                const float *xm = xs + mb * kXfer + 2 * 16 * 64 * 4;
                const float m2 = xm[P * 16 + l16], l2 = xm[32 + P * 16 + l16];
                const float mn = fmaxf(m_run[mb], m2);
                const float a1 = mn == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[mb] - mn);
                const float a2 = mn == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m2 - mn);
                l_run[mb] = a1 * l_run[mb] + a2 * l2;
                m_run[mb] = mn;
                f32x4 a1r, a2r;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    a1r[r] = shfl_f(a1, 4 * g + r);
                    a2r[r] = shfl_f(a2, 4 * g + r);
                }
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    o[mb][16 * K + j] = a1r * o[mb][16 * K + j] + a2r * xo[(P * 16 + j) * 64 + lane];
            }
        };
        if (kp == 0) merge_half(std::integral_constant<int, 0>{});
        else merge_half(std::integral_constant<int, 1>{});
    }
    // dv column block nb is written by this wave (with key halves: the half it merged)
    auto owns = [&](int nb) __attribute__((always_inline)) { return WK == 1 || (nb >> 4) == kp; };

    // ---- write the final output (n_split == 1) or this split's partial
    if (a.n_split == 1) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            float lt = l_run[mb];
            if (a.sinks && m_run[mb] != -INFINITY) {   // the sink joins the normaliser
                const int head = h_base + mb * 16 + l16;
                if (head < a.n_head) lt += __builtin_amdgcn_exp2f(a.sinks[head] * kLog2e - m_run[mb]);
            }
            const float inv = l_run[mb] > 0.f ? 1.f / lt : 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float ir = shfl_f(inv, 4 * g + r);
                const int head = h_base + mb * 16 + 4 * g + r;
                if (head < a.n_head) {
                    float *op = a.out + ((int64_t)row * a.n_head + head) * kDV + l16;
#pragma unroll
                    for (int nb = 0; nb < 32; ++nb)
                        if (owns(nb)) op[16 * nb] = o[mb][nb][r] * ir;
                }
            }
        }
    } else {
        // this split's partial: m, l, and per 256-column half of O/l a scale and the
        // scaled values in f16 (the layout partial_bytes describes)
        const int64_t RH = (int64_t)n_rows * a.n_head;
        float *wm = a.ws;
        float *wl = wm + (int64_t)a.n_split * RH;
        float *wsc = wl + (int64_t)a.n_split * RH;                       // [split][row, head][half]
        uint16_t *wo = reinterpret_cast<uint16_t *>(wsc + 2 * (int64_t)a.n_split * RH);
        const int64_t base = slot * a.n_head;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int head_l = h_base + mb * 16 + l16;
            if (kp == 0 && lane < 16 && head_l < a.n_head) {   // both key halves hold the merged m, l
                wm[base + head_l] = m_run[mb];
                wl[base + head_l] = l_run[mb];
            }
            if (n_tiles > 0) {              // an empty split leaves O unread by the merge
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    if (WK == 2 && hf != kp) continue;            // the other wave's half
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float mx = 0.f;
#pragma unroll
                        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, fabsf(o[mb][16 * hf + j][r]));
                        const int e = partial_exp(group16_max(mx));
                        const float sc = __builtin_amdgcn_ldexpf(1.f, 15 - e);
                        const int head = h_base + mb * 16 + 4 * g + r;
                        if (head < a.n_head) {
                            uint16_t *op = wo + (base + head) * kDV + 256 * hf + l16;
#pragma unroll
                            for (int j = 0; j < 16; ++j)
                                op[16 * j] = (uint16_t)pack_f16x2(o[mb][16 * hf + j][r] * sc, 0.f);
                            if (l16 == 0) wsc[(base + head) * 2 + hf] = __builtin_amdgcn_ldexpf(1.f, e - 15);
                        }
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------------
// The pair kernel (16-bit caches).  A set of 32 heads is served by a pair of waves that
// split the cache row between them: wave d = 0 scores dims 0..287 and accumulates dv
// columns 0..255, wave d = 1 dims 288..575 and dv 256..511.  Every K or V byte a wave
// reads from LDS then feeds 32 heads instead of 16, which halves LDS read traffic per
// MFMA, while the wave still holds Q and O for only 32 x 288 and 32 x 256 values.  The
// pair exchanges two things per stage through LDS: the partial scores of the partner's
// 16 heads after Q.K^T, and the probabilities P of its own 16 heads after the online
// softmax, which wave d runs for heads 16d .. 16d+15 of the set.
//
// Stages are 32 keys.  A 3-slot LDS ring holds stage n (scored in this iteration),
// stage n-1 (its values accumulated in this iteration, so that the softmax of stage n
// and P.V of stage n-1 are independent and can interleave) and stage n+1 (being
// copied).  Two barriers per iteration: X publishes the copied stage and the previous
// softmax results, Y publishes the partial scores.
constexpr int kPK = 32;                                   // keys per stage
constexpr int kPSlots = 3;
constexpr int kPRopeOff = kPK * kVRow;                    // 35,840
constexpr int kPMaskOff = kPRopeOff + kPK * 128;          // 39,936
constexpr int kPIdxOff = kPMaskOff + 256;
constexpr int kPStageBytes = kPIdxOff + 256;              // 40,448
// Exchange area of one pair: partial scores [wave][kb][lane] 16 B, P [stage parity][wave]
// [lane] 16 B, rescale factors [wave][16 heads], rescale flags [wave].
constexpr int kXS = 0, kXP = 4096, kXA = 8192, kXF = 8320, kXBytes = 8448;

template <int NP, int KIND, bool IDX>
__global__ void __launch_bounds__(NP * 128, 1) attn_pair_kernel(AttnArgs a) {
    constexpr int NW = 2 * NP;
    constexpr int kHPW = 32 * NP;
    constexpr int kXOff = kPSlots * kPStageBytes;
    constexpr int kLdsBytes = kXOff + NP * kXBytes;
    static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
    static_assert(kPK % NW == 0 && NW >= kPK / 8, "copy split over waves");
    __shared__ __attribute__((aligned(1024))) unsigned char lds[kLdsBytes];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int pr = wave >> 1;                         // head set of this wave
    const int d = wave & 1;                           // half of the row (and softmax head block)
    const int g = lane >> 4;
    const int l16 = lane & 15;

    int hg, split;
    if (a.head_groups > 1) {
        const int x = blockIdx.x;
        hg = (x >> 3) % a.head_groups;
        split = (x & 7) + 8 * (x / (8 * a.head_groups));
    } else {
        hg = 0;
        split = blockIdx.x;
    }
    if (split >= a.n_split) return;
    const int n_rows = a.n_seq * a.n_tok;
    const int row_lin = (int)blockIdx.y + a.row_base;
    const int s_idx = row_lin / a.n_tok;
    const int t_idx = a.n_tok - 1 - row_lin % a.n_tok;
    const int row = s_idx * a.n_tok + t_idx;
    const uint8_t *kvs = a.kv + (int64_t)s_idx * a.kv_seq_stride;
    const uint16_t *mrow = a.mask ? a.mask + (int64_t)s_idx * a.mask_seq_stride +
                                        (int64_t)t_idx * a.mask_tok_stride
                                  : nullptr;
    const int32_t *irow = IDX ? a.kv_idx + (int64_t)s_idx * a.idx_seq_stride + (int64_t)t_idx * a.idx_tok_stride
                              : nullptr;
    int64_t kend, chunk = a.split_chunk;
    if constexpr (IDX) {
        const int64_t c = a.kv_idx_count[row];          // one count per (sequence, token) row
        kend = c < 0 ? 0 : (c > a.n_kv ? a.n_kv : c);
        chunk = (kend + a.n_split - 1) / a.n_split;
        chunk = (chunk + kTileKeys - 1) / kTileKeys * kTileKeys;
        if (chunk == 0) chunk = kTileKeys;
    } else {
        kend = a.causal ? a.n_kv - a.n_tok + t_idx + 1 : a.n_kv;
    }
    const int64_t k0 = (int64_t)split * chunk;
    const int64_t k1 = k0 + chunk < kend ? k0 + chunk : kend;
    const int n_st = k1 > k0 ? (int)((k1 - k0 + kPK - 1) / kPK) : 0;

    // ---- Q: heads h_base + 16 hb + l16, k-steps 9d .. 9d+8 (dims 32 s + 8 g .. +7)
    const int h_base = hg * kHPW + pr * 32;
    u32x4 qreg[2][9];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
        const int head = h_base + hb * 16 + l16;
        const bool ok = head < a.n_head;
        const u32x4 *qp = reinterpret_cast<const u32x4 *>(
            a.q + ((int64_t)row * a.n_head + (ok ? head : a.n_head - 1)) * kDK + 8 * g) + 4 * 9 * d;
#pragma unroll
        for (int j = 0; j < 9; ++j) {
            const u32x4 v = qp[4 * j];
            qreg[hb][j] = ok ? v : u32x4{0u, 0u, 0u, 0u};
        }
    }

    // softmax state of heads 16 d + l16 (this wave's block); o[hb][nb]: heads 4g..4g+3 of
    // block hb, dv column 256 d + 16 nb + l16
    float m_run = -INFINITY, l_run = 0.f;
    f32x4 o[2][16];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int nb = 0; nb < 16; ++nb) o[hb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // ---- LDS read offsets within a stage.  K-step j of this wave is s = 9 d + j; steps
    // 0..15 are latent dims (byte 64 s + 16 g of the key row), 16 and 17 RoPE chunks.
    // Step 8 of wave 1 reads RoPE chunk 4 + g = chunk (g ^ 4): its swizzled slot is that of
    // step 7 with bit 6 of the byte offset flipped (stage bases and 128-byte rows keep
    // bits 0..6 clear), so one offset register serves both steps.
    const int qk_off = l16 * kVRow + 16 * g + 576 * d;
    const int k7_lo = d ? kPRopeOff + rope_slot(l16, g) : qk_off + 448;
    const int k_hi = d ? 16 * 128 : 16 * kVRow;       // second 16-key block, steps 7 and 8
    const int tr_off = (4 * g + (l16 >> 2)) * kVRow + 8 * (lane & 3) + 512 * d;
    unsigned char *xpair = lds + kXOff + pr * kXBytes;

    int idx0 = 0;
    if constexpr (IDX) {
        int64_t pos = k0 + lane;
        if (pos >= k1) pos = k1 - 1;
        if (n_st > 0) idx0 = clamp_row(irow[pos], a.n_kv);
    }

    // Copy stage n into `dst`: 32 latent rows (one full-wave copy each), the RoPE bytes of
    // 8 rows per copy, the stage's mask values and the index entries of stage n + 1.  The
    // copies are split into 7 parts of at most two instructions, which the copying waves
    // issue one per Q.K^T step: issued all at once they would queue behind each other in
    // the vector memory address unit (64 B per clock per CU) and stall the waves.  Four
    // waves copy (all of them when NP = 2, group A when NP = 4).
    constexpr int kNWC = 4;
    static_assert(kPK % (2 * kNWC) == 0 && kPK / 8 == kNWC, "copy parts");
    constexpr int kCopyParts = 7;
    struct CopyPlan {
        int64_t kt;
        int last;
        const uint8_t *tbase;
        int my_idx;
    };
    auto copy_plan = [&](int n, const unsigned char *__restrict__ idx_src) __attribute__((always_inline)) {
        CopyPlan c;
        c.kt = k0 + (int64_t)n * kPK;
        c.last = (int)((k1 - c.kt) < kPK ? (k1 - c.kt) : kPK) - 1;
        c.my_idx = 0;
        if constexpr (IDX) {
            int ln = lane;
            asm volatile("" : "+v"(ln));
            c.my_idx = n == 0 ? idx0 : clamp_row(reinterpret_cast<const int *>(idx_src + kPIdxOff)[ln], a.n_kv);
        }
        c.tbase = IDX ? kvs : kvs + c.kt * a.kv_row_stride;
        return c;
    };
    auto copy_part = [&](const CopyPlan &c, int part, unsigned char *__restrict__ dst) __attribute__((always_inline)) {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        if (part < 4) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int r = wave + kNWC * (2 * part + e);
                const int rc = r < c.last ? r : c.last;
                const uint8_t *rowp;
                if constexpr (IDX)
                    rowp = c.tbase + (int64_t)__builtin_amdgcn_readlane(c.my_idx, rc) * a.kv_row_stride;
                else
                    rowp = c.tbase + (int64_t)rc * a.kv_row_stride;
                __builtin_amdgcn_global_load_lds((const void *)(rowp + ln * 16), (LDS_PTR(void))(dst + r * kVRow), 16, 0, 0);
            }
        } else if (part == 4) {
            const int q = wave;
            const int r = 8 * q + (ln >> 3);
            const int rc = r < c.last ? r : c.last;
            const int chunk_i = (ln & 7) ^ ((r >> 1) & 7);
            const uint8_t *src;
            if constexpr (IDX)
                src = c.tbase + (int64_t)shfl_int(c.my_idx, rc) * a.kv_row_stride;
            else
                src = c.tbase + (int64_t)rc * a.kv_row_stride;
            __builtin_amdgcn_global_load_lds((const void *)(src + 1024 + 16 * chunk_i),
                                             (LDS_PTR(void))(dst + kPRopeOff + q * 1024), 16, 0, 0);
        } else if (part == 5) {
            if (mrow && wave == kNWC - 1) {
                const int r = ln < c.last ? ln : c.last;
                const int64_t col = IDX ? (int64_t)shfl_int(c.my_idx, r) : c.kt + r;
                __builtin_amdgcn_global_load_lds((const void *)(mrow + col), (LDS_PTR(void))(dst + kPMaskOff), 2, 0, 0);
            }
        } else if (part == 6) {
            if constexpr (IDX) {
                if (wave == kNWC - 2) {
                    int64_t pos = c.kt + kPK + ln;
                    if (pos >= k1) pos = k1 - 1;
                    __builtin_amdgcn_global_load_lds((const void *)(irow + pos), (LDS_PTR(void))(dst + kPIdxOff), 4, 0, 0);
                }
            }
        }
    };

    constexpr int kQkD = 1, kPvD = 3;             // operand ring depths (register budget)
    // Two schedules, one barrier-phase apart.  X (top of iteration n) publishes the copied
    // stage n; Y (mid-iteration) publishes partial scores, P and rescale factors.
    //   group A: [X] Q.K^T(n)                 [Y] softmax(n), P.V(n - 1)
    //   group B: [X] softmax(n - 1)           [Y] Q.K^T(n), P.V(n - 1)
    // With 8 waves, pairs 0-1 run A and pairs 2-3 run B; wave w and w + 4 share a SIMD, so
    // each SIMD has one wave in an MFMA phase while the other runs its softmax.  Both
    // groups read only stages n and n - 1 in iteration n, so the third slot can receive
    // stage n + 1.  P is double-buffered by stage parity; scores and factors are
    // single-buffered (each is read in the phase after it is written, before the next write).
    const bool grp_b = NP == 4 && pr >= 2;

    // Rescale both head blocks by the factors the owners published with P of the last
    // softmax (before that stage's P.V accumulates into O).
    auto rescale = [&](const unsigned char *__restrict__ xch) __attribute__((always_inline)) {
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
            const unsigned flag = __builtin_amdgcn_readfirstlane(*reinterpret_cast<const unsigned *>(xch + kXF + 16 * hb));
            if (flag) {
                const f32x4 al = *reinterpret_cast<const f32x4 *>(xch + kXA + 64 * hb + 16 * g);
#pragma unroll
                for (int nb = 0; nb < 16; ++nb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[hb][nb][r] *= al[r];
            }
        }
    };
    // Partial scores of this wave's dims for both head blocks of stage `st`; the partner's
    // block goes to LDS, this wave's own block is returned.
    auto qk = [&](const unsigned char *__restrict__ st, unsigned char *__restrict__ xch, f32x4 *own,
                  auto &&on_step) __attribute__((always_inline)) {
        f32x4 sacc[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) sacc[kb][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
        u32x4 ka[kQkD + 1][2];
        auto load_k = [&](int j, u32x4 *dstk) __attribute__((always_inline)) {
            int lo, hi;
            if (j < 7) { lo = qk_off + 64 * j; hi = lo + 16 * kVRow; }
            else if (j == 7) { lo = k7_lo; hi = k7_lo + k_hi; }
            else { lo = d ? (k7_lo ^ 64) : k7_lo + 64; hi = lo + k_hi; }
            dstk[0] = *reinterpret_cast<const u32x4 *>(st + lo);
            dstk[1] = *reinterpret_cast<const u32x4 *>(st + hi);
        };
#pragma unroll
        for (int j = 0; j < kQkD; ++j) load_k(j, ka[j]);
#pragma unroll
        for (int j = 0; j < 9; ++j) {
            if (j + kQkD < 9) load_k(j + kQkD, ka[(j + kQkD) % (kQkD + 1)]);
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    sacc[kb][hb] = mfma16x16x32<KIND>(ka[j % (kQkD + 1)][kb], qreg[hb][j], sacc[kb][hb]);
            on_step(j);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            *reinterpret_cast<f32x4 *>(xch + kXS + d * 2048 + kb * 1024 + 16 * lane) = d ? sacc[kb][0] : sacc[kb][1];
            own[kb] = d ? sacc[kb][1] : sacc[kb][0];
        }
    };
    // Online softmax of stage m for this wave's head block: full scores = own partial +
    // the partner's; publishes P(m) (parity m & 1), the rescale factors and the flag.
    auto softmax = [&](int m, const f32x4 *own, const unsigned char *__restrict__ st,
                       unsigned char *__restrict__ xch) __attribute__((always_inline)) {
        const int64_t kt = k0 + (int64_t)m * kPK;
        f32x4 oth[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            oth[kb] = *reinterpret_cast<const f32x4 *>(xch + kXS + (1 - d) * 2048 + kb * 1024 + 16 * lane);
        u32x4 mk[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
        if (mrow) {
            const unsigned *mls = reinterpret_cast<const unsigned *>(st + kPMaskOff);
            mk[0] = *reinterpret_cast<const u32x4 *>(mls + 4 * g);
            mk[1] = *reinterpret_cast<const u32x4 *>(mls + 16 + 4 * g);
        }
        const int64_t rem64 = k1 - kt;
        const int rem = rem64 < kPK ? (int)rem64 : kPK;
        // scores of this lane: i < 4 key 4g + i, i >= 4 key 16 + 4g + (i - 4)
        float tv[8];
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float sc = own[i >> 2][i & 3] + oth[i >> 2][i & 3];
            const float bias = mrow ? f16_bits_to_f32((unsigned short)(mk[i >> 2][i & 3] & 0xFFFFu)) * kLog2e : 0.f;
            const float x = sc * a.scale_log2 + bias;
            tv[i] = 16 * (i >> 2) + 4 * g + (i & 3) < rem ? x : -INFINITY;
            mx = fmaxf(mx, tv[i]);
        }
        mx = wave_max_groups(mx);
        const bool need = mx > m_run + kRescaleThresh;
        const unsigned long long bal = __builtin_amdgcn_ballot_w64(need);
        const float alpha = need ? __builtin_amdgcn_exp2f(m_run - mx) : 1.f;
        m_run = need ? mx : m_run;
        l_run *= alpha;
        const float m_use = m_run == -INFINITY ? 0.f : m_run;
        float pv[8], ps = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            pv[i] = __builtin_amdgcn_exp2f(tv[i] - m_use);
            ps += pv[i];
        }
        l_run += ps;
        // every lane writes its head's factor (lanes with equal l16 agree)
        reinterpret_cast<float *>(xch + kXA + 64 * d)[l16] = alpha;
        *reinterpret_cast<unsigned *>(xch + kXF + 16 * d) = bal != 0ull ? 1u : 0u;
        *reinterpret_cast<u32x4 *>(xch + kXP + (m & 1) * 2048 + d * 1024 + 16 * lane) =
            u32x4{pack_p<KIND>(pv[0], pv[1]), pack_p<KIND>(pv[2], pv[3]),
                  pack_p<KIND>(pv[4], pv[5]), pack_p<KIND>(pv[6], pv[7])};
    };
    // O += P(m) . V(m) for this wave's dv half, V from stage `st`.
    auto pv = [&](int m, const unsigned char *__restrict__ st, const unsigned char *__restrict__ xch)
        __attribute__((always_inline)) {
        const unsigned char *xpp = xch + kXP + (m & 1) * 2048 + 16 * lane;
        const u32x4 pa[2] = {*reinterpret_cast<const u32x4 *>(xpp), *reinterpret_cast<const u32x4 *>(xpp + 1024)};
        auto load_v = [&](int nb) __attribute__((always_inline)) -> u32x4 {
            const int off = tr_off + 32 * nb;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_PTR(s16x4))(st + off));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_PTR(s16x4))(st + off + 16 * kVRow));
            const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
            return u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
        };
        u32x4 vb[kPvD + 1];
#pragma unroll
        for (int nb = 0; nb < kPvD; ++nb) vb[nb] = load_v(nb);
#pragma unroll
        for (int nb = 0; nb < 16; ++nb) {
            if (nb + kPvD < 16) vb[(nb + kPvD) % (kPvD + 1)] = load_v(nb + kPvD);
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) o[hb][nb] = mfma16x16x32<KIND>(pa[hb], vb[nb % (kPvD + 1)], o[hb][nb]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // own-block partial scores of the last Q.K^T, carried from phase Y to the next X (group B)
    f32x4 keep[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    // One iteration.  Restrict-qualified stage pointers: the copy target never overlaps the
    // stages or the exchange area read in the same iteration (without it the compiler
    // would make every LDS read wait for the copies in flight).
    auto step = [&](auto GB_, int n, unsigned char *__restrict__ next, const unsigned char *__restrict__ cur,
                    const unsigned char *__restrict__ prev, unsigned char *__restrict__ xch)
        __attribute__((always_inline)) {
        constexpr bool GB = decltype(GB_)::value;
        if constexpr (!GB) {
            if (n >= 1) rescale(xch);
            f32x4 own[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
            // n + 1 < n_st implies n < n_st: the copy of stage n + 1 rides on this Q.K^T
            if (n + 1 < n_st) {
                const CopyPlan cp = copy_plan(n + 1, cur);
                qk(cur, xch, own, [&](int j) __attribute__((always_inline)) {
                    if (j < kCopyParts) copy_part(cp, j, next);
                });
            } else if (n < n_st) {
                qk(cur, xch, own, [](int) {});
            }
            lds_barrier();                                   // Y
            if (n < n_st) softmax(n, own, cur, xch);
            __builtin_amdgcn_sched_barrier(0);
            if (n >= 1) pv(n - 1, prev, xch);
        } else {
            if (n >= 1) softmax(n - 1, keep, prev, xch);
            lds_barrier();                                   // Y
            if (n >= 1) rescale(xch);
            if (n < n_st) qk(cur, xch, keep, [](int) {});
            __builtin_amdgcn_sched_barrier(0);
            if (n >= 1) pv(n - 1, prev, xch);
        }
    };

    // one loop per schedule (a single loop holding both would hold both live sets)
    auto run = [&](auto GB_) __attribute__((always_inline)) {
        // the prologue copies stage 0 (copying waves only)
        if (wave < kNWC) {
            const CopyPlan cp = copy_plan(0, lds);
#pragma unroll
            for (int part = 0; part < kCopyParts; ++part) copy_part(cp, part, lds);
        }
        // ring slots rotate (prev, cur, next) -> (cur, next, prev) every iteration
        unsigned char *cur = lds, *next = lds + kPStageBytes, *prev = lds + 2 * kPStageBytes;
        for (int n = 0; n <= n_st; ++n) {
            wait_vm0();
            __syncthreads();                         // X: stage n landed
            step(GB_, n, next, cur, prev, xpair);
            unsigned char *t = prev;
            prev = cur;
            cur = next;
            next = t;
        }
    };
    if (n_st > 0) {
        if (grp_b) run(std::true_type{});
        else run(std::false_type{});
    }

    // ---- epilogue: l of both head blocks, then the output or this split's partial
    l_run = wave_sum_groups(l_run);
    __syncthreads();
    float *xl = reinterpret_cast<float *>(xpair + kXA);     // [wave][16] = l of block d
    if (lane < 16) xl[16 * d + lane] = l_run;
    __syncthreads();
    if (a.n_split == 1) {
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
            const f32x4 l4 = *reinterpret_cast<const f32x4 *>(xl + 16 * hb + 4 * g);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float ir = l4[r] > 0.f ? 1.f / l4[r] : 0.f;
                const int head = h_base + hb * 16 + 4 * g + r;
                if (head < a.n_head) {
                    float *op = a.out + ((int64_t)row * a.n_head + head) * kDV + 256 * d + l16;
#pragma unroll
                    for (int nb = 0; nb < 16; ++nb) op[16 * nb] = o[hb][nb][r] * ir;
                }
            }
        }
    } else {
        // this split's partial, in the layout partial_bytes describes (wave d: half d)
        const int64_t RH = (int64_t)n_rows * a.n_head;
        float *wm = a.ws;
        float *wl = wm + (int64_t)a.n_split * RH;
        float *wsc = wl + (int64_t)a.n_split * RH;
        uint16_t *wo = reinterpret_cast<uint16_t *>(wsc + 2 * (int64_t)a.n_split * RH);
        const int64_t base = (int64_t)split * RH + (int64_t)row * a.n_head;
        const int head_l = h_base + 16 * d + l16;
        if (lane < 16 && head_l < a.n_head) {
            wm[base + head_l] = m_run;
            wl[base + head_l] = l_run;
        }
        if (n_st > 0) {
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int head = h_base + hb * 16 + 4 * g + r;
                    float mx = 0.f;
#pragma unroll
                    for (int nb = 0; nb < 16; ++nb) mx = fmaxf(mx, fabsf(o[hb][nb][r]));
                    const int e = partial_exp(group16_max(mx));
                    const float sc = __builtin_amdgcn_ldexpf(1.f, 15 - e);
                    if (head < a.n_head) {
                        uint16_t *op = wo + (base + head) * kDV + 256 * d + l16;
#pragma unroll
                        for (int nb = 0; nb < 16; ++nb) op[16 * nb] = (uint16_t)pack_f16x2(o[hb][nb][r] * sc, 0.f);
                        if (l16 == 0) wsc[(base + head) * 2 + d] = __builtin_amdgcn_ldexpf(1.f, e - 15);
                    }
                }
            }
        }
    }
}

// Merge split partials: out = sum_i 2^(m_i - m*) O_i / sum_i 2^(m_i - m*) l_i; splits with
// m_i = -inf (no kept key) weigh 0 and their O_i never contributes (it may be unwritten);
// a row with no kept key anywhere outputs 0.  One workgroup per (row, head); thread t owns
// dv quad t % 128 of splits t / 128, t / 128 + 4, ...  O_i is stored as f16 values and a
// power-of-two scale per 256-column half (see partial_bytes), so a split's factor for a
// half is 2^(m_i - m*) times that scale.  The partial O reads are the whole cost, so they
// start first: each thread issues its first 8 loads, then (m_i, l_i, scales) of all
// splits are read in one round trip, reduced to the factors in LDS, and the loads already
// in flight are weighted (a select drops unweighted splits, whose values are read but
// may hold any bits); later batches follow, and
// the four split groups are summed through LDS.  Under a length-proportional plan
// (Ragged) a row's pieces are the slots P_r .. P_r + n_r - 1 that the plan gives it; a row
// with no piece outputs 0.
constexpr int kMergeBatch = 8;
template <int G>   // split groups of 128 threads
__global__ void __launch_bounds__(128 * G) merge_kernel(int n_rows, int n_head, int n_split,
                                                        const float *__restrict__ ws, float *__restrict__ out,
                                                        const float *__restrict__ sinks, Ragged rg) {
    constexpr int kThreads = 128 * G;
    __shared__ float w_s[kMaxSplits];
    __shared__ float l_s[kMaxSplits];
    __shared__ f32x2v sc_s[kMaxSplits];
    __shared__ float red[kThreads / 64];
    __shared__ f32x4 part[G - 1 > 0 ? G - 1 : 1][128];
    const int64_t rh = blockIdx.x;                    // row * n_head + head
    const int64_t RH = (int64_t)n_rows * n_head;
    const float *wm = ws;
    const float *wl = wm + (int64_t)n_split * RH;
    const f32x2v *wsc = reinterpret_cast<const f32x2v *>(wl + (int64_t)n_split * RH);
    const uint16_t *wo = reinterpret_cast<const uint16_t *>(wsc + (int64_t)n_split * RH);
    const int tid = threadIdx.x;
    const int q = tid & 127, sg = tid >> 7;
    // (slot, head) entry of this row's first split, the stride between its splits, and
    // their number
    int64_t e0 = rh, es = RH;
    int ns = n_split;
    if (rg.budget) {
        const unsigned v = reinterpret_cast<const unsigned *>(ws + ragged_table_off(n_split, n_rows, n_head))[rh / n_head];
        const int first = (int)(v & 0xFFFFu), n = (int)(v >> 16);
        e0 = (int64_t)(n > 0 ? first : 0) * n_head + rh % n_head;   // (no piece: slot 0, read and weighed 0)
        es = n_head;
        ns = n;
    }
    const u32x2 *op = reinterpret_cast<const u32x2 *>(wo + e0 * kDV) + q;   // 4 f16 values
    const int64_t step4 = es * kDV / 4;               // stride between splits, in quads
    // O of a split = scale of its half x the stored f16 values
    auto f16x4_to_f32 = [](u32x2 v) __attribute__((always_inline)) {
        return __builtin_convertvector(__builtin_bit_cast(f16x4v, v), f32x4);
    };

    u32x2 v0[kMergeBatch];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
        const int i = sg + u * G;
        v0[u] = op[(int64_t)(i < ns ? i : 0) * step4];   // unconditional: no wait until used
    }
    float mloc = -INFINITY;
    for (int i = tid; i < ns; i += kThreads) {
        const float mi = wm[e0 + i * es];
        w_s[i] = mi;
        l_s[i] = wl[e0 + i * es];
        sc_s[i] = wsc[e0 + i * es];
        mloc = fmaxf(mloc, mi);
    }
    for (int off = 32; off > 0; off >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, off));
    if ((tid & 63) == 0) red[tid >> 6] = mloc;
    __syncthreads();
    float mstar = red[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) mstar = fmaxf(mstar, red[i]);
    // weights 2^(m_i - m*) (0 for empty splits, and for every split if all are empty)
    float lloc = 0.f;
    for (int i = tid; i < ns; i += kThreads) {
        const float mi = w_s[i];
        const float wgt = (mstar == -INFINITY || mi == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mi - mstar);
        if (wgt != 0.f) lloc += wgt * l_s[i];
        // per-half factors of the stored values: weight x scale (0 for unweighted splits)
        w_s[i] = wgt != 0.f ? wgt * sc_s[i][0] : 0.f;
        l_s[i] = wgt != 0.f ? wgt * sc_s[i][1] : 0.f;
    }
    for (int off = 32; off > 0; off >>= 1) lloc += __shfl_xor(lloc, off);
    __syncthreads();
    if ((tid & 63) == 0) red[tid >> 6] = lloc;
    __syncthreads();
    float lsum = 0.f;
#pragma unroll
    for (int i = 0; i < kThreads / 64; ++i) lsum += red[i];
    if (sinks && mstar != -INFINITY)   // the sink joins the normaliser (m* in log2 units)
        lsum += __builtin_amdgcn_exp2f(sinks[rh % n_head] * 1.4426950408889634f - mstar);

    const float *f_s = q < 64 ? w_s : l_s;           // this thread's half (uniform per wave)
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
        const int i = sg + u * G;
        const float wgt = i < ns ? f_s[i] : 0.f;
        const f32x4 x = f16x4_to_f32(v0[u]);
        if (wgt != 0.f) acc += wgt * x;
    }
    int i = sg + kMergeBatch * G;
    for (; i + (kMergeBatch - 1) * G < ns; i += kMergeBatch * G) {
        u32x2 v[kMergeBatch];
        float wv[kMergeBatch];
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) {
            wv[u] = f_s[i + u * G];
            v[u] = op[(int64_t)(i + u * G) * step4];
        }
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) {   // unweighted splits may hold any bits: select
            const f32x4 x = f16x4_to_f32(v[u]);
            if (wv[u] != 0.f) acc += wv[u] * x;
        }
    }
    for (; i < ns; i += G) {
        const float wgt = f_s[i];
        if (wgt != 0.f) acc += wgt * f16x4_to_f32(op[(int64_t)i * step4]);
    }
    if (sg > 0) part[sg - 1][q] = acc;
    __syncthreads();
    if (sg == 0) {
#pragma unroll
        for (int k = 0; k < G - 1; ++k) acc += part[k][q];
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
        reinterpret_cast<f32x4 *>(out + rh * kDV)[q] = acc * inv;
    }
}

// One launch per kMaxGridY query rows (the grid's y extent); a.row_base tells each launch
// where its rows start.  A length-proportional plan is one launch with y = 1.
template <typename K>
hipError_t launch_rows(K kernel, const AttnArgs &a, int threads, hipStream_t stream) {
    const int64_t rows = a.ragged.budget ? 1 : (int64_t)a.n_seq * a.n_tok;
    for (int64_t r0 = 0; r0 < rows; r0 += kMaxGridY) {
        AttnArgs b = a;
        b.row_base = (int)r0;
        const int n = (int)(rows - r0 < kMaxGridY ? rows - r0 : kMaxGridY);
        hipLaunchKernelGGL(kernel, dim3(a.grid_x, n), dim3(threads), 0, stream, b);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int MB, int NW, int WK, int KIND, bool IDX>
hipError_t launch_one(const AttnArgs &a, hipStream_t stream) {
    return launch_rows(attn_kernel<MB, NW, WK, KIND, IDX>, a, NW * 64, stream);
}

// Per-sequence lengths, ALiBi, sinks, softcap and length-proportional plans run in the
// single-wave kernel only.
bool uses_extras(const AttnArgs &a) {
    return a.kv_len || a.alibi || a.sinks || a.cap_in != 0.f || a.ragged.budget;
}

template <int NP, int KIND, bool IDX>
hipError_t launch_pair(const AttnArgs &a, hipStream_t stream) {
    return launch_rows(attn_pair_kernel<NP, KIND, IDX>, a, NP * 128, stream);
}

template <int KIND, bool IDX>
hipError_t launch_shape(const AttnArgs &a, int shape, hipStream_t stream) {
    switch (shape) {
        case SHAPE_H16: return launch_one<1, 2, 2, KIND, IDX>(a, stream);
        case SHAPE_H32: return launch_one<1, 4, 2, KIND, IDX>(a, stream);
        case SHAPE_H64: return launch_one<1, 8, 2, KIND, IDX>(a, stream);
        case SHAPE_H128: return launch_one<1, 8, 1, KIND, IDX>(a, stream);
        // pair shapes: dense 16-bit caches only; Q8_0 and indexed rows run the single-wave
        // kernel with the same heads per workgroup (so the plan's head groups still hold)
        case SHAPE_P64:
            if constexpr (KIND != KV_Q8 && !IDX)
                if (!uses_extras(a)) return launch_pair<2, KIND, IDX>(a, stream);
            return launch_one<1, 8, 2, KIND, IDX>(a, stream);
        case SHAPE_P128:
            if constexpr (KIND != KV_Q8 && !IDX)
                if (!uses_extras(a)) return launch_pair<4, KIND, IDX>(a, stream);
            return launch_one<1, 8, 1, KIND, IDX>(a, stream);
    }
    return hipErrorInvalidValue;
}

template <int KIND>
hipError_t launch_kind(const AttnArgs &a, int shape, hipStream_t stream) {
    return a.kv_idx ? launch_shape<KIND, true>(a, shape, stream) : launch_shape<KIND, false>(a, shape, stream);
}

}  // namespace

hipError_t launch_attention(const AttnArgs &a, int kv_kind, int shape, hipStream_t stream) {
    switch (kv_kind) {
        case KV_BF16: return launch_kind<KV_BF16>(a, shape, stream);
        case KV_F16: return launch_kind<KV_F16>(a, shape, stream);
        case KV_Q8: return launch_kind<KV_Q8>(a, shape, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_merge(int n_rows, int n_head, int n_split, const float *ws, float *out,
                        const float *sinks, const Ragged &ragged, hipStream_t stream) {
    // Four split groups per (row, head), or two when that lets every workgroup of the
    // launch be resident at once (up to 8,192 waves on the chip).
    const int64_t pairs = (int64_t)n_rows * n_head;
    if (pairs > 1024 && pairs <= 2048)
        hipLaunchKernelGGL(merge_kernel<2>, dim3((unsigned)pairs), dim3(256), 0, stream, n_rows, n_head, n_split,
                           ws, out, sinks, ragged);
    else
        hipLaunchKernelGGL(merge_kernel<4>, dim3((unsigned)pairs), dim3(512), 0, stream, n_rows, n_head, n_split,
                           ws, out, sinks, ragged);
    return hipGetLastError();
}

}  // namespace mlafa
