// mha.hip -- per-head flash attention for the non-absorbed MLA prefill shape (gfx950).
//
// Each head has its own 192-wide keys (128 dims + 64 RoPE) and 128-wide values: the
// DK=192 / DV=128 configuration the Metal tensor-API flash-attention kernel lists
// ("llama.cpp Metal: tensor-API flash attention for F16 KV caches" news item), i.e. the
// per-head K/V that the "Vulkan backend fused Flash Attention: DeepSeek MLA local
// inference" page (section 3.3) decompresses from the latent cache.  The online softmax
// is the same as in the latent kernel (same page, sections 2.1-2.2).
//
// Design (gfx950-specific):
//   * A workgroup serves 256 query tokens of one head: 8 waves x 32 tokens.  The
//     tokens play the part heads play in the latent kernel: S^T = K.Q^T has keys as M and
//     tokens as N, so its accumulator (lane = token) is directly the A operand of P.V.
//     Q and O of 32 tokens take 48 + 64 VGPRs, so each K or V byte read from LDS feeds
//     32 tokens.
//   * 64-key stages of K (384 B per key) and V (256 B per key) are copied HBM -> LDS by
//     full-wave global_load_lds_dwordx4 copies into unpadded areas, in a ring of three
//     stages (two copies in flight while one stage is computed).  16-byte chunks are
//     XOR-swizzled per key so that both read patterns are bank-conflict free: K chunk c of
//     key r sits at slot (c & ~7) | ((c & 7) ^ ((r >> 1) & 7)) (16 keys reading one chunk
//     hit 16 distinct bank groups); V chunk c of key r at slot c ^ ((r & 7) << 1) (the
//     transpose read's 8 keys x 32 bytes hit 16 distinct groups).
//   * Causal: token t sees keys j <= n_kv - n_tok + t.  Workgroups with later tokens are
//     dispatched first (they have the most keys); a wave skips the tiles its tokens cannot
//     see.  The optional f16 mask [n_tok][n_kv] is added to the scaled score (-inf drops
//     the cell).  Its words travel the same way as K and V: each wave copies its own
//     tokens' 64 keys per stage into a swizzled 4 KiB area (a ring of two 72 KiB stages
//     then), so the loop never holds a register result of a global load.
#include "mla_fa_internal.h"

namespace mlafa {
namespace {

#include "device_common.h"

constexpr int kMDK = 192, kMDV = 128;
constexpr int kMKeys = 64;                          // keys per stage
constexpr int kSubKeys = 32;                        // keys per softmax step
constexpr int kMKRow = kMDK * 2, kMVRow = kMDV * 2;  // 384, 256 bytes
constexpr int kMKArea = kMKeys * kMKRow;            // 24,576
constexpr int kMVArea = kMKeys * kMVRow;            // 16,384
constexpr int kMStage = kMKArea + kMVArea;          // 40,960
constexpr int kMNW = 8, kMMB = 2;                   // waves, 16-token blocks per wave
constexpr int kMTokens = kMNW * kMMB * 16;          // 256 tokens per workgroup
constexpr float kMRescaleThresh = 8.0f;
constexpr int kMMaskWave = kMMB * 16 * kMKeys * 2;   // mask words of one wave's tokens: 4,096 B
constexpr int kMMaskArea = kMNW * kMMaskWave;       // 32,768

// LDS ring: three K/V stages without a mask (copies two tiles ahead); with one, two stages
// that also hold the mask (copies one tile ahead).
template <bool MASK> struct MhaRing {
    static constexpr int kStages = MASK ? 2 : 3;
    static constexpr int kAhead = MASK ? 1 : 2;    // tiles copied ahead of the one computed
    static constexpr int kStageBytes = kMStage + (MASK ? kMMaskArea : 0);
    static constexpr int kCopies = kStageBytes / 1024 / kMNW;   // 1 KiB copies per wave per stage
};
static_assert(kMKArea % (1024 * kMNW) == 0 && kMVArea % (1024 * kMNW) == 0, "copies per wave");
static_assert(kMMaskWave % 1024 == 0, "mask copies per wave");

__device__ __forceinline__ int k_slot(int r, int c) { return (c & ~7) | ((c & 7) ^ ((r >> 1) & 7)); }
__device__ __forceinline__ int v_slot(int r, int c) { return c ^ ((r & 7) << 1); }
// mask words of token u (0..31 within the wave), 16-byte chunk c (8 keys) of the stage
__device__ __forceinline__ int m_slot(int u, int c) { return c ^ ((u >> 1) & 7); }

template <int KIND, bool MASK>
__global__ void __launch_bounds__(kMNW * 64, 1) mha_kernel(MhaArgs a) {
    using Ring = MhaRing<MASK>;
    __shared__ __attribute__((aligned(1024))) unsigned char lds[Ring::kStages * Ring::kStageBytes];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, l16 = lane & 15;
    // Workgroup -> (head, token tile).  Workgroups are dealt to the 8 XCDs round-robin by
    // linear id; when the head count allows, every token tile of a head goes to the same
    // XCD (head = 8 (k / n_tt) + id % 8 for the k-th workgroup of that XCD), so the tiles
    // that sweep one head's keys together share that XCD's L2.  Within a head, later token
    // tiles (more keys) come first.
    const int n_tt = (a.n_tok + kMTokens - 1) / kMTokens;
    const int wg = blockIdx.x;
    int head, tile_rev;
    if (a.n_head % 8 == 0) {
        const int k = wg >> 3;
        head = 8 * (k / n_tt) + (wg & 7);
        tile_rev = k % n_tt;
    } else {
        head = wg / n_tt;
        tile_rev = wg % n_tt;
    }
    const int tile = n_tt - 1 - tile_rev;
    const int t0 = tile * kMTokens;
    const int tw = t0 + wave * kMMB * 16;                    // first token of this wave
    const int64_t off = a.n_kv - a.n_tok;                    // token t sees j <= off + t when causal

    // key range of the workgroup and of this wave (exclusive ends)
    const int t_last = (t0 + kMTokens < a.n_tok ? t0 + kMTokens : a.n_tok) - 1;
    const int64_t kend = a.causal ? off + t_last + 1 : a.n_kv;
    const int n_tiles = kend > 0 ? (int)((kend + kMKeys - 1) / kMKeys) : 0;
    const int tw_last = (tw + kMMB * 16 < a.n_tok ? tw + kMMB * 16 : a.n_tok) - 1;
    const int64_t wend = tw > t_last ? 0 : (a.causal ? off + tw_last + 1 : a.n_kv);

    // Q of this wave's tokens: B operand of S^T (dims 32 s + 8 g .. +7)
    u32x4 qreg[kMMB][6];
    int lim[kMMB];                                           // last key each lane's token sees (n_kv < 2^31)
#pragma unroll
    for (int mb = 0; mb < kMMB; ++mb) {
        const int t = tw + mb * 16 + l16;
        const bool ok = t < a.n_tok;
        const u32x4 *qp = reinterpret_cast<const u32x4 *>(
            a.q + ((int64_t)(ok ? t : a.n_tok - 1) * a.n_head + head) * kMDK + 8 * g);
#pragma unroll
        for (int s = 0; s < 6; ++s) qreg[mb][s] = ok ? qp[4 * s] : u32x4{0u, 0u, 0u, 0u};
        lim[mb] = !ok ? -1 : (int)(a.causal ? off + t : a.n_kv - 1);
    }
    wait_vm0();   // Q is in registers before the loop: no wait inside it counts these loads

    // running state per lane and 16-token block: reference mu (log2 units), threshold,
    // O (rows 4 g + r) and the row sums of P (rows 4 g + r, all columns equal)
    float mu[kMMB], thr[kMMB];
    f32x4 o[kMMB][8], lsum[kMMB];
    int lim_lo[kMMB];                                        // smallest lim of the block's tokens
#pragma unroll
    for (int mb = 0; mb < kMMB; ++mb) {
        mu[mb] = 0.f;
        thr[mb] = -INFINITY;
        lsum[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) o[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int tb = tw + mb * 16;
        lim_lo[mb] = tb + 15 >= a.n_tok ? -1 : (int)(a.causal ? off + tb : a.n_kv - 1);
    }
    const unsigned one2 = KIND == KV_BF16 ? 0x3F803F80u : 0x3C003C00u;   // two 1.0 values
    const u32x4 kOnes = u32x4{one2, one2, one2, one2};

    // per-lane LDS read offsets: K (S^T A operand) row l16, chunk 4 s + g; V (P.V B operand
    // by transpose read) row 4 G + j / 4, byte 32 nb + 8 (j % 4) before the swizzle
    const int fk = (l16 >> 1) & 7;
    const int k_even = l16 * kMKRow + 16 * (g ^ fk);         // chunk & 7 = g      (s even)
    const int k_odd = l16 * kMKRow + 16 * ((4 + g) ^ fk);    // chunk & 7 = 4 + g  (s odd)
    const int vr = 4 * g + (l16 >> 2);
    const int v_base = kMKArea + vr * kMVRow + 8 * (lane & 3);
    const int v_x = (vr & 7) << 5;                            // 32 * (row & 7): the swizzle, in bytes

    // Copy tile `it` into stage `dst` in Ring::kCopies parts of one 1 KiB full-wave copy each:
    // parts 0..2 are K copies w, w + 8, w + 16 of wave w (24 in all), parts 3, 4 V copies w,
    // w + 8 (16 in all) and, with a mask, parts 5..8 four copies of the wave's own tokens'
    // mask words.  Every wave issues every part, which the waits in the loop count on.
    const int64_t jmax8 = (a.n_kv - 1) & ~(int64_t)7;
    constexpr int kKParts = kMKArea / 1024 / kMNW, kVParts = kMVArea / 1024 / kMNW;
    auto issue_part = [&](int it, int part, unsigned char *__restrict__ dst) __attribute__((always_inline)) {
        const int64_t kt = (int64_t)it * kMKeys;
        const int last = (int)((kend - kt) < kMKeys ? (kend - kt) : kMKeys) - 1;
        int ln = lane;
        asm volatile("" : "+v"(ln));
        if (part < kKParts) {
            const int b = wave + part * kMNW;
            const int gs = b * 64 + ln;                      // slot index in the K area
            const int r = gs / 24, p = gs - (gs / 24) * 24;
            const int c = k_slot(r, p);                      // the swizzle is its own inverse
            const int rc = r < last ? r : last;
            const uint8_t *src = a.k + (kt + rc) * a.k_row_stride + (int64_t)head * kMKRow + 16 * c;
            __builtin_amdgcn_global_load_lds((const void *)src, (LDS_PTR(void))(dst + b * 1024), 16, 0, 0);
        } else if (part < kKParts + kVParts) {
            const int vb = wave + (part - kKParts) * kMNW;
            const int r = 4 * vb + (ln >> 4), p = ln & 15;
            const int c = v_slot(r, p);
            const int rc = r < last ? r : last;
            const uint8_t *src = a.v + (kt + rc) * a.v_row_stride + (int64_t)head * kMVRow + 16 * c;
            __builtin_amdgcn_global_load_lds((const void *)src, (LDS_PTR(void))(dst + kMKArea + vb * 1024), 16, 0, 0);
        } else if constexpr (MASK) {
            // this wave's 32 tokens x 64 keys: copy q covers tokens 8 q .. 8 q + 7, lane l
            // token 8 q + l / 8, slot l % 8 holding key chunk m_slot(token, l % 8).  The chunk
            // holding key n_kv - 1 stands in for chunks past it (those keys are dropped by
            // the range check); its 16-byte block is aligned, so it does not leave its page.
            const int q = part - kKParts - kVParts;
            const int u = 8 * q + (ln >> 3);
            const int c = m_slot(u, ln & 7);
            const int t = tw + u < a.n_tok ? tw + u : a.n_tok - 1;
            const int64_t j = kt + 8 * c < jmax8 ? kt + 8 * c : jmax8;
            const uint16_t *src = a.mask + (int64_t)t * a.mask_row_stride + j;
            __builtin_amdgcn_global_load_lds((const void *)src,
                                             (LDS_PTR(void))(dst + kMStage + wave * kMMaskWave + q * 1024), 16, 0, 0);
        }
    };
    auto issue = [&](int it, unsigned char *__restrict__ dst) __attribute__((always_inline)) {
#pragma unroll
        for (int part = 0; part < Ring::kCopies; ++part) issue_part(it, part, dst);
    };

    constexpr int kQkD = 2, kPvD = 3;
    typedef f32x4 SAcc[2][kMMB];          // S^T of one 32-key sub-tile: [key half][token block]
    typedef float TV[kMMB][8];            // its scores in log2 units, relative to mu

    // S^T = K . Q^T for keys sub0 .. sub0 + 31 of stage `st` (K chunks read once, used for
    // both token blocks).
    auto qk = [&](const unsigned char *__restrict__ st, int sub0, SAcc &sacc) __attribute__((always_inline)) {
        const unsigned char *sk = st + sub0 * kMKRow;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int mb = 0; mb < kMMB; ++mb) sacc[kb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
        u32x4 ka[kQkD + 1][2];
        auto load_k = [&](int s, u32x4 *dk) __attribute__((always_inline)) {
            const int o_ = ((s & 1) ? k_odd : k_even) + 128 * (s >> 1);
            dk[0] = *reinterpret_cast<const u32x4 *>(sk + o_);
            dk[1] = *reinterpret_cast<const u32x4 *>(sk + o_ + 16 * kMKRow);
        };
#pragma unroll
        for (int s = 0; s < kQkD; ++s) load_k(s, ka[s]);
#pragma unroll
        for (int s = 0; s < 6; ++s) {
            if (s + kQkD < 6) load_k(s + kQkD, ka[(s + kQkD) % (kQkD + 1)]);
#pragma unroll
            for (int mb = 0; mb < kMMB; ++mb)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    sacc[kb][mb] = mfma16x16x32<KIND>(ka[s % (kQkD + 1)][kb], qreg[mb][s], sacc[kb][mb]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Softmax, in log2 units relative to the lane's running reference mu (lane: token l16 of
    // block mb; keys 4 g + i and 16 + 4 g + i of the sub-tile).  pre: t = s * scale * log2(e)
    // - mu (one FMA), plus the mask, minus infinity past the token's last key, and the lane
    // maximum.  Returns whether any lane has a t above its threshold (8 once started, -inf
    // before the first kept key); only then does `rare` run: the token's maximum over its
    // four lanes moves mu up, rescales O and the row sums, and shifts t.  Otherwise
    // p = exp2(t) is already consistent across the four lanes of a token.
    // minus infinity for the keys past each lane's token's last key
    auto range_mask = [&](TV &tv, int64_t kbase) __attribute__((always_inline)) {
#pragma unroll
        for (int mb = 0; mb < kMMB; ++mb) {
            if (kbase + kSubKeys - 1 > lim_lo[mb]) {   // some token of the block ends inside
                const int64_t d64 = (int64_t)lim[mb] - kbase;
                const int e = (int)(d64 < -1 ? -1 : d64 > kSubKeys ? kSubKeys : d64) - 4 * g;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    if (16 * (i >> 2) + (i & 3) > e) tv[mb][i] = -INFINITY;
            }
        }
    };
    auto pre = [&](const SAcc &sacc, const unsigned char *__restrict__ st, int64_t kbase, int sub0, TV &tv,
                   float (&ml)[kMMB]) __attribute__((always_inline)) -> bool {
#pragma unroll
        for (int mb = 0; mb < kMMB; ++mb) {
#pragma unroll
            for (int i = 0; i < 8; ++i) tv[mb][i] = __builtin_fmaf(sacc[i >> 2][mb][i & 3], a.scale_log2, -mu[mb]);
            if constexpr (MASK) {
                // keys sub0 + 16 h + 4 g .. + 3 of token mb * 16 + l16: 8-byte word g & 1 of
                // chunk sub0 / 8 + 2 h + g / 2
                const unsigned char *mrow = st + kMStage + wave * kMMaskWave + (mb * 16 + l16) * (kMKeys * 2);
                u32x2 mw[2];
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    mw[h] = *reinterpret_cast<const u32x2 *>(
                        mrow + 16 * m_slot(l16, sub0 / 8 + 2 * h + (g >> 1)) + 8 * (g & 1));
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const unsigned w = mw[i >> 2][(i & 3) >> 1];
                    const unsigned short b = (unsigned short)((i & 1) ? (w >> 16) : (w & 0xFFFFu));
                    tv[mb][i] = __builtin_fmaf(f16_bits_to_f32(b), kLog2e, tv[mb][i]);   // -inf stays -inf
                }
            }
        }
        range_mask(tv, kbase);
        bool any = false;
#pragma unroll
        for (int mb = 0; mb < kMMB; ++mb) {
            float m_ = tv[mb][0];
#pragma unroll
            for (int i = 1; i < 8; ++i) m_ = fmaxf(m_, tv[mb][i]);
            ml[mb] = m_;
            any = any || m_ > thr[mb];
        }
        return __builtin_amdgcn_ballot_w64(any) != 0;
    };
    auto rare = [&](TV &tv, const float (&ml)[kMMB]) __attribute__((always_inline)) {
#pragma unroll
        for (int mb = 0; mb < kMMB; ++mb) {
            const float mx = wave_max_groups(ml[mb]);   // the token's maximum
            const bool need = mx > thr[mb];
            const float alpha = !need ? 1.f : thr[mb] == kMRescaleThresh ? __builtin_amdgcn_exp2f(-mx) : 0.f;
            const float shift = need ? mx : 0.f;
            if (need) {
                mu[mb] += mx;
                thr[mb] = kMRescaleThresh;
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) tv[mb][i] -= shift;
            float ar[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) ar[r] = shfl_f(alpha, 4 * g + r);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                lsum[mb][r] *= ar[r];
#pragma unroll
                for (int nb = 0; nb < 8; ++nb) o[mb][nb][r] *= ar[r];
            }
        }
    };
    auto post = [&](const TV &tv, u32x4 (&pa)[kMMB]) __attribute__((always_inline)) {
#pragma unroll
        for (int mb = 0; mb < kMMB; ++mb)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                pa[mb][j] = pack_p<KIND>(__builtin_amdgcn_exp2f(tv[mb][2 * j]), __builtin_amdgcn_exp2f(tv[mb][2 * j + 1]));
    };
    // one 32-key sub-tile up to P (S^T, softmax); P . V follows separately
    auto scores = [&](const unsigned char *__restrict__ st, int64_t kbase, int sub0, u32x4 (&pa)[kMMB])
        __attribute__((always_inline)) {
        SAcc sacc;
        TV tv;
        float ml[kMMB];
        qk(st, sub0, sacc);
        if (pre(sacc, st, kbase, sub0, tv, ml)) rare(tv, ml);
        post(tv, pa);
    };

    // O += P . V for keys sub0 .. sub0 + 31 of stage `st` (transpose reads through the
    // swizzle), and the row sums of P (the same rounded P that weights V): P . ones.
    auto pv = [&](const unsigned char *__restrict__ st, int sub0, const u32x4 (&pa)[kMMB]) __attribute__((always_inline)) {
        const unsigned char *sv = st + v_base + sub0 * kMVRow;
        u32x4 vb[kPvD + 1];
        auto load_v = [&](int nb) __attribute__((always_inline)) -> u32x4 {
            int vx = v_x;
            asm volatile("" : "+v"(vx));      // one v_xad per read instead of 8 addresses held in registers
            const int o_ = (32 * nb) ^ vx;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_PTR(s16x4))(sv + o_));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_PTR(s16x4))(sv + o_ + 16 * kMVRow));
            const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
            return u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
        };
#pragma unroll
        for (int nb = 0; nb < kPvD; ++nb) vb[nb] = load_v(nb);
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
            if (nb + kPvD < 8) vb[(nb + kPvD) % (kPvD + 1)] = load_v(nb + kPvD);
#pragma unroll
            for (int mb = 0; mb < kMMB; ++mb) o[mb][nb] = mfma16x16x32<KIND>(pa[mb], vb[nb % (kPvD + 1)], o[mb][nb]);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int mb = 0; mb < kMMB; ++mb) lsum[mb] = mfma16x16x32<KIND>(pa[mb], kOnes, lsum[mb]);
    };

    // ---- main loop over a ring of R stages, tile s in stage s % R.  Each iteration waits
    // for tile `it` (the copies issued after it are tile it + 1's, Ring::kCopies per wave,
    // when the copies run two tiles ahead and there is a tile it + 1), then a barrier
    // publishes it and frees the stage that the iteration's copies overwrite (tile
    // it + kAhead's, in the stage of tile it + kAhead - R).  The loop holds no register
    // result of a global load, so the compiler adds no memory wait of its own.
    constexpr int R = Ring::kStages;
    auto stage = [&](int t) __attribute__((always_inline)) { return lds + (t % R) * Ring::kStageBytes; };
    const int n_sub = (int)((wend + kSubKeys - 1) / kSubKeys);   // sub-tiles holding keys of this wave
    u32x4 pa[kMMB];
    for (int t = 0; t < Ring::kAhead && t < n_tiles; ++t) issue(t, stage(t));
    for (int it = 0; it < n_tiles; ++it) {
        if (Ring::kAhead == 2 && it + 1 < n_tiles) wait_vm<Ring::kCopies>();
        else wait_vm0();
        lds_barrier();
        if (it + Ring::kAhead < n_tiles) issue(it + Ring::kAhead, stage(it + Ring::kAhead));
        const unsigned char *cur = stage(it);
        const int64_t kt = (int64_t)it * kMKeys;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            if (2 * it + sub < n_sub) {
                scores(cur, kt + sub * kSubKeys, sub * kSubKeys, pa);
                pv(cur, sub * kSubKeys, pa);
            }
        }
    }

    // out = O / l (rows with no visible key: 0)
#pragma unroll
    for (int mb = 0; mb < kMMB; ++mb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float ir = lsum[mb][r] > 0.f ? 1.f / lsum[mb][r] : 0.f;
            const int t = tw + mb * 16 + 4 * g + r;
            if (t < a.n_tok) {
                float *op = a.out + ((int64_t)t * a.n_head + head) * kMDV + l16;
#pragma unroll
                for (int nb = 0; nb < 8; ++nb) op[16 * nb] = o[mb][nb][r] * ir;
            }
        }
    }
}

}  // namespace

hipError_t launch_mha(const MhaArgs &a, int kv_kind, hipStream_t stream) {
    const dim3 grid((unsigned)((a.n_tok + kMTokens - 1) / kMTokens) * (unsigned)a.n_head), block(kMNW * 64);
    const bool m = a.mask != nullptr;
    void (*kern)(MhaArgs);
    if (kv_kind == KV_BF16)
        kern = m ? mha_kernel<KV_BF16, true> : mha_kernel<KV_BF16, false>;
    else if (kv_kind == KV_F16)
        kern = m ? mha_kernel<KV_F16, true> : mha_kernel<KV_F16, false>;
    else
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(kern, grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace mlafa
