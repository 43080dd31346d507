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
//     full-wave global_load_lds_dwordx4 copies into unpadded areas, double-buffered.
//     16-byte chunks are XOR-swizzled per key so that both read patterns are bank-conflict
//     free: K chunk c of key r sits at slot (c & ~7) | ((c & 7) ^ ((r >> 1) & 7)) (16 keys
//     reading one chunk hit 16 distinct bank groups); V chunk c of key r at slot
//     c ^ ((r & 7) << 1) (the transpose read's 8 keys x 32 bytes hit 16 distinct groups).
//   * Causal: token t sees keys j <= n_kv - n_tok + t.  Workgroups with later tokens are
//     dispatched first (they have the most keys); a wave skips the tiles its tokens cannot
//     see.  The optional f16 mask [n_tok][n_kv] is added to the scaled score (-inf drops
//     the cell); each lane loads the 8-byte runs of mask values for its own token before
//     the stage's copies are issued, so waiting for them never waits for a copy.
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

__device__ __forceinline__ int k_slot(int r, int c) { return (c & ~7) | ((c & 7) ^ ((r >> 1) & 7)); }
__device__ __forceinline__ int v_slot(int r, int c) { return c ^ ((r & 7) << 1); }

template <int KIND, bool MASK>
__global__ void __launch_bounds__(kMNW * 64, 1) mha_kernel(MhaArgs a) {
    __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * kMStage];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, l16 = lane & 15;
    const int head = blockIdx.y;
    const int tile = (int)gridDim.x - 1 - (int)blockIdx.x;   // later tokens first
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
    int64_t lim[kMMB];                                       // last key each lane's token sees
#pragma unroll
    for (int mb = 0; mb < kMMB; ++mb) {
        const int t = tw + mb * 16 + l16;
        const bool ok = t < a.n_tok;
        const u32x4 *qp = reinterpret_cast<const u32x4 *>(
            a.q + ((int64_t)(ok ? t : a.n_tok - 1) * a.n_head + head) * kMDK + 8 * g);
#pragma unroll
        for (int s = 0; s < 6; ++s) qreg[mb][s] = ok ? qp[4 * s] : u32x4{0u, 0u, 0u, 0u};
        lim[mb] = !ok ? -1 : (a.causal ? off + t : a.n_kv - 1);
    }
    wait_vm0();   // Q is in registers before the loop: no wait inside it counts these loads

    float m_run[kMMB], l_run[kMMB];
    f32x4 o[kMMB][8];
#pragma unroll
    for (int mb = 0; mb < kMMB; ++mb) {
        m_run[mb] = -INFINITY;
        l_run[mb] = 0.f;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) o[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // per-lane LDS read offsets: K (S^T A operand) row l16, chunk 4 s + g; V (P.V B operand
    // by transpose read) row 4 G + j / 4, byte 32 nb + 8 (j % 4) before the swizzle
    const int fk = (l16 >> 1) & 7;
    const int k_even = l16 * kMKRow + 16 * (g ^ fk);         // chunk & 7 = g      (s even)
    const int k_odd = l16 * kMKRow + 16 * ((4 + g) ^ fk);    // chunk & 7 = 4 + g  (s odd)
    const int vr = 4 * g + (l16 >> 2);
    const int v_base = kMKArea + vr * kMVRow + 8 * (lane & 3);
    const int v_x = (vr & 7) << 5;                            // 32 * (row & 7): the swizzle, in bytes

    // Copy stage `it` into `dst`: 24 K copies then 16 V copies of 1 KiB, spread over waves.
    auto issue = [&](int it, unsigned char *__restrict__ dst) __attribute__((always_inline)) {
        const int64_t kt = (int64_t)it * kMKeys;
        const int last = (int)((kend - kt) < kMKeys ? (kend - kt) : kMKeys) - 1;
        int ln = lane;
        asm volatile("" : "+v"(ln));
#pragma unroll
        for (int j = 0; j < (40 + kMNW - 1) / kMNW; ++j) {
            const int b = wave + j * kMNW;
            if (b < 24) {
                const int gs = b * 64 + ln;                  // slot index in the K area
                const int r = gs / 24, p = gs - (gs / 24) * 24;
                const int c = k_slot(r, p);                  // the swizzle is its own inverse
                const int rc = r < last ? r : last;
                const uint8_t *src = a.k + (kt + rc) * a.k_row_stride + (int64_t)head * kMKRow + 16 * c;
                __builtin_amdgcn_global_load_lds((const void *)src, (LDS_PTR(void))(dst + b * 1024), 16, 0, 0);
            } else if (b < 40) {
                const int vb = b - 24;
                const int r = 4 * vb + (ln >> 4), p = ln & 15;
                const int c = v_slot(r, p);
                const int rc = r < last ? r : last;
                const uint8_t *src = a.v + (kt + rc) * a.v_row_stride + (int64_t)head * kMVRow + 16 * c;
                __builtin_amdgcn_global_load_lds((const void *)src, (LDS_PTR(void))(dst + kMKArea + vb * 1024),
                                                 16, 0, 0);
            }
        }
    };

    constexpr int kQkD = 2, kPvD = 3;
    // One 32-key sub-tile (keys kt + sub0 ..) of stage `st` for this wave's 32 tokens.
    auto compute_sub = [&](const unsigned char *__restrict__ st, int64_t kt, int sub0, const u32x2 (&mk)[kMMB][2])
        __attribute__((always_inline)) {
        const unsigned char *sk = st + sub0 * kMKRow;
        f32x4 sacc[2][kMMB];
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
        // softmax per 16-token block (lane: token l16; keys 4g + i and 16 + 4g + i)
        u32x4 pa[kMMB];
        const int64_t kbase = kt + sub0;
#pragma unroll
        for (int mb = 0; mb < kMMB; ++mb) {
            float tv[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) tv[i] = sacc[i >> 2][mb][i & 3] * a.scale_log2;
            if constexpr (MASK) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const unsigned w = mk[mb][i >> 2][(i & 3) >> 1];
                    const unsigned short b = (unsigned short)((i & 1) ? (w >> 16) : (w & 0xFFFFu));
                    tv[i] += f16_bits_to_f32(b) * kLog2e;         // -inf stays -inf
                }
            }
            if (kbase + kSubKeys - 1 > lim[mb] || kbase + kSubKeys > a.n_kv) {   // edge of the range
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int64_t j = kbase + 16 * (i >> 2) + 4 * g + (i & 3);
                    if (j > lim[mb]) tv[i] = -INFINITY;
                }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < 8; ++i) mx = fmaxf(mx, tv[i]);
            mx = wave_max_groups(mx);
            const bool need = mx > m_run[mb] + kMRescaleThresh;
            if (__builtin_amdgcn_ballot_w64(need)) {
                const float alpha = need ? __builtin_amdgcn_exp2f(m_run[mb] - mx) : 1.f;
                if (need) m_run[mb] = mx;
                l_run[mb] *= alpha;
                float ar[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) ar[r] = shfl_f(alpha, 4 * g + r);
#pragma unroll
                for (int nb = 0; nb < 8; ++nb)
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
        // O += P . V (V of keys sub0 .. sub0 + 31, transpose reads through the swizzle)
        const unsigned char *sv = st + v_base + sub0 * kMVRow;
        u32x4 vb[kPvD + 1];
        auto load_v = [&](int nb) __attribute__((always_inline)) -> u32x4 {
            const int o_ = (32 * nb) ^ v_x;
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
    };

    // Mask values of this lane's tokens for keys kt + sub0 + 16 h + 4 g .. + 3, one aligned
    // 8-byte word each.  A word past the end of the row is replaced by the row's last word
    // (its keys lie past n_kv, so the range check drops them whatever the values are); the
    // word holding key n_kv - 1 may extend past the row end but not past its 8-byte word.
    const int64_t jmax = (a.n_kv - 1) & ~(int64_t)3;
    auto load_mask = [&](int64_t kt, int sub0, u32x2 (&mk)[kMMB][2]) __attribute__((always_inline)) {
#pragma unroll
        for (int mb = 0; mb < kMMB; ++mb) {
            const int t = tw + mb * 16 + l16;
            const uint16_t *row = a.mask + (int64_t)(t < a.n_tok ? t : a.n_tok - 1) * a.mask_row_stride;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int64_t j0 = kt + sub0 + 16 * h + 4 * g;
                mk[mb][h] = *reinterpret_cast<const u32x2 *>(row + (j0 < jmax ? j0 : jmax));
            }
        }
    };

    // One loop step: load the mask words of tile `it + 1` and start copying its K and V
    // into `next`, then compute tile `it` from `cur` with the mask words loaded one step
    // earlier.  Every load of the step is waited for at the top of the next iteration, so
    // no wait inside the compute counts a copy still in flight.
    u32x2 mk_cur[2][kMMB][2], mk_nxt[2][kMMB][2];
    auto step = [&](int it, unsigned char *__restrict__ next, const unsigned char *__restrict__ cur)
        __attribute__((always_inline)) {
        const int64_t kt = (int64_t)it * kMKeys;
        if (it + 1 < n_tiles) {
            if constexpr (MASK) {
#pragma unroll
                for (int sub = 0; sub < 2; ++sub)
                    if (kt + kMKeys + sub * kSubKeys < wend) load_mask(kt + kMKeys, sub * kSubKeys, mk_nxt[sub]);
            }
            issue(it + 1, next);
        }
        if (it >= 0) {
#pragma unroll
            for (int sub = 0; sub < 2; ++sub)
                if (kt + sub * kSubKeys < wend) compute_sub(cur, kt, sub * kSubKeys, mk_cur[sub]);
        }
        if constexpr (MASK) {
#pragma unroll
            for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                for (int mb = 0; mb < kMMB; ++mb)
#pragma unroll
                    for (int h = 0; h < 2; ++h) mk_cur[sub][mb][h] = mk_nxt[sub][mb][h];
        }
    };
    for (int it = -1; it < n_tiles; ++it) {
        if (it >= 0) {
            wait_vm0();
            __syncthreads();
        }
        unsigned char *next = lds + ((it + 1) & 1) * kMStage;
        const unsigned char *cur = lds + (it & 1) * kMStage;
        step(it, next, cur);
    }

    // out = O / l (rows with no visible key: 0)
#pragma unroll
    for (int mb = 0; mb < kMMB; ++mb) {
        l_run[mb] = wave_sum_groups(l_run[mb]);
        const float inv = l_run[mb] > 0.f ? 1.f / l_run[mb] : 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float ir = shfl_f(inv, 4 * g + r);
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
    const dim3 grid((a.n_tok + kMTokens - 1) / kMTokens, a.n_head), block(kMNW * 64);
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
