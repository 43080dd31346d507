// proj.hip -- the per-head projections either side of absorbed MLA attention (gfx950).
//
// The per-head up-projection of the latent cache is split into W_UK (key dims from the
// 512 latent) and W_UV (value dims from the latent); rather than decompressing every
// cached row, W_UK is folded into the query and W_UV applied to the attention output
// ("ik_llama.cpp -mla flag deep-dive": wkv_b split per head into wk_b / wv_b; "Vulkan
// backend fused Flash Attention: DeepSeek MLA local inference", sections 3.2-3.3).  Both
// are per-head products C[r][h] = A[r][h] . W[h]^T with W stored output-major (a linear
// layer's [out][in]), so both MFMA operands are contiguous along the reduction:
//   query side:  q[r][h][0:512] = W_UK[h] q_nope[r][h]   (K = 128, N = 512), written as
//                16-bit values straight into the 576-wide query rows the attention
//                kernel reads, with q_pe copied into columns 512..575;
//   output side: out[r][h] = W_UV[h] O[r][h]             (K = 512, N = 128), O the fp32
//                latent attention output, split into a 16-bit head and a 16-bit
//                remainder, each an MFMA operand (two MFMAs per block).
//
// A workgroup (4 waves) computes a 64-row x 128-column tile of one head; wave (wr, wc)
// the 32 x 64 sub-tile at rows 32 wr, columns 64 wc: 2 x 4 blocks of 16x16x32 MFMAs per
// 32-wide reduction step.  Operands are loaded straight from global memory into MFMA
// layout (lane: row or column l % 16, reduction elements 8 (l / 16) .. + 7, one 16-byte
// load), one step ahead of the MFMAs.  These products are small beside the attention
// (decode: bound by the 16 MB of weights per side; prefill: ~2% of the attention flops),
// so the kernel stays simple.
#include "mla_fa_internal.h"

namespace mlafa {
namespace {

#include "device_common.h"

constexpr int kPRows = 64, kPCols = 128;        // workgroup tile

// 16-bit value back to fp32 (exact)
template <int KIND> __device__ __forceinline__ float unpack_lo(unsigned v) {
    if constexpr (KIND == KV_BF16)
        return bf16_bits_to_f32(v & 0xFFFFu);
    else
        return f16_bits_to_f32((unsigned short)(v & 0xFFFFu));
}

// A operand, 8 reduction elements.  16-bit A is loaded as is.  An fp32 A is split into a
// 16-bit head and the 16-bit rounding of its remainder (a = hi + lo to ~16 significant
// bits), both used as MFMA operands, so the product is not limited by one 16-bit rounding
// of A.
template <int KIND, bool A_F32>
__device__ __forceinline__ void load_a(const ProjArgs &p, int row, int h, int k, u32x4 &hi, u32x4 &lo) {
    if constexpr (A_F32) {
        const float *src = static_cast<const float *>(p.a) + (int64_t)row * p.a_rs + (int64_t)h * p.a_hs + k;
        const f32x4 x0 = *reinterpret_cast<const f32x4 *>(src);
        const f32x4 x1 = *reinterpret_cast<const f32x4 *>(src + 4);
        const float x[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const unsigned ph = pack_p<KIND>(x[2 * j], x[2 * j + 1]);
            hi[j] = ph;
            lo[j] = pack_p<KIND>(x[2 * j] - unpack_lo<KIND>(ph), x[2 * j + 1] - unpack_lo<KIND>(ph >> 16));
        }
    } else {
        const uint16_t *src = static_cast<const uint16_t *>(p.a) + (int64_t)row * p.a_rs + (int64_t)h * p.a_hs + k;
        hi = *reinterpret_cast<const u32x4 *>(src);
        lo = u32x4{0u, 0u, 0u, 0u};
    }
}

template <int KIND, bool A_F32, bool C_F32>
__global__ void __launch_bounds__(256) proj_kernel(ProjArgs p) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 4, l16 = lane & 15;
    const int h = blockIdx.y;
    const int n_ct = p.N / kPCols;
    const int mt = blockIdx.x / n_ct, nt = blockIdx.x % n_ct;
    const int row0 = mt * kPRows + 32 * (wave & 1);
    const int col0 = nt * kPCols + 64 * (wave >> 1);

    // this lane's operand rows / columns (rows past M re-read row M - 1 and are not stored)
    int arow[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const int r = row0 + 16 * rb + l16;
        arow[rb] = r < p.M ? r : p.M - 1;
    }
    const uint16_t *wrow[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) wrow[cb] = p.w + ((int64_t)h * p.N + col0 + 16 * cb + l16) * p.K + 8 * g;

    f32x4 acc[2][4];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 av[2][2], al[2][2], bv[2][4];           // [buffer][block]
    auto load = [&](int ks, int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) load_a<KIND, A_F32>(p, arow[rb], h, 32 * ks + 8 * g, av[buf][rb], al[buf][rb]);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) bv[buf][cb] = *reinterpret_cast<const u32x4 *>(wrow[cb] + 32 * ks);
    };
    const int n_ks = p.K / 32;
    load(0, 0);
    for (int ks = 0; ks < n_ks; ks += 2) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int kk = ks + half;
            if (kk + 1 < n_ks) load(kk + 1, half ^ 1);
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) {
                    acc[rb][cb] = mfma16x16x32<KIND>(av[half][rb], bv[half][cb], acc[rb][cb]);
                    if constexpr (A_F32) acc[rb][cb] = mfma16x16x32<KIND>(al[half][rb], bv[half][cb], acc[rb][cb]);
                }
        }
    }

    // C element (row 16 rb + 4 g + r, column 16 cb + l16) of the wave's sub-tile
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = row0 + 16 * rb + 4 * g + r;
            if (row >= p.M) continue;
            const int64_t base = (int64_t)row * p.c_rs + (int64_t)h * p.c_hs + col0 + l16;
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                if constexpr (C_F32) {
                    static_cast<float *>(p.c)[base + 16 * cb] = acc[rb][cb][r];
                } else {
                    const unsigned pk = pack_p<KIND>(acc[rb][cb][r], 0.f);
                    static_cast<uint16_t *>(p.c)[base + 16 * cb] = (uint16_t)(pk & 0xFFFFu);
                }
            }
        }

    // the RoPE part of the query, copied next to the projected part (first column tile)
    if (p.extra && nt == 0) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int q = threadIdx.x + 256 * i;          // 64 rows x 8 chunks of 16 bytes
            const int row = mt * kPRows + (q >> 3), part = q & 7;
            if (row < p.M) {
                const u32x4 v = *reinterpret_cast<const u32x4 *>(p.extra + (int64_t)row * p.extra_rs +
                                                                 (int64_t)h * p.extra_hs + 8 * part);
                *reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(p.c) + (int64_t)row * p.c_rs +
                                           (int64_t)h * p.c_hs + p.N + 8 * part) = v;
            }
        }
    }
}

// Few rows (decode: M <= 16): the product is bound by reading W, and a 64-row tile would
// leave most workgroups walking K one load round trip at a time.  A workgroup here takes
// 16 rows x 64 columns of one head and its four waves split K into quarters, each loading
// its whole quarter (at most 4 steps of 32) before the MFMAs, then the four partial tiles
// are summed through LDS.
constexpr int kSRows = 16, kSCols = 64, kSMaxSteps = 4;

template <int KIND, bool A_F32, bool C_F32>
__global__ void __launch_bounds__(256) proj_skinny_kernel(ProjArgs p) {
    __shared__ float red[4][4][4][64];            // [wave][column block][register][lane]
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 4, l16 = lane & 15;
    const int h = blockIdx.y;
    const int n_ct = p.N / kSCols;
    const int mt = blockIdx.x / n_ct, nt = blockIdx.x % n_ct;
    const int col0 = nt * kSCols;
    const int r_ = mt * kSRows + l16;
    const int arow = r_ < p.M ? r_ : p.M - 1;
    const int kq = p.K / 4, steps = kq / 32;      // this wave's K quarter
    const int k0 = wave * kq;

    u32x4 av[kSMaxSteps], al[kSMaxSteps], bv[kSMaxSteps][4];
#pragma unroll
    for (int s = 0; s < kSMaxSteps; ++s) {
        if (s < steps) {
            const int k = k0 + 32 * s + 8 * g;
            load_a<KIND, A_F32>(p, arow, h, k, av[s], al[s]);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
                bv[s][cb] = *reinterpret_cast<const u32x4 *>(p.w + ((int64_t)h * p.N + col0 + 16 * cb + l16) * p.K + k);
        }
    }
    f32x4 acc[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kSMaxSteps; ++s)
        if (s < steps)
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                acc[cb] = mfma16x16x32<KIND>(av[s], bv[s][cb], acc[cb]);
                if constexpr (A_F32) acc[cb] = mfma16x16x32<KIND>(al[s], bv[s][cb], acc[cb]);
            }
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][cb][r][lane] = acc[cb][r];
    __syncthreads();
    // thread t sums column block t / 64's four registers over the four waves
    const int cb = threadIdx.x >> 6;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float v = red[0][cb][r][lane] + red[1][cb][r][lane] + red[2][cb][r][lane] + red[3][cb][r][lane];
        const int row = mt * kSRows + 4 * g + r;
        if (row < p.M) {
            const int64_t o = (int64_t)row * p.c_rs + (int64_t)h * p.c_hs + col0 + 16 * cb + l16;
            if constexpr (C_F32)
                static_cast<float *>(p.c)[o] = v;
            else
                static_cast<uint16_t *>(p.c)[o] = (uint16_t)(pack_p<KIND>(v, 0.f) & 0xFFFFu);
        }
    }
    // the RoPE part of the query (first column tile): 16 rows x 8 chunks of 16 bytes
    if (p.extra && nt == 0 && threadIdx.x < kSRows * 8) {
        const int row = mt * kSRows + (threadIdx.x >> 3), part = threadIdx.x & 7;
        if (row < p.M) {
            const u32x4 v = *reinterpret_cast<const u32x4 *>(p.extra + (int64_t)row * p.extra_rs +
                                                             (int64_t)h * p.extra_hs + 8 * part);
            *reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(p.c) + (int64_t)row * p.c_rs + (int64_t)h * p.c_hs +
                                       p.N + 8 * part) = v;
        }
    }
}

// ---------------------------------------------------------------------------------
// Split merge + output projection in one launch (the epilogue of split absorbed
// decode).  A workgroup takes 4 query rows of one head and 64 of the 128 output
// columns: it starts its share of W (64 x 512, 64 KiB) loading, merges the 4 rows'
// partials into fp32 O in LDS (the merge rule of the plain path: weights 2^(m_i - m*),
// empty splits weigh 0, per-half scales of the f16 values), then computes
// C[n][r] = W[n] . O[r] on MFMA with the rows as the B operand's columns (4 of 16 used),
// O split into a 16-bit head and remainder as in the separate projection.  The two
// column halves of a (row block, head) are workgroups x and x + 8, so that they run on
// one XCD and can share the partials through its L2.  (One workgroup per (row block,
// head) over all 128 columns reads the partials once but runs on half the CUs: 12.0
// against 10.2 us on the 4 x 128-head decode.)
constexpr int kMPRows = 4;                      // query rows per workgroup
constexpr int kMPThreads = 512;
constexpr int kMPBatch = 16;                    // partial loads in flight per thread
constexpr int kMPPer = kMaxSplits / 128;        // splits per factor thread

template <int KIND>
__global__ void __launch_bounds__(kMPThreads) merge_proj_kernel(MergeProjArgs a) {
    __shared__ float fac_s[2][kMPRows][kMaxSplits];   // per-half factors: weight x scale
    __shared__ float red_m[kMPThreads / 64], red_l[kMPThreads / 64];
    __shared__ f32x4 part_s[kMPThreads];               // split group 1's sums
    __shared__ __attribute__((aligned(16))) float o_s[kMPRows][kDV];
    __shared__ f32x4 acc_s[4][64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, l16 = lane & 15;
    const int wg = blockIdx.x;
    const int half = (wg >> 3) & 1;                    // output columns 64 half .. + 63
    const int rest = (wg >> 4) * 8 + (wg & 7);         // (row block, head)
    const int n_rb = (a.n_rows + kMPRows - 1) / kMPRows;
    if (rest >= n_rb * a.n_head) return;
    const int h = rest % a.n_head, r0 = (rest / a.n_head) * kMPRows;
    const int nrow = a.n_rows - r0 < kMPRows ? a.n_rows - r0 : kMPRows;
    const int S = a.n_split;
    const int64_t RH = (int64_t)a.n_rows * a.n_head;
    const float *wm = a.ws;
    const float *wl = wm + (int64_t)S * RH;
    const f32x2v *wsc = reinterpret_cast<const f32x2v *>(wl + (int64_t)S * RH);
    const uint16_t *wo = reinterpret_cast<const uint16_t *>(wsc + (int64_t)S * RH);
    // Row r of the block: the (slot, head) entry of its first split, the stride between
    // its splits, and their number.  Under a length-proportional plan its splits are the
    // slots the row table gives it (a row with none reads slot 0 and weighs it 0).
    auto row_splits = [&](int r, int64_t &e0, int64_t &es, int &ns) __attribute__((always_inline)) {
        if (a.ragged) {
            const unsigned v = reinterpret_cast<const unsigned *>(a.ws + ragged_table_off(S, a.n_rows, a.n_head))[r0 + r];
            ns = (int)(v >> 16);
            e0 = (int64_t)(ns > 0 ? (int)(v & 0xFFFFu) : 0) * a.n_head + h;
            es = a.n_head;
        } else {
            e0 = (int64_t)(r0 + r) * a.n_head + h;
            es = RH;
            ns = S;
        }
    };

    // W rows of this wave: n-block nb of the half, reduction half kh (8 steps of 32)
    const int nb = wave & 3, kh = wave >> 2;
    const uint16_t *wp = a.w + ((int64_t)h * 128 + 64 * half + 16 * nb + l16) * kDV + 256 * kh + 8 * g;
    u32x4 wv[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) wv[s] = *reinterpret_cast<const u32x4 *>(wp + 32 * s);

    // partial O loads of this thread: (row pr, octet oc) of the block, splits sg, sg + 2, ...
    const int pair = tid & 255, sg = tid >> 8;
    const int pr = pair >> 6, oc = pair & 63;
    const bool prow = pr < nrow;
    int64_t pe0, pes;
    int ps;                                            // splits of row pr
    row_splits(prow ? pr : 0, pe0, pes, ps);
    const u32x4 *op = reinterpret_cast<const u32x4 *>(wo + pe0 * kDV) + oc;
    const int64_t step8 = pes * kDV / 8;              // stride between splits, in octets
    u32x4 v0[kMPBatch];
#pragma unroll
    for (int u = 0; u < kMPBatch; ++u) {
        const int i = sg + 2 * u;
        v0[u] = op[(int64_t)(i < ps ? i : 0) * step8];   // unconditional: no wait until used
    }

    // (m, l, scales) of row fr, splits ft, ft + 128, ...: max, weights, normaliser
    const int fr = tid >> 7, ft = tid & 127;
    const bool frow = fr < nrow;
    int64_t fe0, fes;
    int fs;                                            // splits of row fr
    row_splits(frow ? fr : 0, fe0, fes, fs);
    float mv[kMPPer], lv[kMPPer];
    f32x2v scv[kMPPer];
    float mloc = -INFINITY;
#pragma unroll
    for (int j = 0; j < kMPPer; ++j) {
        const int i = ft + 128 * j;
        mv[j] = -INFINITY;
        if (frow && i < fs) {
            mv[j] = wm[fe0 + i * fes];
            lv[j] = wl[fe0 + i * fes];
            scv[j] = wsc[fe0 + i * fes];
            mloc = fmaxf(mloc, mv[j]);
        }
    }
    for (int off = 32; off > 0; off >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, off));
    if (lane == 0) red_m[wave] = mloc;
    __syncthreads();
    const float mstar = fmaxf(red_m[2 * fr], red_m[2 * fr + 1]);
    float lloc = 0.f;
#pragma unroll
    for (int j = 0; j < kMPPer; ++j) {
        const int i = ft + 128 * j;
        if (frow && i < fs) {
            const float wgt = (mstar == -INFINITY || mv[j] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mv[j] - mstar);
            if (wgt != 0.f) lloc += wgt * lv[j];
            fac_s[0][fr][i] = wgt != 0.f ? wgt * scv[j][0] : 0.f;
            fac_s[1][fr][i] = wgt != 0.f ? wgt * scv[j][1] : 0.f;
        }
    }
    for (int off = 32; off > 0; off >>= 1) lloc += __shfl_xor(lloc, off);
    if (lane == 0) red_l[wave] = lloc;
    __syncthreads();

    // weighted sums of this thread's splits (rows past the block weigh 0)
    auto lo4 = [](u32x4 v) __attribute__((always_inline)) {
        return __builtin_convertvector(__builtin_bit_cast(f16x4v, u32x2{v[0], v[1]}), f32x4);
    };
    auto hi4 = [](u32x4 v) __attribute__((always_inline)) {
        return __builtin_convertvector(__builtin_bit_cast(f16x4v, u32x2{v[2], v[3]}), f32x4);
    };
    const float *f_s = fac_s[oc < 32 ? 0 : 1][pr];
    f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
#pragma unroll
    for (int u = 0; u < kMPBatch; ++u) {
        const int i = sg + 2 * u;
        const float wgt = prow && i < ps ? f_s[i] : 0.f;
        if (wgt != 0.f) {                              // unweighted splits may hold any bits
            a0 += wgt * lo4(v0[u]);
            a1 += wgt * hi4(v0[u]);
        }
    }
    for (int i0 = sg + 2 * kMPBatch; i0 < ps; i0 += 2 * kMPBatch) {
        u32x4 v[kMPBatch];
        float wt[kMPBatch];
#pragma unroll
        for (int u = 0; u < kMPBatch; ++u) {
            const int i = i0 + 2 * u;
            wt[u] = prow && i < ps ? f_s[i] : 0.f;
            v[u] = op[(int64_t)(i < ps ? i : 0) * step8];
        }
#pragma unroll
        for (int u = 0; u < kMPBatch; ++u)
            if (wt[u] != 0.f) {
                a0 += wt[u] * lo4(v[u]);
                a1 += wt[u] * hi4(v[u]);
            }
    }
    if (sg == 1) {
        part_s[2 * pair] = a0;
        part_s[2 * pair + 1] = a1;
    }
    __syncthreads();
    if (sg == 0) {
        a0 += part_s[2 * pair];
        a1 += part_s[2 * pair + 1];
        const float lsum = red_l[2 * pr] + red_l[2 * pr + 1];
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
        f32x4 *dst = reinterpret_cast<f32x4 *>(&o_s[pr][8 * oc]);
        dst[0] = a0 * inv;
        dst[1] = a1 * inv;
    }
    __syncthreads();

    // C[n][r] over this wave's reduction half: B column l16 = row l16 of the block
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        u32x4 bh = {0u, 0u, 0u, 0u}, bl = bh;
        if (l16 < nrow) {
            const int k = 256 * kh + 32 * s + 8 * g;
            const f32x4 x0 = *reinterpret_cast<const f32x4 *>(&o_s[l16][k]);
            const f32x4 x1 = *reinterpret_cast<const f32x4 *>(&o_s[l16][k + 4]);
            const float x[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const unsigned ph = pack_p<KIND>(x[2 * j], x[2 * j + 1]);
                bh[j] = ph;
                bl[j] = pack_p<KIND>(x[2 * j] - unpack_lo<KIND>(ph), x[2 * j + 1] - unpack_lo<KIND>(ph >> 16));
            }
        }
        acc = mfma16x16x32<KIND>(wv[s], bh, acc);
        acc = mfma16x16x32<KIND>(wv[s], bl, acc);
    }
    if (kh == 1) acc_s[nb][lane] = acc;
    __syncthreads();
    if (kh == 0 && l16 < nrow) {                       // lane: outputs 16 nb + 4 g .. + 3 of row l16
        acc += acc_s[nb][lane];
        *reinterpret_cast<f32x4 *>(a.out + (int64_t)(r0 + l16) * a.out_rs + (int64_t)h * 128 + 64 * half + 16 * nb +
                                   4 * g) = acc;
    }
}

}  // namespace

hipError_t launch_merge_proj(const MergeProjArgs &a, int kind, hipStream_t stream) {
    if (a.n_rows < 1 || a.n_head < 1 || a.n_split < 2 || a.n_split > kMaxSplits) return hipErrorInvalidValue;
    const int64_t blocks = (int64_t)((a.n_rows + kMPRows - 1) / kMPRows) * a.n_head;   // (row block, head)
    const int64_t grid = 16 * ((blocks + 7) / 8);       // two column halves, x and x + 8
    if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    void (*kern)(MergeProjArgs) = kind == KV_BF16 ? merge_proj_kernel<KV_BF16>
                                  : kind == KV_F16 ? merge_proj_kernel<KV_F16> : nullptr;
    if (!kern) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kMPThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_proj(const ProjArgs &p, int kind, bool a_f32, bool c_f32, hipStream_t stream) {
    if (p.M < 1 || p.H < 1 || p.N % kPCols || p.K % 128 || p.K > 4 * 32 * kSMaxSteps) return hipErrorInvalidValue;
    const bool skinny = p.M <= kSRows;
    const dim3 grid(skinny ? (unsigned)(p.N / kSCols)
                           : (unsigned)((p.M + kPRows - 1) / kPRows) * (unsigned)(p.N / kPCols),
                    (unsigned)p.H);
    void (*kern)(ProjArgs) = nullptr;
#define MLAFA_PROJ_PICK(K_, AF, CF) kern = skinny ? proj_skinny_kernel<K_, AF, CF> : proj_kernel<K_, AF, CF>
    if (kind == KV_BF16) {
        if (!a_f32 && !c_f32) MLAFA_PROJ_PICK(KV_BF16, false, false);
        else if (a_f32 && c_f32) MLAFA_PROJ_PICK(KV_BF16, true, true);
    } else if (kind == KV_F16) {
        if (!a_f32 && !c_f32) MLAFA_PROJ_PICK(KV_F16, false, false);
        else if (a_f32 && c_f32) MLAFA_PROJ_PICK(KV_F16, true, true);
    }
#undef MLAFA_PROJ_PICK
    if (!kern) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace mlafa
