// compact.hip -- single-scan sparse-mask index compaction for gfx950.
//
// For each f16 mask row, write the ascending list of cells whose mask is not -inf and
// its length.  The scheme follows the sparse-FA commit text ("llama.cpp Vulkan backend
// adds sparse Flash Attention for quantized K/V", b11413): split the row into
// contiguous segments, one per subgroup; count the kept cells of each segment with
// ballots over coalesced loads; one scan over the segment counts gives every segment
// its output offset; the list stays ascending.  The superseded design (one workgroup
// walking the row in 1024-cell chunks with a workgroup scan per chunk) is not used.
//
// gfx950 specifics: one workgroup of 16 wave64s per row; each lane loads 16 bytes
// (8 cells) per step, so a wave covers 512 consecutive cells per load, and whole batches
// of 8 steps issue their 8 loads back to back before any is used (a row's segments are
// otherwise walked one memory round trip per step).  Per-lane kept
// counts (0..8) are prefix-summed across the wave with four ballots (one per count
// bit) and mbcnt, so the scan inside a wave costs no LDS.  Pass 1 also leaves each
// lane's 8 kept bits in LDS (a byte per 8 cells, for rows of up to 2^20 cells), so pass 2
// reads the row's mask only once in all.  Rows whose base is not 16-byte aligned take a
// one-cell-per-lane path with the same structure (and re-read the mask).
#include "mla_fa_internal.h"

namespace mlafa {
namespace {

typedef unsigned short u16x8 __attribute__((__vector_size__(16)));
constexpr int kWaves = 16;
constexpr unsigned short kNegInf = 0xFC00;

__device__ __forceinline__ unsigned lanes_below(unsigned long long m) {
    return __builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
}

// Kept-cell bits (bit e = cell base+e) of the 8 cells a lane covers; cells at or past
// n_kv count as not kept.
__device__ __forceinline__ unsigned kept_bits8(const unsigned short *row, int64_t base, int64_t n_kv) {
    unsigned bits = 0;
    if (base + 8 <= n_kv) {
        const u16x8 v = *reinterpret_cast<const u16x8 *>(row + base);
#pragma unroll
        for (int e = 0; e < 8; ++e) bits |= (unsigned)(v[e] != kNegInf) << e;
    } else {
        for (int e = 0; e < 8; ++e)
            if (base + e < n_kv) bits |= (unsigned)(row[base + e] != kNegInf) << e;
    }
    return bits;
}

// Exclusive prefix (over lanes below) and wave total of per-lane counts c in [0, 15].
__device__ __forceinline__ void wave_scan4(unsigned c, unsigned &below, unsigned &total) {
    below = 0;
    total = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const unsigned long long m = __builtin_amdgcn_ballot_w64((c >> b) & 1u);
        below += lanes_below(m) << b;
        total += (unsigned)__builtin_popcountll(m) << b;
    }
}

// Rows of up to kLdsCells cells keep pass 1's kept-bits in LDS (one byte per 8 cells, in
// dynamic LDS sized to the row), so pass 2 reads no mask bytes from memory again.
constexpr int64_t kLdsCells = 1 << 20;

__global__ void __launch_bounds__(kWaves * 64) compact_kernel(const unsigned short *__restrict__ mask,
                                                              int64_t row_stride, int64_t n_kv,
                                                              int32_t *__restrict__ idx,
                                                              int64_t idx_stride,
                                                              int32_t *__restrict__ count,
                                                              int keep_bits) {
    __shared__ unsigned seg_count[kWaves];
    extern __shared__ unsigned char kbits[];          // byte c / 8: kept bits of cells c .. c + 7
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const unsigned short *row = mask + (int64_t)blockIdx.x * row_stride;
    int32_t *out = idx + (int64_t)blockIdx.x * idx_stride;
    const bool vec = (reinterpret_cast<uintptr_t>(row) & 15) == 0;
    const bool keep = vec && keep_bits;                // LDS bits (launch sized them for n_kv)
    const int step = vec ? 512 : 64;                         // cells per wave per load
    // contiguous segment of this wave, a whole number of load steps
    int64_t seg = (n_kv + kWaves - 1) / kWaves;
    seg = (seg + step - 1) / step * step;
    const int64_t s0 = (int64_t)wave * seg;
    const int64_t s1 = s0 + seg < n_kv ? s0 + seg : n_kv;

    // pass 1: count this segment's kept cells (whole batches of kBatch steps first); a
    // lane's 8 cells start at a multiple of 8, and only bytes of this segment are written
    constexpr int kBatch = 8;
    unsigned my_total = 0;
    int64_t b = s0;
    if (vec) {
        for (; b + kBatch * 512 <= s1; b += kBatch * 512) {
            u16x8 v[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) v[u] = *reinterpret_cast<const u16x8 *>(row + b + 512 * u + 8 * lane);
            unsigned c = 0;
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                unsigned k = 0;
#pragma unroll
                for (int e = 0; e < 8; ++e) k |= (unsigned)(v[u][e] != kNegInf) << e;
                if (keep) kbits[(b + 512 * u) / 8 + lane] = (unsigned char)k;
                c += __builtin_popcount(k);
            }
            // c <= 64: the wave total by ballots over its 7 bits
#pragma unroll
            for (int bit = 0; bit < 7; ++bit)
                my_total += (unsigned)__builtin_popcountll(__builtin_amdgcn_ballot_w64((c >> bit) & 1u)) << bit;
        }
    }
    for (; b < s1; b += step) {
        if (vec) {
            const int64_t base = b + 8 * lane;
            const unsigned k = kept_bits8(row, base, s1);
            if (keep && base < s1) kbits[base / 8] = (unsigned char)k;
            unsigned below, tot;
            wave_scan4(__builtin_popcount(k), below, tot);
            my_total += tot;
        } else {
            const int64_t j = b + lane;
            const bool kept = j < s1 && row[j] != kNegInf;
            my_total += (unsigned)__builtin_popcountll(__builtin_amdgcn_ballot_w64(kept));
        }
    }
    if (lane == 0) seg_count[wave] = my_total;
    __syncthreads();
    // one exclusive scan over the segment counts
    unsigned offset = 0, all = 0;
    for (int i = 0; i < kWaves; ++i) {
        const unsigned c = seg_count[i];
        offset += i < wave ? c : 0u;
        all += c;
    }
    if (threadIdx.x == 0) count[blockIdx.x] = (int32_t)all;

    // pass 2: write this segment's kept cells, ascending (whole batches first); the kept
    // bits come from LDS when pass 1 left them there, else from the mask again
    b = s0;
    if (vec) {
        for (; b + kBatch * 512 <= s1; b += kBatch * 512) {
            unsigned kk[kBatch];
            if (keep) {
#pragma unroll
                for (int u = 0; u < kBatch; ++u) kk[u] = kbits[(b + 512 * u) / 8 + lane];
            } else {
                u16x8 v[kBatch];
#pragma unroll
                for (int u = 0; u < kBatch; ++u) v[u] = *reinterpret_cast<const u16x8 *>(row + b + 512 * u + 8 * lane);
#pragma unroll
                for (int u = 0; u < kBatch; ++u) {
                    kk[u] = 0;
#pragma unroll
                    for (int e = 0; e < 8; ++e) kk[u] |= (unsigned)(v[u][e] != kNegInf) << e;
                }
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int64_t base = b + 512 * u + 8 * lane;
                unsigned k = kk[u];
                unsigned below, tot;
                wave_scan4(__builtin_popcount(k), below, tot);
                unsigned pos = offset + below;
                while (k) {
                    const int e = __builtin_ctz(k);
                    out[pos++] = (int32_t)(base + e);
                    k &= k - 1;
                }
                offset += tot;
            }
        }
    }
    for (; b < s1; b += step) {
        if (vec) {
            const int64_t base = b + 8 * lane;
            unsigned k = keep ? (base < s1 ? (unsigned)kbits[base / 8] : 0u) : kept_bits8(row, base, s1);
            unsigned below, tot;
            wave_scan4(__builtin_popcount(k), below, tot);
            unsigned pos = offset + below;
            while (k) {
                const int e = __builtin_ctz(k);
                out[pos++] = (int32_t)(base + e);
                k &= k - 1;
            }
            offset += tot;
        } else {
            const int64_t j = b + lane;
            const bool kept = j < s1 && row[j] != kNegInf;
            const unsigned long long m = __builtin_amdgcn_ballot_w64(kept);
            if (kept) out[offset + lanes_below(m)] = (int32_t)j;
            offset += (unsigned)__builtin_popcountll(m);
        }
    }
}

// ---------------------------------------------------------------------------------
// Multi-workgroup form, for callers that pass a workspace: the row is split into
// kChunk-cell chunks, one workgroup of kCWaves waves each, so a row is read by many CUs
// instead of one.  The same two passes as above, as two launches with the chunk counts
// in the workspace between them: count each chunk's kept cells; then every chunk sums
// the counts before it (its output offset), recounts its own cells, and writes them.
// Each wave covers 1024 consecutive cells as two 512-cell steps (16 bytes per lane).
constexpr int kChunk = 4096;
constexpr int kCWaves = 4;
static_assert(kChunk == kCWaves * 2 * 512, "two 512-cell steps per wave");

// kept bits of this lane's 8 cells in each of the wave's two steps
__device__ __forceinline__ void chunk_bits(const unsigned short *row, int64_t w0, int lane, int64_t n_kv,
                                           unsigned &k0, unsigned &k1) {
    k0 = kept_bits8(row, w0 + 8 * lane, n_kv);
    k1 = kept_bits8(row, w0 + 512 + 8 * lane, n_kv);
}

// wave total of per-lane counts c in [0, 31]
__device__ __forceinline__ unsigned wave_total5(unsigned c) {
    unsigned t = 0;
#pragma unroll
    for (int b = 0; b < 5; ++b) t += (unsigned)__builtin_popcountll(__builtin_amdgcn_ballot_w64((c >> b) & 1u)) << b;
    return t;
}

__global__ void __launch_bounds__(kCWaves * 64) chunk_count_kernel(const unsigned short *__restrict__ mask,
                                                                   int64_t row_stride, int64_t n_kv, int n_chunks,
                                                                   int32_t *__restrict__ ws) {
    __shared__ unsigned wc[kCWaves];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const unsigned short *row = mask + (int64_t)blockIdx.y * row_stride;
    unsigned k0, k1;
    chunk_bits(row, (int64_t)blockIdx.x * kChunk + wave * (kChunk / kCWaves), lane, n_kv, k0, k1);
    const unsigned t = wave_total5(__builtin_popcount(k0) + __builtin_popcount(k1));
    if (lane == 0) wc[wave] = t;
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned all = 0;
#pragma unroll
        for (int i = 0; i < kCWaves; ++i) all += wc[i];
        ws[(int64_t)blockIdx.y * n_chunks + blockIdx.x] = (int32_t)all;
    }
}

__global__ void __launch_bounds__(kCWaves * 64) chunk_write_kernel(const unsigned short *__restrict__ mask,
                                                                   int64_t row_stride, int64_t n_kv, int n_chunks,
                                                                   const int32_t *__restrict__ ws,
                                                                   int32_t *__restrict__ idx, int64_t idx_stride,
                                                                   int32_t *__restrict__ count) {
    __shared__ unsigned red[2][kCWaves];
    __shared__ unsigned wc[kCWaves];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = blockIdx.x;
    const unsigned short *row = mask + (int64_t)blockIdx.y * row_stride;
    const int32_t *cnt = ws + (int64_t)blockIdx.y * n_chunks;
    // this chunk's kept bits (loads first), then the counts of the chunks before it
    const int64_t w0 = (int64_t)c * kChunk + wave * (kChunk / kCWaves);
    unsigned k0, k1;
    chunk_bits(row, w0, lane, n_kv, k0, k1);
    unsigned pre = 0, all = 0;
    for (int i = threadIdx.x; i < n_chunks; i += kCWaves * 64) {
        const unsigned v = (unsigned)cnt[i];
        all += v;
        pre += i < c ? v : 0u;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        pre += __shfl_xor(pre, off);
        all += __shfl_xor(all, off);
    }
    const unsigned t = wave_total5(__builtin_popcount(k0) + __builtin_popcount(k1));
    if (lane == 0) {
        red[0][wave] = pre;
        red[1][wave] = all;
        wc[wave] = t;
    }
    __syncthreads();
    unsigned offset = 0, total = 0;
#pragma unroll
    for (int i = 0; i < kCWaves; ++i) {
        offset += red[0][i] + (i < wave ? wc[i] : 0u);
        total += red[1][i];
    }
    if (c == 0 && threadIdx.x == 0) count[blockIdx.y] = (int32_t)total;
    int32_t *out = idx + (int64_t)blockIdx.y * idx_stride;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int64_t base = w0 + 512 * s + 8 * lane;
        unsigned k = s == 0 ? k0 : k1;
        unsigned below, tot;
        wave_scan4(__builtin_popcount(k), below, tot);
        unsigned pos = offset + below;
        while (k) {
            const int e = __builtin_ctz(k);
            out[pos++] = (int32_t)(base + e);
            k &= k - 1;
        }
        offset += tot;
    }
}

}  // namespace

int64_t compact_chunks(int64_t n_kv) {
    return n_kv <= kCompactChunkedMax ? (n_kv + kChunk - 1) / kChunk : 0;
}

hipError_t launch_compact_chunked(const uint16_t *mask, int64_t mask_row_stride, int n_rows, int64_t n_kv,
                                  int32_t *idx, int64_t idx_row_stride, int32_t *count, int32_t *ws,
                                  hipStream_t stream) {
    const int n_chunks = (int)compact_chunks(n_kv);
    const auto *m = reinterpret_cast<const unsigned short *>(mask);
    hipLaunchKernelGGL(chunk_count_kernel, dim3(n_chunks, n_rows), dim3(kCWaves * 64), 0, stream, m,
                       mask_row_stride, n_kv, n_chunks, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(chunk_write_kernel, dim3(n_chunks, n_rows), dim3(kCWaves * 64), 0, stream, m,
                       mask_row_stride, n_kv, n_chunks, ws, idx, idx_row_stride, count);
    return hipGetLastError();
}

hipError_t launch_compact(const uint16_t *mask, int64_t mask_row_stride, int n_rows, int64_t n_kv,
                          int32_t *idx, int64_t idx_row_stride, int32_t *count,
                          hipStream_t stream) {
    // kept-bits in LDS for rows of up to kLdsCells cells: ceil(n_kv / 8) bytes, rounded to
    // whole 64-byte steps of a wave's segment
    const int keep = n_kv <= kLdsCells ? 1 : 0;
    const size_t bytes = keep ? (size_t)((n_kv + 511) / 512 * 64) : 0;
    hipLaunchKernelGGL(compact_kernel, dim3(n_rows), dim3(kWaves * 64), bytes, stream,
                       reinterpret_cast<const unsigned short *>(mask), mask_row_stride, n_kv, idx,
                       idx_row_stride, count, keep);
    return hipGetLastError();
}

}  // namespace mlafa
