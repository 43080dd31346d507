// peaks.hip -- achievable-peak micro-benchmarks for gfx950 (measurement support only).
//
// These kernels are not part of the attention path.  They measure what one MI355X
// actually delivers on the three resources the attention kernels are bound by, so that
// roofline fractions can be stated against measured peaks beside the published ones:
//   * HBM stream read: every byte of a large buffer read once with 16-byte loads, eight
//     loads in flight per thread (the buffer is sized past the 256 MB Infinity Cache);
//   * dense bf16 MFMA issue: v_mfma_f32_16x16x32_bf16 on eight independent accumulator
//     chains per wave, no memory traffic;
//   * LDS read: ds_read_b128 (row-major, conflict-free) or ds_read_b64_tr_b16 (the
//     transpose read the P.V operand uses) from a 64 KiB LDS array, eight or sixteen
//     reads in flight per wave.
// Every kernel folds what it read or computed into a sink that the host can check, so
// no work can be dropped by the compiler.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "mla_peaks.h"

namespace {

typedef unsigned u32x4 __attribute__((__vector_size__(16)));
typedef __bf16 bf16x8 __attribute__((__vector_size__(16)));
typedef float f32x4 __attribute__((__vector_size__(16)));
typedef short s16x4 __attribute__((__vector_size__(8)));
typedef unsigned u32x2 __attribute__((__vector_size__(8)));

constexpr int kThreads = 256;

__device__ __forceinline__ unsigned wg_xor(unsigned x) {
    __shared__ unsigned acc;
    if (threadIdx.x == 0) acc = 0;
    __syncthreads();
    atomicXor(&acc, x);
    __syncthreads();
    return acc;
}

__global__ void __launch_bounds__(kThreads) hbm_read_kernel(const u32x4 *__restrict__ p, int64_t n16,
                                                            unsigned *__restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    constexpr int kU = 8;
    for (; i + (kU - 1) * stride < n16; i += kU * stride) {
        u32x4 v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < kU; ++u) acc ^= v[u];
    }
    for (; i < n16; i += stride) acc ^= p[i];
    const unsigned x = wg_xor(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]);
    if (threadIdx.x == 0) sink[blockIdx.x] = x;
}

// a = 1.0 and b = `b_val` in every element: each MFMA adds 32 * b_val to every
// accumulator element, so after `iters` steps a thread's eight accumulators (4 values
// each) sum to exactly 8 * 4 * 32 * b_val * iters when that is representable.
__global__ void __launch_bounds__(kThreads) mfma_bf16_kernel(int iters, float b_val, float *__restrict__ sink) {
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)1.0f;
        b[e] = (__bf16)b_val;
    }
    // Eight chains in one asm block: left to itself the compiler rotates the accumulators
    // through spare AGPRs every iteration, which would time the moves as well.  A chain's
    // next MFMA is eight issues later, past the XDL result latency.  The compiler does not
    // see MFMAs inside the asm, so the wait states around the loop are explicit: 5 after
    // its own AGPR writes (accumulator set-up), 21 before it reads the results (8-pass
    // XDL result to VALU read).
    f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0, c4 = c0, c5 = c0, c6 = c0, c7 = c0;
    asm volatile("s_nop 4" : "+a"(c0), "+a"(c1), "+a"(c2), "+a"(c3), "+a"(c4), "+a"(c5), "+a"(c6), "+a"(c7));
    for (int it = 0; it < iters; ++it) {
        asm volatile(
            "v_mfma_f32_16x16x32_bf16 %0, %8, %9, %0\n\t"
            "v_mfma_f32_16x16x32_bf16 %1, %8, %9, %1\n\t"
            "v_mfma_f32_16x16x32_bf16 %2, %8, %9, %2\n\t"
            "v_mfma_f32_16x16x32_bf16 %3, %8, %9, %3\n\t"
            "v_mfma_f32_16x16x32_bf16 %4, %8, %9, %4\n\t"
            "v_mfma_f32_16x16x32_bf16 %5, %8, %9, %5\n\t"
            "v_mfma_f32_16x16x32_bf16 %6, %8, %9, %6\n\t"
            "v_mfma_f32_16x16x32_bf16 %7, %8, %9, %7"
            : "+a"(c0), "+a"(c1), "+a"(c2), "+a"(c3), "+a"(c4), "+a"(c5), "+a"(c6), "+a"(c7)
            : "v"(a), "v"(b));
    }
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" : "+a"(c0), "+a"(c1), "+a"(c2), "+a"(c3), "+a"(c4), "+a"(c5), "+a"(c6), "+a"(c7));
    const f32x4 t = ((c0 + c1) + (c2 + c3)) + ((c4 + c5) + (c6 + c7));
    sink[(int64_t)blockIdx.x * kThreads + threadIdx.x] = (t[0] + t[1]) + (t[2] + t[3]);
}

// 64 KiB of LDS per workgroup (two workgroups per CU).  Word w holds h(w) in both 16-bit
// halves, h(w) = (w * 40503) mod 2^16, so the host can predict what a b128 pass XORs to.
constexpr int kLdsWords = 16384;
__host__ __device__ constexpr unsigned lds_word(unsigned w) {
    return ((w * 40503u) & 0xFFFFu) * 0x10001u;
}

// One step of a wave: eight reads of 1 KiB (b128) or sixteen of 512 B (transpose), all
// issued before one wait inside the same asm block (so no read is in flight once the
// block ends); the outputs are early-clobber, since the first read returns while the
// address register is still needed by the later ones.  The asm always moves every byte; only the first dword of each read is
// folded into the result, which keeps the VALU work per LDS byte small enough not to be
// what is measured.  `p` is the LDS byte address of the wave's 8 KiB slot plus the
// lane's offset.
__device__ __forceinline__ unsigned lds_step_b128(unsigned p) {
    u32x4 r[8];
    asm volatile(
        "ds_read_b128 %0, %8\n\tds_read_b128 %1, %8 offset:1024\n\t"
        "ds_read_b128 %2, %8 offset:2048\n\tds_read_b128 %3, %8 offset:3072\n\t"
        "ds_read_b128 %4, %8 offset:4096\n\tds_read_b128 %5, %8 offset:5120\n\t"
        "ds_read_b128 %6, %8 offset:6144\n\tds_read_b128 %7, %8 offset:7168\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
        : "v"(p)
        : "memory");
    return (r[0][0] ^ r[1][0] ^ r[2][0]) ^ (r[3][0] ^ r[4][0] ^ r[5][0]) ^ (r[6][0] ^ r[7][0]);
}

__device__ __forceinline__ unsigned lds_step_tr16(unsigned p) {
    u32x2 r[16];
    asm volatile(
        "ds_read_b64_tr_b16 %0, %16\n\tds_read_b64_tr_b16 %1, %16 offset:512\n\t"
        "ds_read_b64_tr_b16 %2, %16 offset:1024\n\tds_read_b64_tr_b16 %3, %16 offset:1536\n\t"
        "ds_read_b64_tr_b16 %4, %16 offset:2048\n\tds_read_b64_tr_b16 %5, %16 offset:2560\n\t"
        "ds_read_b64_tr_b16 %6, %16 offset:3072\n\tds_read_b64_tr_b16 %7, %16 offset:3584\n\t"
        "ds_read_b64_tr_b16 %8, %16 offset:4096\n\tds_read_b64_tr_b16 %9, %16 offset:4608\n\t"
        "ds_read_b64_tr_b16 %10, %16 offset:5120\n\tds_read_b64_tr_b16 %11, %16 offset:5632\n\t"
        "ds_read_b64_tr_b16 %12, %16 offset:6144\n\tds_read_b64_tr_b16 %13, %16 offset:6656\n\t"
        "ds_read_b64_tr_b16 %14, %16 offset:7168\n\tds_read_b64_tr_b16 %15, %16 offset:7680\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]),
          "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]), "=&v"(r[12]), "=&v"(r[13]), "=&v"(r[14]), "=&v"(r[15])
        : "v"(p)
        : "memory");
    unsigned x = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) x ^= r[i][0];
    return x;
}

template <bool TR>
__global__ void __launch_bounds__(kThreads) lds_read_kernel(int iters, unsigned *__restrict__ sink) {
    __shared__ __attribute__((aligned(16))) unsigned lds[kLdsWords];
    for (int w = threadIdx.x; w < kLdsWords; w += kThreads) lds[w] = lds_word((unsigned)w);
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // b128: lane l reads 16 B at byte 16 l of each KiB; transpose: lane l reads 8 B at row
    // l / 4 of 32-byte rows, column 8 (l % 4), so each read covers 512 contiguous bytes
    const unsigned lane_off = TR ? (unsigned)((lane >> 2) * 32 + (lane & 3) * 8) : (unsigned)(lane * 16);
    const unsigned base = (unsigned)(uintptr_t)(__attribute__((address_space(3))) unsigned *)lds;
    unsigned acc = 0;
    for (int it = 0; it < iters; ++it) {
        // the wave's 8 KiB slot alternates between two halves of the array with `it`
        const unsigned p = base + (unsigned)(((it & 1) * 4 + wave) * 8192) + lane_off;
        acc ^= TR ? lds_step_tr16(p) : lds_step_b128(p);
    }
    const unsigned x = wg_xor(acc);
    if (threadIdx.x == 0) sink[blockIdx.x] = x;
}

}  // namespace

extern "C" {

int mla_peak_hbm_read(const void *buf, size_t bytes, unsigned *sink, int n_wg, void *stream) {
    if (!buf || !sink || n_wg < 1 || bytes == 0 || bytes % 16 || (reinterpret_cast<uintptr_t>(buf) & 15))
        return -1;
    hipLaunchKernelGGL(hbm_read_kernel, dim3(n_wg), dim3(kThreads), 0, (hipStream_t)stream,
                       static_cast<const u32x4 *>(buf), (int64_t)(bytes / 16), sink);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

int mla_peak_mfma_bf16(int iters, float b_val, float *sink, int n_wg, void *stream) {
    if (!sink || n_wg < 1 || iters < 1) return -1;
    hipLaunchKernelGGL(mfma_bf16_kernel, dim3(n_wg), dim3(kThreads), 0, (hipStream_t)stream, iters, b_val, sink);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

int mla_peak_lds_read(int iters, int transpose, unsigned *sink, int n_wg, void *stream) {
    if (!sink || n_wg < 1 || iters < 1) return -1;
    if (transpose)
        hipLaunchKernelGGL(lds_read_kernel<true>, dim3(n_wg), dim3(kThreads), 0, (hipStream_t)stream, iters, sink);
    else
        hipLaunchKernelGGL(lds_read_kernel<false>, dim3(n_wg), dim3(kThreads), 0, (hipStream_t)stream, iters, sink);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
