// Internal interface between the C-ABI host layer (api.hip) and the kernel
// translation units (attn.hip, compact.hip).  Not installed, not part of the ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mlafa {

constexpr int kDK = 576;                 // latent 512 + RoPE 64
constexpr int kDV = 512;                 // V = first 512 columns of the row
constexpr int kRowBytes16 = kDK * 2;     // an f16/bf16 latent row
constexpr int kQ8RowBytes = 18 * 34;     // a Q8_0 latent row
constexpr int kTileKeys = 64;            // keys per LDS-staged tile
constexpr int kMaxSplits = 1024;

enum KvKind { KV_BF16 = 0, KV_F16 = 1, KV_Q8 = 2 };

// Workgroup shapes.  H*: MB 16-head blocks per wave, NW waves, WK waves sharing one
// head set and splitting each tile's keys between them; heads per workgroup =
// (NW / WK) * 16 * MB.  P*: pair kernel (16-bit caches only), 32 heads per wave pair.
enum Shape { SHAPE_H16 = 0, SHAPE_H32 = 1, SHAPE_H64 = 2, SHAPE_H128 = 3, SHAPE_P64 = 4, SHAPE_P128 = 5 };

// Rows whose lengths only the device holds (per-sequence valid lengths, or index-list
// counts) can share the call's partial slots in proportion to their lengths instead of
// splitting every row into n_split pieces (budget > 0).  Each piece then covers at most C
// tiles, C the smallest value with sum over rows of ceil(tiles / C) <= budget, and piece j
// of row r fills partial slot P_r + j, P_r the pieces of rows 0 .. r-1.  The attention
// launch derives the plan from the lengths and leaves a row table (P_r, pieces of r) in the
// workspace's tail after the partials; the merge reads it.
constexpr int kRaggedRows = 256;         // rows such a plan can hold
struct Ragged {
    const int32_t *kv_len;         // [n_seq] valid cells, or nullptr
    const int32_t *count;          // [n_seq * n_tok] index-list lengths, or nullptr
    int64_t n_kv;
    int n_tok, causal;
    int rows;                      // n_seq * n_tok, at most kRaggedRows
    int budget;                    // pieces (at most rows * n_split); 0 = no such plan
};

struct AttnArgs {
    const uint16_t *q;             // [n_seq][n_tok][n_head][576]
    const uint8_t *kv;             // byte base of the cache
    int64_t kv_row_stride;         // bytes
    int64_t kv_seq_stride;         // bytes (0 = shared)
    const uint16_t *mask;          // f16 bits or nullptr
    int64_t mask_seq_stride;       // elements
    int64_t mask_tok_stride;       // elements
    const int32_t *kv_idx;         // sparse index lists or nullptr: row (s, t) at
    const int32_t *kv_idx_count;   //   kv_idx + s * idx_seq_stride + t * idx_tok_stride,
    int64_t idx_seq_stride;        //   its length at kv_idx_count[s * n_tok + t]
    int64_t idx_tok_stride;
    float *out;                    // [n_seq*n_tok][n_head][512], used when n_split == 1
    float *ws;                     // partials, used when n_split > 1
    int64_t n_kv;
    int64_t split_chunk;           // keys per split for dense rows (multiple of kTileKeys)
    int n_seq, n_tok, n_head;
    int causal;
    int n_split;
    int head_groups;               // workgroups along the head axis
    int grid_x;                    // blockIdx.x extent (head_groups * splits, padded)
    int q_bf16;                    // q bits are bf16 (else f16)
    float scale_log2;              // scale * log2(e)
    const int32_t *kv_len;         // [n_seq] valid cells per sequence, or nullptr (= n_kv)
    const float *alibi;            // [n_head] slope multiplying the mask of kept cells, or nullptr
    const float *sinks;            // [n_head] sink logits (natural log), or nullptr
    float cap_in;                  // softcap: score = cap_out * tanh(dot * cap_in) in log2 units;
    float cap_out;                 //   cap_in = 0 means no softcap
    int row_base;                  // query row of blockIdx.y = 0 (launches cover at most
                                   //   kMaxGridY rows each)
    Ragged ragged;                 // budget > 0: length-proportional pieces, one launch,
                                   //   blockIdx.x = piece (and head group)
};
constexpr int kMaxGridY = 65535;   // rows per launch (the grid's y extent)

// Split partials inside the workspace, for R = n_seq*n_tok rows, H heads, S splits, in
// this order: m [S][R][H] fp32 (log2 units), l [S][R][H] fp32, scale [S][R][H][2] fp32,
// O [S][R][H][512] f16 (slot = split * R + row; under a length-proportional plan slot =
// P_r + piece, the [S][R] slots read as one list), then a 1 KiB tail that holds that
// plan's row table.  O is the unnormalised output, each 256-column half stored times
// 2^(15 - e) where max |O| < 2^e over the half (the scale kept is 2^(e - 15)), so every
// value keeps f16's relative precision (2^-11) whatever the magnitude of the cache's
// values.
constexpr size_t kPartialEntryBytes = 4 * sizeof(float) + kDV * sizeof(uint16_t);   // 1040
constexpr size_t kRaggedTableBytes = kRaggedRows * sizeof(int32_t);
inline size_t partial_bytes(int64_t rows, int heads, int splits) {
    return (size_t)splits * rows * heads * kPartialEntryBytes + kRaggedTableBytes;
}
// The row table's offset in floats from the partials' base: one int32 per row, its first
// slot | its piece count << 16 (both at most kRaggedRows).
__host__ __device__ inline int64_t ragged_table_off(int splits, int rows, int heads) {
    return (int64_t)splits * rows * heads * (int64_t)(kPartialEntryBytes / sizeof(float));
}

// Per-head attention with separate K (192 wide) and V (128 wide), 16-bit types.
struct MhaArgs {
    const uint16_t *q;             // [n_tok][n_head][192]
    const uint8_t *k;              // key j, head h at k + j * k_row_stride + h * 384
    const uint8_t *v;              // key j, head h at v + j * v_row_stride + h * 256
    int64_t k_row_stride;          // bytes
    int64_t v_row_stride;          // bytes
    const uint16_t *mask;          // f16 bits, token t at mask + t * mask_row_stride, or nullptr
    int64_t mask_row_stride;       // elements, a multiple of 8 (16-byte mask copies)
    float *out;                    // [n_tok][n_head][128] fp32
    int64_t n_kv;
    int n_tok, n_head;
    int causal;                    // token t sees keys j <= n_kv - n_tok + t
    float scale_log2;              // scale * log2(e)
};

// Per-head product C[r][h] = A[r][h] . W[h]^T (W output-major, 16-bit, same type as the
// MFMA): element (r, h, k) of A at a + r*a_rs + h*a_hs + k, W[h][n][k] at
// w + (h*N + n)*K + k, C (r, h, n) at c + r*c_rs + h*c_hs + n (all in elements); A and C
// 16-bit or fp32.  With `extra`, the 16-bit row part (r, h) at extra + r*extra_rs +
// h*extra_hs (64 elements) is copied to C columns N .. N + 63.
struct ProjArgs {
    const void *a;
    int64_t a_rs, a_hs;
    const uint16_t *w;
    void *c;
    int64_t c_rs, c_hs;
    const uint16_t *extra;
    int64_t extra_rs, extra_hs;
    int M, N, K, H;
};

// The merge of split partials fused with the output projection of absorbed attention:
// out[r][h][n] = sum_k W[h][n][k] * O[r][h][k] for n < 128, k < 512, where O[r][h] is the
// merged latent output (as merge_kernel computes it); W 16-bit [H][128][512], out fp32 at
// out + r * out_rs + h * 128 + n.
struct MergeProjArgs {
    const float *ws;               // the split partials (layout of partial_bytes)
    const uint16_t *w;
    float *out;
    int64_t out_rs;                // elements
    int n_rows, n_head, n_split;
    int ragged;                    // nonzero: the partials follow a length-proportional plan
                                   //   (each row's slots from the row table)
};

hipError_t launch_attention(const AttnArgs &a, int kv_kind, int shape, hipStream_t stream);
hipError_t launch_merge_proj(const MergeProjArgs &a, int kind, hipStream_t stream);
hipError_t launch_proj(const ProjArgs &p, int kind, bool a_f32, bool c_f32, hipStream_t stream);
hipError_t launch_merge(int n_rows, int n_head, int n_split, const float *ws, float *out,
                        const float *sinks, const Ragged &ragged, hipStream_t stream);
hipError_t launch_mha(const MhaArgs &a, int kv_kind, hipStream_t stream);
hipError_t launch_compact(const uint16_t *mask, int64_t mask_row_stride, int n_rows, int64_t n_kv,
                          int32_t *idx, int64_t idx_row_stride, int32_t *count,
                          hipStream_t stream);
// Multi-workgroup compaction (rows of up to kCompactChunkedMax cells, 16-byte aligned):
// compact_chunks(n_kv) int32 chunk counts per row of workspace; 0 = not available.
constexpr int64_t kCompactChunkedMax = (int64_t)1 << 22;
int64_t compact_chunks(int64_t n_kv);
hipError_t launch_compact_chunked(const uint16_t *mask, int64_t mask_row_stride, int n_rows, int64_t n_kv,
                                  int32_t *idx, int64_t idx_row_stride, int32_t *count, int32_t *ws,
                                  hipStream_t stream);

// Heads per workgroup of each shape.
inline int shape_heads(int shape) {
    switch (shape) {
        case SHAPE_P64: return 64;
        case SHAPE_P128: return 128;
    }
    return 16 << shape;
}

}  // namespace mlafa
