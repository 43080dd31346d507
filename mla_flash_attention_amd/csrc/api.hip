// api.hip -- the extern "C" boundary of libmlafa: argument validation (before any HIP
// call), split planning, workspace layout and launches.  See include/mla_fa.h for the
// contract of every entry point.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/mla_fa.h"
#include "mla_fa_internal.h"

using namespace mlafa;

namespace {

constexpr int kMinTilesPerSplit = 1;   // short caches: one tile per split is fastest (latency-bound)
constexpr int kMaxDevices = 64;

// Compute units of the current device.  The plans give each CU one workgroup (the
// attention kernels' LDS use allows no more), so a partitioned GPU, with fewer CUs per
// device, gets plans of its own size.  256, the MI355X's count, when HIP cannot say (no
// device), so that the host-only sizing calls still answer; a failed query's error is
// cleared so that no later launch check reports it.  Cached per device.
constexpr int kDefaultCUs = 256;
int device_cus() {
    static std::atomic<int> cache[kMaxDevices];          // 0 = not asked yet
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return kDefaultCUs;
    }
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) {
            (void)hipGetLastError();
            n = kDefaultCUs;
        }
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Failure injection for tests of the launch-error path.  With MLA_FA_FAIL_LAUNCH=<k> in
// the environment, an entry point launches nothing: it walks its launch sequence and
// reports its k-th launch (1-based) as failed, so every MLA_FA_ERR_HIP return can be
// reached without a GPU.  Read once per call; thread-local, so concurrent calls on other
// threads keep their own count.
thread_local int t_launch_no = 0, t_fail_at = 0;
void begin_call() {
    t_launch_no = 0;
    const char *e = std::getenv("MLA_FA_FAIL_LAUNCH");
    t_fail_at = e && *e ? std::atoi(e) : 0;
}
// Whether the next launch is to be skipped; *failed says whether it reports failure.
bool launch_skipped(bool *failed) {
    ++t_launch_no;
    *failed = t_launch_no == t_fail_at;
    return t_fail_at > 0;
}
// hipSuccess / a launch error for a launch the test hook skipped.
hipError_t skipped_status(bool failed) { return failed ? hipErrorLaunchFailure : hipSuccess; }

int kv_kind_of(int kv_type) {
    return kv_type == MLA_FA_BF16 ? KV_BF16 : kv_type == MLA_FA_F16 ? KV_F16 : KV_Q8;
}

int check_types(int q_type, int kv_type) {
    if (q_type != MLA_FA_F16 && q_type != MLA_FA_BF16) return MLA_FA_ERR_INVALID;
    if (kv_type != MLA_FA_F16 && kv_type != MLA_FA_BF16 && kv_type != MLA_FA_Q8_0)
        return MLA_FA_ERR_INVALID;
    if (kv_type == MLA_FA_Q8_0) return MLA_FA_OK;
    if (kv_type != q_type) return MLA_FA_ERR_UNSUPPORTED;
    return MLA_FA_OK;
}

int check_heads(int n_head) {
    if (n_head < 1) return MLA_FA_ERR_INVALID;
    if (n_head % 16 != 0 || n_head > 128) return MLA_FA_ERR_UNSUPPORTED;
    return MLA_FA_OK;
}

int row_bytes(int kv_type) { return kv_type == MLA_FA_Q8_0 ? kQ8RowBytes : kRowBytes16; }

// Environment override of the automatic split count (tuning only; results change by
// float reassociation alone).
int env_splits() {
    const char *e = std::getenv("MLA_FA_NSPLIT");
    if (!e || !*e) return 0;
    int v = std::atoi(e);
    return v >= 1 && v <= kMaxSplits ? v : 0;
}

// Workgroup shape: heads per workgroup.  Split calls over 16-bit caches use 64-head
// workgroups whose two key halves merge in LDS (half the partial bytes of 128-head
// workgroups); unsplit calls use 128-head workgroups so each tile is read once per query
// row.  Q8_0 caches use 128-head workgroups while that takes at most 64 splits: each
// dequantised tile then serves every head (measured on the 4 x 128-head x 65536-cell
// Q8_0 decode: kernel 116 -> 97 us with twice the splits); past that (one or two rows,
// as in sparse decoding) twice the partials cost more than the dequantisation saves
// (the 131,072-cell sparse Q8_0 step: 40 -> 52 us).  The pair-kernel shapes (p64, p128: half the LDS reads per
// MFMA, two exchanges per stage) are selected only through the tuning override; measured
// on gfx950 they do not beat these.
constexpr int kQ8WideMaxSplits = 64;

int pick_shape(int n_head, int n_split, int kv_type) {
    if (const char *e = std::getenv("MLA_FA_SHAPE")) {       // tuning only
        const bool q8 = kv_type == MLA_FA_Q8_0;
        if (!std::strcmp(e, "16")) return SHAPE_H16;
        if (!std::strcmp(e, "32")) return SHAPE_H32;
        if (!std::strcmp(e, "64")) return SHAPE_H64;
        if (!std::strcmp(e, "128")) return SHAPE_H128;
        if (!std::strcmp(e, "p64") && !q8) return SHAPE_P64;
        if (!std::strcmp(e, "p128") && !q8) return SHAPE_P128;
    }
    if (n_head <= 16) return SHAPE_H16;
    if (n_head <= 32) return SHAPE_H32;
    if (n_head <= 64) return SHAPE_H64;
    if (n_split <= 1) return SHAPE_H128;
    return kv_type == MLA_FA_Q8_0 && n_split <= kQ8WideMaxSplits ? SHAPE_H128 : SHAPE_H64;
}

int auto_splits(int64_t n_rows, int n_head, int64_t n_kv, int kv_type) {
    const int env = env_splits();
    if (env) return env;
    const int cus = device_cus();
    const int hu = shape_heads(pick_shape(n_head, 1, kv_type));
    if (n_rows * ((n_head + hu - 1) / hu) >= cus) return 1;
    // splits that fill the chip with the split shape: the wide Q8_0 shape when that plan
    // stays within its split limit, else the 16-bit one
    int hs = shape_heads(pick_shape(n_head, 2, kv_type));
    int64_t s = (cus + n_rows * ((n_head + hs - 1) / hs) - 1) / (n_rows * ((n_head + hs - 1) / hs));
    // (the wide shape also needs the rounded-up plan to stay near one workgroup per CU)
    if (shape_heads(pick_shape(n_head, (int)(s < kMaxSplits ? s : kMaxSplits), kv_type)) != hs ||
        n_rows * s * ((n_head + hs - 1) / hs) > cus + cus / 4) {
        hs = shape_heads(pick_shape(n_head, kMaxSplits, kv_type));
        const int64_t hg = (n_head + hs - 1) / hs;
        s = (cus + n_rows * hg - 1) / (n_rows * hg);
    }
    const int64_t max_by_len = (n_kv + kTileKeys * kMinTilesPerSplit - 1) / (kTileKeys * kMinTilesPerSplit);
    if (s > max_by_len) s = max_by_len;
    if (s < 1) s = 1;
    if (s > kMaxSplits) s = kMaxSplits;
    return (int)s;
}

struct Plan {
    int n_split;
    int shape;
    int head_groups;
    int grid_x;
    int64_t split_chunk;
};

Plan make_plan(int64_t n_rows, int n_head, int64_t n_kv, int kv_type, int n_split) {
    Plan p;
    p.n_split = n_split > 0 ? n_split : auto_splits(n_rows, n_head, n_kv, kv_type);
    p.shape = pick_shape(n_head, p.n_split, kv_type);
    const int hpw = shape_heads(p.shape);
    p.head_groups = (n_head + hpw - 1) / hpw;
    p.grid_x = p.head_groups > 1 ? 8 * p.head_groups * ((p.n_split + 7) / 8) : p.n_split;
    int64_t chunk = (n_kv + p.n_split - 1) / p.n_split;
    p.split_chunk = (chunk + kTileKeys - 1) / kTileKeys * kTileKeys;
    return p;
}

struct Common {
    const void *q;
    int q_type;
    const void *kv;
    int kv_type;
    int64_t kv_row_stride, kv_seq_stride;
    int n_seq, n_tok, n_head;
    int64_t n_kv;
    int causal;
    const uint16_t *mask;
    int64_t mask_seq_stride, mask_tok_stride;
    const int32_t *kv_idx, *kv_idx_count;
    int64_t idx_seq_stride;
    int64_t idx_tok_stride = 0;
    float scale;
    float *out;
    int n_split;
    void *ws;
    size_t ws_bytes;
    const int32_t *kv_len = nullptr;
    const float *alibi = nullptr;
    const float *sinks = nullptr;
    float softcap = 0.f;
    bool ragged_ok = false;        // the call runs its own merge (which reads the plan's row
                                   //   table): rows may share slots by length
};

int validate(const Common &c) {
    if (!c.q || !c.kv || !c.out) return MLA_FA_ERR_INVALID;
    int st = check_types(c.q_type, c.kv_type);
    if (st) return st;
    st = check_heads(c.n_head);
    if (st) return st;
    if (c.n_seq < 1 || c.n_tok < 1 || c.n_kv < 1 || c.n_kv > 0x7FFFFFFFLL) return MLA_FA_ERR_INVALID;
    if ((int64_t)c.n_seq * c.n_tok * c.n_head > 0x7FFFFFFFLL) return MLA_FA_ERR_INVALID;   // merge grid
    if (!std::isfinite(c.scale)) return MLA_FA_ERR_INVALID;
    if (c.n_split < 0 || c.n_split > kMaxSplits) return MLA_FA_ERR_INVALID;
    if (!aligned(c.q, 16) || !aligned(c.out, 16)) return MLA_FA_ERR_INVALID;
    const size_t kva = c.kv_type == MLA_FA_Q8_0 ? 4 : 16;
    if (!aligned(c.kv, kva) || c.kv_row_stride < row_bytes(c.kv_type) || c.kv_row_stride % kva ||
        c.kv_seq_stride < 0 || c.kv_seq_stride % kva)
        return MLA_FA_ERR_INVALID;
    // Q8_0 tiles address their rows with 32-bit offsets from the tile's first row
    if (c.kv_type == MLA_FA_Q8_0 && c.kv_row_stride > (int64_t)1 << 26) return MLA_FA_ERR_INVALID;
    if (c.causal && !c.kv_len && c.n_tok > c.n_kv) return MLA_FA_ERR_INVALID;
    if (c.mask) {
        if (!aligned(c.mask, 2) || c.mask_seq_stride < 0 || c.mask_tok_stride < 0)
            return MLA_FA_ERR_INVALID;
        if (c.n_seq > 1 && c.mask_seq_stride < c.n_kv) return MLA_FA_ERR_INVALID;
        if (c.n_tok > 1 && c.mask_tok_stride < c.n_kv) return MLA_FA_ERR_INVALID;
    }
    if (!(c.softcap >= 0.f) || !std::isfinite(c.softcap)) return MLA_FA_ERR_INVALID;
    if (!aligned(c.kv_len, 4) || !aligned(c.alibi, 4) || !aligned(c.sinks, 4)) return MLA_FA_ERR_INVALID;
    if ((c.kv_idx == nullptr) != (c.kv_idx_count == nullptr)) return MLA_FA_ERR_INVALID;
    if (c.kv_idx) {
        // an index list says which cells its row sees: no causal edge or valid lengths on top
        if (c.causal || c.kv_len) return MLA_FA_ERR_INVALID;
        if (!aligned(c.kv_idx, 4) || !aligned(c.kv_idx_count, 4)) return MLA_FA_ERR_INVALID;
        if (c.idx_seq_stride < 0 || c.idx_tok_stride < 0) return MLA_FA_ERR_INVALID;
        if ((c.n_seq > 1 && c.idx_seq_stride < c.n_kv) || (c.n_tok > 1 && c.idx_tok_stride < c.n_kv))
            return MLA_FA_ERR_INVALID;
    }
    return MLA_FA_OK;
}

// Rows whose lengths only the device holds (valid lengths or index-list counts) get a
// length-proportional plan when the call splits and runs its own merge: the kernel shares
// the call's rows * n_split partial slots out by length, at most one piece per workgroup
// slot of the chip (CUs / head groups pieces, at least one per row).  With every row cut
// into n_split pieces instead, the longest row's pieces set the call's time.
Ragged ragged_for(const Common &c, const Plan &p) {
    Ragged g;
    std::memset(&g, 0, sizeof(g));
    const int64_t rows = (int64_t)c.n_seq * c.n_tok;
    if (!c.ragged_ok || p.n_split <= 1 || rows > kRaggedRows || (!c.kv_len && !c.kv_idx)) return g;
    const int64_t slots = rows * p.n_split;
    const int64_t chip = std::max<int64_t>(rows, device_cus() / p.head_groups);
    g.budget = (int)std::min(slots, chip);
    g.kv_len = c.kv_idx ? nullptr : c.kv_len;
    g.count = c.kv_idx ? c.kv_idx_count : nullptr;
    g.n_kv = c.n_kv;
    g.n_tok = c.n_tok;
    g.causal = c.causal ? 1 : 0;
    g.rows = (int)rows;
    return g;
}

int run_partials(const Common &c, const Plan &p, hipStream_t stream) {
    const int64_t n_rows = (int64_t)c.n_seq * c.n_tok;
    if (p.n_split > 1) {
        const size_t need = partial_bytes(n_rows, c.n_head, p.n_split);
        if (!c.ws || c.ws_bytes < need || !aligned(c.ws, 16)) return MLA_FA_ERR_WORKSPACE;
    }
    if (n_rows > 0x7FFFFFFFLL || p.grid_x > 0x7FFFFFFF) return MLA_FA_ERR_INVALID;
    AttnArgs a;
    std::memset(&a, 0, sizeof(a));
    a.q = static_cast<const uint16_t *>(c.q);
    a.kv = static_cast<const uint8_t *>(c.kv);
    a.kv_row_stride = c.kv_row_stride;
    a.kv_seq_stride = c.kv_seq_stride;
    a.mask = c.mask;
    a.mask_seq_stride = c.mask_seq_stride;
    a.mask_tok_stride = c.mask_tok_stride;
    a.kv_idx = c.kv_idx;
    a.kv_idx_count = c.kv_idx_count;
    a.idx_seq_stride = c.idx_seq_stride;
    a.idx_tok_stride = c.idx_tok_stride;
    a.out = c.out;
    a.ws = static_cast<float *>(c.ws);
    a.n_kv = c.n_kv;
    a.split_chunk = p.split_chunk;
    a.n_seq = c.n_seq;
    a.n_tok = c.n_tok;
    a.n_head = c.n_head;
    a.causal = c.causal ? 1 : 0;
    a.n_split = p.n_split;
    a.head_groups = p.head_groups;
    a.grid_x = p.grid_x;
    a.q_bf16 = c.q_type == MLA_FA_BF16;
    a.scale_log2 = c.scale * 1.4426950408889634f;
    a.kv_len = c.kv_len;
    a.alibi = c.alibi;
    a.sinks = c.sinks;
    a.cap_in = c.softcap > 0.f ? c.scale / c.softcap : 0.f;
    a.cap_out = c.softcap * 1.4426950408889634f;
    a.ragged = ragged_for(c, p);
    if (a.ragged.budget)   // one launch, one workgroup per (piece, head group)
        a.grid_x = p.head_groups > 1 ? 8 * p.head_groups * ((a.ragged.budget + 7) / 8) : a.ragged.budget;
    if (std::getenv("MLA_FA_LOG"))
        fprintf(stderr,
                "mla_fa: rows=%lld heads=%d n_kv=%lld split=%d chunk=%lld shape=%d hg=%d grid=%dx%lld pieces=%d\n",
                (long long)n_rows, c.n_head, (long long)c.n_kv, p.n_split, (long long)p.split_chunk,
                p.shape, p.head_groups, a.grid_x, a.ragged.budget ? 1LL : (long long)n_rows, a.ragged.budget);
    bool fail;
    hipError_t e = launch_skipped(&fail) ? skipped_status(fail) : launch_attention(a, kv_kind_of(c.kv_type), p.shape, stream);
    return e == hipSuccess ? MLA_FA_OK : MLA_FA_ERR_HIP;
}

int run_merge(int64_t n_rows, int n_head, int n_split, float *out, const void *ws, size_t ws_bytes,
              hipStream_t stream, const float *sinks = nullptr, const Ragged *ragged = nullptr) {
    if (n_split <= 1) return MLA_FA_OK;
    if (n_rows * n_head > 0x7FFFFFFFLL) return MLA_FA_ERR_INVALID;   // one merge workgroup per (row, head)
    const size_t need = partial_bytes(n_rows, n_head, n_split);
    if (!ws || ws_bytes < need || !aligned(ws, 16)) return MLA_FA_ERR_WORKSPACE;
    bool fail;
    hipError_t e = launch_skipped(&fail) ? skipped_status(fail)
                                         : launch_merge((int)n_rows, n_head, n_split, static_cast<const float *>(ws),
                                                        out, sinks, ragged ? *ragged : Ragged{}, stream);
    return e == hipSuccess ? MLA_FA_OK : MLA_FA_ERR_HIP;
}

Common decode_common(const void *q, int q_type, const void *kv, int kv_type, int64_t kv_row_stride,
                     int64_t kv_seq_stride, int n_seq, int n_head, int64_t n_kv,
                     const uint16_t *mask, int64_t mask_seq_stride, const int32_t *kv_idx,
                     const int32_t *kv_idx_count, int64_t idx_seq_stride, float scale, float *out,
                     int n_split, void *ws, size_t ws_bytes) {
    Common c;
    c.q = q; c.q_type = q_type; c.kv = kv; c.kv_type = kv_type;
    c.kv_row_stride = kv_row_stride; c.kv_seq_stride = kv_seq_stride;
    c.n_seq = n_seq; c.n_tok = 1; c.n_head = n_head; c.n_kv = n_kv; c.causal = 0;
    c.mask = mask; c.mask_seq_stride = mask_seq_stride; c.mask_tok_stride = 0;
    c.kv_idx = kv_idx; c.kv_idx_count = kv_idx_count; c.idx_seq_stride = idx_seq_stride;
    c.scale = scale; c.out = out; c.n_split = n_split; c.ws = ws; c.ws_bytes = ws_bytes;
    return c;
}

hipError_t run_proj(const ProjArgs &pa, int kind, bool a_f32, bool c_f32, hipStream_t s) {
    bool fail;
    return launch_skipped(&fail) ? skipped_status(fail) : launch_proj(pa, kind, a_f32, c_f32, s);
}

// Workspace of mla_fa_absorbed: the 576-wide queries (16-bit), the latent outputs (fp32)
// and the split partials, each section 256-byte aligned.
struct AbsorbedLayout {
    size_t q_off, o_off, part_off, total;
};
AbsorbedLayout absorbed_layout(int64_t n_rows, int n_head, int n_split) {
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    AbsorbedLayout l;
    l.q_off = 0;
    l.o_off = up((size_t)n_rows * n_head * kDK * 2);
    l.part_off = l.o_off + up((size_t)n_rows * n_head * kDV * sizeof(float));
    l.total = l.part_off + (n_split > 1 ? partial_bytes(n_rows, n_head, n_split) : 0);
    return l;
}

// Scratch of mla_fa_decode_noalloc: the split partials of callers that cannot allocate.
// Each GPU the library runs on holds its own copy for the life of the process.  Host code
// never uses the array's name as an address: the device address comes from
// hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kScratchBytes = MLA_FA_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// The current device's scratch address (nullptr on a HIP error).
void *device_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

const char *mla_fa_strerror(int status) {
    switch (status) {
        case MLA_FA_OK: return "ok";
        case MLA_FA_ERR_INVALID: return "invalid argument (null pointer, size, stride or alignment)";
        case MLA_FA_ERR_UNSUPPORTED: return "unsupported type pair or head count";
        case MLA_FA_ERR_WORKSPACE: return "workspace missing or too small";
        case MLA_FA_ERR_HIP: return "HIP launch failed";
    }
    return "unknown status";
}

int mla_fa_version(void) { return 20100; }

int mla_fa_auto_splits(int n_rows, int n_head, int64_t n_kv, int kv_type) {
    if (n_rows < 1 || n_kv < 1 || check_heads(n_head)) return 1;
    return auto_splits(n_rows, n_head, n_kv, kv_type);
}

size_t mla_fa_workspace_size(int n_rows, int n_head, int64_t n_kv, int kv_type, int n_split) {
    if (n_rows < 1 || n_kv < 1 || check_heads(n_head) || n_split < 0 || n_split > kMaxSplits) return 0;
    Plan p = make_plan(n_rows, n_head, n_kv, kv_type, n_split);
    return p.n_split > 1 ? partial_bytes(n_rows, n_head, p.n_split) : 0;
}

int mla_fa_decode_partials(const void *q, int q_type, const void *kv, int kv_type,
                           int64_t kv_row_stride, int64_t kv_seq_stride, int n_seq, int n_head,
                           int64_t n_kv, const uint16_t *mask, int64_t mask_seq_stride,
                           const int32_t *kv_idx, const int32_t *kv_idx_count,
                           int64_t idx_seq_stride, float scale, float *out, int n_split,
                           void *workspace, size_t workspace_bytes, void *stream) {
    begin_call();
    Common c = decode_common(q, q_type, kv, kv_type, kv_row_stride, kv_seq_stride, n_seq, n_head, n_kv,
                             mask, mask_seq_stride, kv_idx, kv_idx_count, idx_seq_stride, scale, out,
                             n_split, workspace, workspace_bytes);
    int st = validate(c);
    if (st) return st;
    Plan p = make_plan(n_seq, n_head, n_kv, kv_type, n_split);
    return run_partials(c, p, static_cast<hipStream_t>(stream));
}

int mla_fa_merge_partials(int n_rows, int n_head, int n_split, float *out, const void *workspace,
                          size_t workspace_bytes, void *stream) {
    begin_call();
    if (!out || n_rows < 1 || n_split < 1 || n_split > kMaxSplits || !aligned(out, 16))
        return MLA_FA_ERR_INVALID;
    int st = check_heads(n_head);
    if (st) return st;
    return run_merge(n_rows, n_head, n_split, out, workspace, workspace_bytes,
                     static_cast<hipStream_t>(stream));
}

int mla_fa_decode(const void *q, int q_type, const void *kv, int kv_type, int64_t kv_row_stride,
                  int64_t kv_seq_stride, int n_seq, int n_head, int64_t n_kv,
                  const uint16_t *mask, int64_t mask_seq_stride, const int32_t *kv_idx,
                  const int32_t *kv_idx_count, int64_t idx_seq_stride, float scale, float *out,
                  int n_split, void *workspace, size_t workspace_bytes, void *stream) {
    begin_call();
    Common c = decode_common(q, q_type, kv, kv_type, kv_row_stride, kv_seq_stride, n_seq, n_head, n_kv,
                             mask, mask_seq_stride, kv_idx, kv_idx_count, idx_seq_stride, scale, out,
                             n_split, workspace, workspace_bytes);
    c.ragged_ok = n_seq > 1;       // index lists of several sequences: share slots by count
    int st = validate(c);
    if (st) return st;
    Plan p = make_plan(n_seq, n_head, n_kv, kv_type, n_split);
    if (p.n_split > 1 && (!workspace || workspace_bytes < partial_bytes(n_seq, n_head, p.n_split)))
        return MLA_FA_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    st = run_partials(c, p, s);
    if (st) return st;
    const Ragged rg = ragged_for(c, p);
    return run_merge(n_seq, n_head, p.n_split, out, workspace, workspace_bytes, s, nullptr, &rg);
}

int mla_fa_decode_noalloc(const void *q, int q_type, const void *kv, int kv_type, int64_t kv_row_stride,
                          int64_t kv_seq_stride, int n_seq, int n_head, int64_t n_kv, const uint16_t *mask,
                          int64_t mask_seq_stride, const int32_t *kv_idx, const int32_t *kv_idx_count,
                          int64_t idx_seq_stride, float scale, float *out, int n_split, void *stream) {
    begin_call();
    Common c = decode_common(q, q_type, kv, kv_type, kv_row_stride, kv_seq_stride, n_seq, n_head, n_kv,
                             mask, mask_seq_stride, kv_idx, kv_idx_count, idx_seq_stride, scale, out,
                             n_split, nullptr, 0);
    c.ragged_ok = n_seq > 1;       // as mla_fa_decode
    int st = validate(c);
    if (st) return st;
    Plan p = make_plan(n_seq, n_head, n_kv, kv_type, n_split);
    const size_t need = p.n_split > 1 ? partial_bytes(n_seq, n_head, p.n_split) : 0;
    if (need > kScratchBytes) return MLA_FA_ERR_WORKSPACE;      // past the scratch's fixed size
    if (need) {
        c.ws = device_scratch();
        if (!c.ws) return MLA_FA_ERR_HIP;
        c.ws_bytes = kScratchBytes;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    st = run_partials(c, p, s);
    if (st) return st;
    const Ragged rg = ragged_for(c, p);
    return run_merge(n_seq, n_head, p.n_split, out, c.ws, c.ws_bytes, s, nullptr, &rg);
}

int mla_fa_prefill(const void *q, int q_type, const void *kv, int kv_type, int64_t kv_row_stride,
                   int n_tok, int n_head, int64_t n_kv, int causal, const uint16_t *mask,
                   int64_t mask_row_stride, float scale, float *out, int n_split,
                   void *workspace, size_t workspace_bytes, void *stream) {
    begin_call();
    Common c;
    c.q = q; c.q_type = q_type; c.kv = kv; c.kv_type = kv_type;
    c.kv_row_stride = kv_row_stride; c.kv_seq_stride = 0;
    c.n_seq = 1; c.n_tok = n_tok; c.n_head = n_head; c.n_kv = n_kv; c.causal = causal;
    c.mask = mask; c.mask_seq_stride = 0; c.mask_tok_stride = mask_row_stride;
    c.kv_idx = nullptr; c.kv_idx_count = nullptr; c.idx_seq_stride = 0;
    c.scale = scale; c.out = out; c.n_split = n_split; c.ws = workspace; c.ws_bytes = workspace_bytes;
    int st = validate(c);
    if (st) return st;
    Plan p = make_plan(n_tok, n_head, n_kv, kv_type, n_split);
    if (p.n_split > 1 && (!workspace || workspace_bytes < partial_bytes(n_tok, n_head, p.n_split)))
        return MLA_FA_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    st = run_partials(c, p, s);
    if (st) return st;
    return run_merge(n_tok, n_head, p.n_split, out, workspace, workspace_bytes, s);
}

int mla_fa_attend(const void *q, int q_type, const void *kv, int kv_type, int64_t kv_row_stride,
                  int64_t kv_seq_stride, int n_seq, int n_tok, int n_head, int64_t n_kv,
                  const int32_t *kv_len, int causal, const uint16_t *mask, int64_t mask_seq_stride,
                  int64_t mask_tok_stride, const int32_t *kv_idx, const int32_t *kv_idx_count,
                  int64_t idx_seq_stride, int64_t idx_tok_stride, const float *alibi_slopes,
                  const float *sinks, float softcap, float scale, float *out, int n_split, void *workspace,
                  size_t workspace_bytes, void *stream) {
    begin_call();
    Common c;
    c.q = q; c.q_type = q_type; c.kv = kv; c.kv_type = kv_type;
    c.kv_row_stride = kv_row_stride; c.kv_seq_stride = kv_seq_stride;
    c.n_seq = n_seq; c.n_tok = n_tok; c.n_head = n_head; c.n_kv = n_kv; c.causal = causal;
    c.mask = mask; c.mask_seq_stride = mask_seq_stride; c.mask_tok_stride = mask_tok_stride;
    c.kv_idx = kv_idx; c.kv_idx_count = kv_idx_count; c.idx_seq_stride = idx_seq_stride;
    c.idx_tok_stride = idx_tok_stride;
    c.scale = scale; c.out = out; c.n_split = n_split; c.ws = workspace; c.ws_bytes = workspace_bytes;
    c.kv_len = kv_len; c.alibi = alibi_slopes; c.sinks = sinks; c.softcap = softcap;
    c.ragged_ok = true;
    int st = validate(c);
    if (st) return st;
    const int64_t n_rows = (int64_t)n_seq * n_tok;
    Plan p = make_plan(n_rows, n_head, n_kv, kv_type, n_split);
    if (p.n_split > 1 && (!workspace || workspace_bytes < partial_bytes(n_rows, n_head, p.n_split)))
        return MLA_FA_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    st = run_partials(c, p, s);
    if (st) return st;
    const Ragged rg = ragged_for(c, p);
    return run_merge(n_rows, n_head, p.n_split, out, workspace, workspace_bytes, s, sinks, &rg);
}

int mla_fa_prefill_mha(const void *q, int q_type, const void *k, const void *v, int kv_type,
                       int64_t k_row_stride, int64_t v_row_stride, int n_tok, int n_head, int64_t n_kv,
                       int causal, const uint16_t *mask, int64_t mask_row_stride, float scale,
                       float *out, void *stream) {
    begin_call();
    if (!q || !k || !v || !out) return MLA_FA_ERR_INVALID;
    if (q_type != MLA_FA_F16 && q_type != MLA_FA_BF16) return MLA_FA_ERR_INVALID;
    if (kv_type != MLA_FA_F16 && kv_type != MLA_FA_BF16 && kv_type != MLA_FA_Q8_0) return MLA_FA_ERR_INVALID;
    if (kv_type != q_type) return MLA_FA_ERR_UNSUPPORTED;
    if (n_tok < 1 || n_head < 1 || n_head > 65535 || n_kv < 1 || n_kv > 0x7FFFFFFFLL) return MLA_FA_ERR_INVALID;
    if (causal && n_tok > n_kv) return MLA_FA_ERR_INVALID;
    if ((int64_t)((n_tok + 255) / 256) * n_head > 0x7FFFFFFFLL) return MLA_FA_ERR_INVALID;   // grid size
    if (!std::isfinite(scale)) return MLA_FA_ERR_INVALID;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return MLA_FA_ERR_INVALID;
    if (k_row_stride < (int64_t)n_head * 384 || k_row_stride % 16 || v_row_stride < (int64_t)n_head * 256 ||
        v_row_stride % 16)
        return MLA_FA_ERR_INVALID;
    if (mask) {
        if (!aligned(mask, 16) || mask_row_stride < 0 || mask_row_stride % 8) return MLA_FA_ERR_INVALID;
        if (n_tok > 1 && mask_row_stride < n_kv) return MLA_FA_ERR_INVALID;
    }
    MhaArgs a;
    std::memset(&a, 0, sizeof(a));
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint8_t *>(k);
    a.v = static_cast<const uint8_t *>(v);
    a.k_row_stride = k_row_stride;
    a.v_row_stride = v_row_stride;
    a.mask = mask;
    a.mask_row_stride = mask_row_stride;
    a.out = out;
    a.n_kv = n_kv;
    a.n_tok = n_tok;
    a.n_head = n_head;
    a.causal = causal ? 1 : 0;
    a.scale_log2 = scale * 1.4426950408889634f;
    bool fail;
    hipError_t e = launch_skipped(&fail) ? skipped_status(fail)
                                         : launch_mha(a, kv_kind_of(kv_type), static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MLA_FA_OK : MLA_FA_ERR_HIP;
}

size_t mla_fa_absorbed_workspace_size(int n_rows, int n_head, int64_t n_kv, int kv_type, int n_split) {
    if (n_rows < 1 || n_kv < 1 || check_heads(n_head) || n_split < 0 || n_split > kMaxSplits) return 0;
    Plan p = make_plan(n_rows, n_head, n_kv, kv_type, n_split);
    return absorbed_layout(n_rows, n_head, p.n_split).total;
}

int mla_fa_absorbed(const void *q_nope, const void *q_pe, int q_type, const void *w_uk, const void *w_uv,
                    const void *kv, int kv_type, int64_t kv_row_stride, int64_t kv_seq_stride, int n_seq,
                    int n_tok, int n_head, int64_t n_kv, const int32_t *kv_len, int causal, const uint16_t *mask,
                    int64_t mask_seq_stride, int64_t mask_tok_stride, float scale, float *out, int n_split,
                    void *workspace, size_t workspace_bytes, void *stream) {
    begin_call();
    if (!q_nope || !q_pe || !w_uk || !w_uv || !out) return MLA_FA_ERR_INVALID;
    if (!aligned(q_nope, 16) || !aligned(q_pe, 16) || !aligned(w_uk, 16) || !aligned(w_uv, 16) ||
        !aligned(out, 16) || !aligned(workspace, 256))
        return MLA_FA_ERR_INVALID;
    if (n_seq < 1 || n_tok < 1 || (int64_t)n_seq * n_tok > 0x7FFFFFFFLL) return MLA_FA_ERR_INVALID;
    const int64_t n_rows = (int64_t)n_seq * n_tok;
    int st = check_heads(n_head);
    if (st) return st;
    if (n_split < 0 || n_split > kMaxSplits || n_kv < 1) return MLA_FA_ERR_INVALID;
    const Plan p = make_plan(n_rows, n_head, n_kv, kv_type, n_split);
    const AbsorbedLayout lay = absorbed_layout(n_rows, n_head, p.n_split);
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    // the attention part, on the queries the first projection writes into the workspace
    Common c;
    c.q = ws ? ws + lay.q_off : nullptr; c.q_type = q_type; c.kv = kv; c.kv_type = kv_type;
    c.kv_row_stride = kv_row_stride; c.kv_seq_stride = kv_seq_stride;
    c.n_seq = n_seq; c.n_tok = n_tok; c.n_head = n_head; c.n_kv = n_kv; c.causal = causal;
    c.mask = mask; c.mask_seq_stride = mask_seq_stride; c.mask_tok_stride = mask_tok_stride;
    c.kv_idx = nullptr; c.kv_idx_count = nullptr; c.idx_seq_stride = 0;
    c.scale = scale; c.out = ws ? reinterpret_cast<float *>(ws + lay.o_off) : nullptr; c.n_split = p.n_split;
    c.ws = ws ? ws + lay.part_off : nullptr; c.ws_bytes = lay.total - lay.part_off;
    c.kv_len = kv_len;
    c.ragged_ok = true;            // merge_proj_kernel follows a length-proportional plan
    if (!workspace || workspace_bytes < lay.total) {
        // report argument errors first: validate with stand-in buffers
        Common v = c;
        v.q = q_nope; v.out = out;
        st = validate(v);
        return st ? st : MLA_FA_ERR_WORKSPACE;
    }
    st = validate(c);
    if (st) return st;
    const int kind = q_type == MLA_FA_BF16 ? KV_BF16 : KV_F16;
    hipStream_t s = static_cast<hipStream_t>(stream);
    ProjArgs qa;
    qa.a = q_nope; qa.a_rs = (int64_t)n_head * 128; qa.a_hs = 128;
    qa.w = static_cast<const uint16_t *>(w_uk);
    qa.c = ws + lay.q_off; qa.c_rs = (int64_t)n_head * kDK; qa.c_hs = kDK;
    qa.extra = static_cast<const uint16_t *>(q_pe); qa.extra_rs = (int64_t)n_head * 64; qa.extra_hs = 64;
    qa.M = (int)n_rows; qa.N = kDV; qa.K = 128; qa.H = n_head;
    if (run_proj(qa, kind, false, false, s) != hipSuccess) return MLA_FA_ERR_HIP;
    st = run_partials(c, p, s);
    if (st) return st;
    if (p.n_split > 1) {
        // split plan: the merge and the output projection are one launch
        MergeProjArgs ma;
        ma.ws = static_cast<const float *>(c.ws);
        ma.w = static_cast<const uint16_t *>(w_uv);
        ma.out = out; ma.out_rs = (int64_t)n_head * 128;
        ma.n_rows = (int)n_rows; ma.n_head = n_head; ma.n_split = p.n_split;
        ma.ragged = ragged_for(c, p).budget > 0;
        bool fail;
        const hipError_t e = launch_skipped(&fail) ? skipped_status(fail) : launch_merge_proj(ma, kind, s);
        return e == hipSuccess ? MLA_FA_OK : MLA_FA_ERR_HIP;
    }
    ProjArgs oa;
    oa.a = c.out; oa.a_rs = (int64_t)n_head * kDV; oa.a_hs = kDV;
    oa.w = static_cast<const uint16_t *>(w_uv);
    oa.c = out; oa.c_rs = (int64_t)n_head * 128; oa.c_hs = 128;
    oa.extra = nullptr; oa.extra_rs = 0; oa.extra_hs = 0;
    oa.M = (int)n_rows; oa.N = 128; oa.K = kDV; oa.H = n_head;
    return run_proj(oa, kind, true, true, s) == hipSuccess ? MLA_FA_OK : MLA_FA_ERR_HIP;
}

int fa_mask_compact(const uint16_t *mask, int64_t mask_row_stride, int n_rows, int64_t n_kv,
                    int32_t *idx, int64_t idx_row_stride, int32_t *count, void *stream) {
    begin_call();
    if (!mask || !idx || !count || n_rows < 1 || n_kv < 1 || n_kv > 0x7FFFFFFFLL)
        return MLA_FA_ERR_INVALID;
    if (!aligned(mask, 2) || !aligned(idx, 4) || !aligned(count, 4)) return MLA_FA_ERR_INVALID;
    if (idx_row_stride < n_kv || (n_rows > 1 && mask_row_stride < n_kv) || mask_row_stride < 0)
        return MLA_FA_ERR_INVALID;
    bool fail;
    hipError_t e = launch_skipped(&fail) ? skipped_status(fail)
                                         : launch_compact(mask, mask_row_stride, n_rows, n_kv, idx, idx_row_stride,
                                                          count, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MLA_FA_OK : MLA_FA_ERR_HIP;
}

size_t fa_mask_compact_workspace_size(int n_rows, int64_t n_kv) {
    if (n_rows < 1 || n_rows > kMaxGridY || n_kv < 1 || n_kv > 0x7FFFFFFFLL) return 0;
    return (size_t)n_rows * (size_t)compact_chunks(n_kv) * sizeof(int32_t);
}

int fa_mask_compact_ws(const uint16_t *mask, int64_t mask_row_stride, int n_rows, int64_t n_kv,
                       int32_t *idx, int64_t idx_row_stride, int32_t *count, void *workspace,
                       size_t workspace_bytes, void *stream) {
    begin_call();
    if (!mask || !idx || !count || n_rows < 1 || n_kv < 1 || n_kv > 0x7FFFFFFFLL)
        return MLA_FA_ERR_INVALID;
    if (!aligned(mask, 2) || !aligned(idx, 4) || !aligned(count, 4)) return MLA_FA_ERR_INVALID;
    if (idx_row_stride < n_kv || (n_rows > 1 && mask_row_stride < n_kv) || mask_row_stride < 0)
        return MLA_FA_ERR_INVALID;
    const size_t need = fa_mask_compact_workspace_size(n_rows, n_kv);
    const bool vec_rows = aligned(mask, 16) && (n_rows == 1 || mask_row_stride % 8 == 0);
    hipError_t e;
    bool fail;
    if (need == 0 || !vec_rows) {     // the one-workgroup-per-row kernel; workspace untouched
        e = launch_skipped(&fail) ? skipped_status(fail)
                                  : launch_compact(mask, mask_row_stride, n_rows, n_kv, idx, idx_row_stride, count,
                                                   static_cast<hipStream_t>(stream));
    } else {
        if (!workspace || workspace_bytes < need || !aligned(workspace, 4)) return MLA_FA_ERR_WORKSPACE;
        e = launch_skipped(&fail) ? skipped_status(fail)
                                  : launch_compact_chunked(mask, mask_row_stride, n_rows, n_kv, idx, idx_row_stride,
                                                           count, static_cast<int32_t *>(workspace),
                                                           static_cast<hipStream_t>(stream));
    }
    return e == hipSuccess ? MLA_FA_OK : MLA_FA_ERR_HIP;
}

}  // extern "C"
