// kvq_api.hip -- C ABI of libkvq.so (declared in include/kvq.h).
//
// Host side only: argument checks, the split planner, template dispatch and
// launches on the caller's stream.  No allocation, no synchronization, no
// printing, no fallback to another format or path.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "kvq.h"
#include "kvq_decode.hpp"
#include "kvq_device.hpp"
#include "kvq_prefill.hpp"
#include "kvq_write.hpp"

namespace {

using namespace kvq;

constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, 2 = other device
std::atomic<int> g_arch_ok[kMaxDevices];
std::atomic<int> g_cus[kMaxDevices];

kvq_status check_device(int *dev_out = nullptr)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return KVQ_ERR_HIP;
    if (dev >= kMaxDevices)
        return KVQ_ERR_UNSUPPORTED;
    int state = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (state == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return KVQ_ERR_HIP;
        state = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
        g_arch_ok[dev].store(state, std::memory_order_relaxed);
    }
    if (dev_out)
        *dev_out = dev;
    return state == 1 ? KVQ_OK : KVQ_ERR_UNSUPPORTED;
}

// Compute units of the current device (256 on MI355X if the query fails).
int device_cus()
{
    int dev = 0;
    if (check_device(&dev) == KVQ_ERR_HIP || dev >= kMaxDevices)
        return 256;
    const int c = g_cus[dev].load(std::memory_order_relaxed);
    return c > 0 ? c : 256;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

kvq_status check_format(int32_t dtype, int32_t head_dim, int32_t block_size,
                        int32_t group_size)
{
    if (dtype != KVQ_FP16 && dtype != KVQ_INT8 && dtype != KVQ_FP8_E4M3 &&
        dtype != KVQ_FP8_E5M2 && dtype != KVQ_INT4)
        return KVQ_ERR_UNSUPPORTED;
    if (dtype == KVQ_INT4 &&
        (head_dim != 128 || (group_size != 64 && group_size != 128)))
        return KVQ_ERR_UNSUPPORTED;
    if (head_dim != 64 && head_dim != 128)
        return KVQ_ERR_UNSUPPORTED;
    if (block_size != 16 && block_size != 32)
        return KVQ_ERR_UNSUPPORTED;
    if (dtype == KVQ_INT8 || dtype == KVQ_FP8_E4M3) {
        // 0: static scales; 64 / 128: per-group scales
        if (group_size != 0 && group_size != 64 && group_size != 128)
            return KVQ_ERR_UNSUPPORTED;
        if (group_size > head_dim)
            return KVQ_ERR_UNSUPPORTED;
    }
    if (dtype == KVQ_FP8_E5M2 && group_size != 0)
        return KVQ_ERR_UNSUPPORTED;
    return KVQ_OK;
}

// Per-group scale arrays exist (written by the cache write).
bool has_group_scales(int32_t dtype, int32_t group_size)
{
    return (dtype == KVQ_INT8 || dtype == KVQ_FP8_E4M3 || dtype == KVQ_INT4) && group_size > 0;
}

// Bytes of one block's codes in one pool.
int64_t block_code_bytes(int32_t dtype, int32_t num_kv_heads, int32_t block_size,
                         int32_t head_dim)
{
    const int64_t elems = (int64_t)num_kv_heads * block_size * head_dim;
    return dtype == KVQ_FP16 ? 2 * elems : (dtype == KVQ_INT4 ? elems / 2 : elems);
}

kvq_status launch_status()
{
    return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

// ---------------------------------------------------------------- scratch
// Device scratch of kvq_paged_decode_noalloc (the decode workspace of
// callers that cannot allocate).  In host code `scratch` names a host-side
// stand-in, not device memory: its address on a device comes from
// hipGetSymbolAddress with that device current, once per device, and only
// that address is ever passed to kernels.
static __device__ __align__(256) uint8_t scratch[KVQ_NOALLOC_SCRATCH_BYTES];
std::atomic<void *> g_scratch[kMaxDevices];

// Device address of `scratch` on device dev (the current device), or null.
void *scratch_address(int dev)
{
    void *ptr = g_scratch[dev].load(std::memory_order_acquire);
    if (ptr)
        return ptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
        return nullptr;
    g_scratch[dev].store(ptr, std::memory_order_release);
    return ptr;
}

// ---------------------------------------------------------------- run plan
// split_tokens == 0: balanced runs, one per wavefront the GPU holds at once
// (compute units x resident wavefronts per CU for the kernel instance, capped
// at run_waves_per_cu), at most one run per 4 tiles of the largest possible
// batch.  With the wavefront priorities, two waves per SIMD keep HBM as busy
// as three for 1-byte and fp16 codes (and make fewer partials: measured equal
// on C3 / C5 / fp16, 1-3 % faster on C2 / C4; a fourth was 1-5 % slower).
// INT4 tiles carry half the bytes, so INT4 needs more waves per SIMD for the
// same bytes in flight: four where its registers allow it (126 VGPRs: C3
// shape 0.140 ms, against 0.152 ms with three and 12 % more with two).
// split_tokens > 0: one run per span; the launch covers the largest
// possible count.
constexpr int kMaxWavesPerCU = 32;  // hardware bound used for workspace sizing
constexpr int run_waves_per_cu(int fmt)
{
    return fmt == FMT_INT4 ? 16 : 8;  // 4 / 2 per SIMD
}

bool valid_split(int32_t split_tokens)
{
    return split_tokens >= 0 && split_tokens % 16 == 0;
}

int64_t max_tiles(int32_t num_seqs, int32_t num_kv_heads, int32_t max_ctx)
{
    return (int64_t)num_seqs * num_kv_heads * ((max_ctx + 15) / 16);
}

int64_t runs_bound(int32_t num_seqs, int32_t num_kv_heads, int32_t max_ctx,
                   int32_t split_tokens, int64_t balanced_runs)
{
    if (split_tokens > 0)
        return (int64_t)num_seqs * num_kv_heads * ((max_ctx + split_tokens - 1) / split_tokens);
    const int64_t t = max_tiles(num_seqs, num_kv_heads, max_ctx);
    int64_t w = std::min<int64_t>(balanced_runs, (t + 3) / 4);
    return std::max<int64_t>(w, 1);
}

struct WsLayout {
    size_t s_off, meta_off, rec_off, ml_off, acc_off, total;
};

// cols: MFMA columns per unit (query heads per KV head, times the chunk
// tokens of the short-chunk prefill path)
bool workspace_layout(int32_t num_seqs, int32_t cols, int32_t head_dim, int64_t runs, WsLayout &w)
{
    if (num_seqs < 0 || cols <= 0 || head_dim <= 0 || runs < 0)
        return false;
    auto up256 = [](size_t x) { return (x + 255) / 256 * 256; };
    w.s_off = 0;
    w.meta_off = up256((size_t)(num_seqs + 1) * sizeof(int32_t));
    w.rec_off = w.meta_off + 256;
    w.ml_off = w.rec_off + up256((size_t)runs * sizeof(PlanRecord));
    w.acc_off = w.ml_off + up256((size_t)runs * 2 * cols * 2 * sizeof(float));
    w.total = w.acc_off + up256((size_t)runs * 2 * cols * head_dim * sizeof(float));
    return true;
}

// ---------------------------------------------------------------- dispatch
template <int FMT, int D, int G>
void launch_write(const WriteParams &p, hipStream_t s)
{
    const int64_t pairs = (int64_t)p.num_tokens * p.Hkv;
    const int64_t grid = (pairs + kWriteWaves - 1) / kWriteWaves;
    hipLaunchKernelGGL((cache_write_kernel<FMT, D, G>), dim3((unsigned)grid),
                       dim3(64 * kWriteWaves), 0, s, p);
}

template <int FMT, int D>
kvq_status dispatch_write_g(const WriteParams &p, int G, hipStream_t s)
{
    if constexpr (FMT == FMT_INT4) {
        if constexpr (D == 128) {
            if (G == 64)
                launch_write<FMT, D, 64>(p, s);
            else
                launch_write<FMT, D, 128>(p, s);
        } else {
            return KVQ_ERR_UNSUPPORTED;
        }
    } else if constexpr (FMT == FMT_INT8 || FMT == FMT_FP8) {
        if (G == 0)
            launch_write<FMT, D, 0>(p, s);
        else if (G == 64)
            launch_write<FMT, D, 64>(p, s);
        else if constexpr (D >= 128)
            launch_write<FMT, D, 128>(p, s);
        else
            return KVQ_ERR_UNSUPPORTED;
    } else {
        launch_write<FMT, D, 0>(p, s);
    }
    return launch_status();
}

template <int FMT>
kvq_status dispatch_write_d(const WriteParams &p, int D, int G, hipStream_t s)
{
    return D == 64 ? dispatch_write_g<FMT, 64>(p, G, s) : dispatch_write_g<FMT, 128>(p, G, s);
}

// Resident 64-lane workgroups per CU for a kernel instance (cached per device).
template <int FMT, int D, int BS, int NG, int QG = 1>
int waves_per_cu()
{
    static std::atomic<int> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return 4;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        int n = 0;
        const void *kernel =
            reinterpret_cast<const void *>(&paged_decode_kernel<FMT, D, BS, NG, QG>);
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, 64, 0) != hipSuccess ||
            n <= 0)
            n = 4;
        v = std::min(n, run_waves_per_cu(FMT));
        cache[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

struct LaunchPlan {
    int32_t groups;        // MFMA column groups per wavefront (1, or 2 for > 16 columns)
    int32_t split_tokens;
    int32_t max_ctx;
    size_t ws_bytes;
    uint8_t *ws;
};

template <int FMT, int D, int BS, int NG, int QG>
kvq_status launch_decode(DecodeParams p, const LaunchPlan &lp, hipStream_t s)
{
    const int64_t balanced = (int64_t)device_cus() * waves_per_cu<FMT, D, BS, NG, QG>();
    const int64_t runs = runs_bound(p.B, p.Hkv, lp.max_ctx, lp.split_tokens, balanced);
    if (runs > (1 << 30))
        return KVQ_ERR_UNSUPPORTED;
    WsLayout w;
    workspace_layout(p.B, p.cols, D, runs, w);
    if (!lp.ws || lp.ws_bytes < w.total)
        return KVQ_ERR_WORKSPACE;
    int32_t *S = reinterpret_cast<int32_t *>(lp.ws + w.s_off);
    int32_t *meta = reinterpret_cast<int32_t *>(lp.ws + w.meta_off);
    PlanRecord *rec = reinterpret_cast<PlanRecord *>(lp.ws + w.rec_off);
    p.plan_meta = meta;
    p.plan_rec = rec;
    p.inline_plan = (lp.split_tokens == 0 && p.B <= 64 * kInlineSeqs) ? 1 : 0;
    p.ws_ml = reinterpret_cast<float *>(lp.ws + w.ml_off);
    p.ws_acc = reinterpret_cast<float *>(lp.ws + w.acc_off);
    p.W = (int32_t)runs;

    PlanParams pp;
    pp.context_lens = p.context_lens;
    pp.S = S;
    pp.rec = rec;
    pp.meta = meta;
    pp.B = p.B;
    pp.Hkv = p.Hkv;
    pp.max_ctx = lp.max_ctx;
    pp.W = (int32_t)runs;
    pp.span_tiles = lp.split_tokens / 16;
    if (!p.inline_plan)
        hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, pp);
    hipLaunchKernelGGL((paged_decode_kernel<FMT, D, BS, NG, QG>), dim3((unsigned)runs),
                       dim3(64), 0, s, p);
    if (runs > 1)
        hipLaunchKernelGGL((merge_runs_kernel<D>),
                           dim3((unsigned)(runs - 1),
                                (unsigned)((p.cols + kMergeCols - 1) / kMergeCols)),
                           dim3(64 * std::min(p.cols, kMergeCols)), 0, s, p);
    return launch_status();
}

// Chunked prefill (the walk): one workgroup of kPfWaves wavefronts per
// (sequence, KV head, block of 128 / r chunk tokens); p.groups query blocks
// per pair.
template <int FMT, int D, int BS, int NG>
kvq_status launch_prefill(const DecodeParams &p, hipStream_t s)
{
    // query blocks per (sequence, KV head) pair, times the pairs rounded up
    // to the 8 XCDs (see the kernel)
    const int64_t grid = (int64_t)p.groups * (((int64_t)p.B * p.Hkv + 7) / 8 * 8);
    if (grid > (int64_t)INT32_MAX)
        return KVQ_ERR_UNSUPPORTED;
    if (grid == 0)
        return KVQ_OK;
    hipLaunchKernelGGL((prefill_kernel<FMT, D, BS, NG>), dim3((unsigned)grid),
                       dim3(64 * kPfWaves), 0, s, p);
    return launch_status();
}

template <int FMT, int D, int BS, int NG>
kvq_status launch_attention(const DecodeParams &p, const LaunchPlan *lp, hipStream_t s)
{
    if (!lp)
        return launch_prefill<FMT, D, BS, NG>(p, s);
    return lp->groups == 2 ? launch_decode<FMT, D, BS, NG, 2>(p, *lp, s)
                           : launch_decode<FMT, D, BS, NG, 1>(p, *lp, s);
}

// Kernel instances: NG = head_dim / group_size for per-group scales, 0 for
// static scales (FP8 per head, INT8 per channel) and fp16.  lp == nullptr
// selects chunked prefill.
template <int FMT, int D, int BS>
kvq_status dispatch_decode_ng(const DecodeParams &p, const LaunchPlan *lp, int G, hipStream_t s)
{
    if constexpr (FMT == FMT_INT4) {
        if constexpr (D == 128)
            return G == 64 ? launch_attention<FMT, D, BS, 2>(p, lp, s)
                           : launch_attention<FMT, D, BS, 1>(p, lp, s);
        return KVQ_ERR_UNSUPPORTED;
    } else if constexpr (FMT == FMT_INT8 || FMT == FMT_FP8) {
        if (G == 0)
            return launch_attention<FMT, D, BS, 0>(p, lp, s);
        const int NG = D / G;
        if (NG == 1)
            return launch_attention<FMT, D, BS, 1>(p, lp, s);
        if constexpr (D == 128)
            return launch_attention<FMT, D, BS, 2>(p, lp, s);
        return KVQ_ERR_UNSUPPORTED;
    } else {
        return launch_attention<FMT, D, BS, 0>(p, lp, s);
    }
}

template <int FMT>
kvq_status dispatch_decode(const DecodeParams &p, const LaunchPlan *lp, int D, int BS, int G,
                           hipStream_t s)
{
    if (D == 64)
        return BS == 16 ? dispatch_decode_ng<FMT, 64, 16>(p, lp, G, s)
                        : dispatch_decode_ng<FMT, 64, 32>(p, lp, G, s);
    return BS == 16 ? dispatch_decode_ng<FMT, 128, 16>(p, lp, G, s)
                    : dispatch_decode_ng<FMT, 128, 32>(p, lp, G, s);
}

kvq_status dispatch_attention(const DecodeParams &p, const LaunchPlan *lp, int32_t dtype,
                              int D, int BS, int G, hipStream_t s)
{
    switch (dtype) {
    case KVQ_INT8: return dispatch_decode<FMT_INT8>(p, lp, D, BS, G, s);
    case KVQ_FP8_E4M3: return dispatch_decode<FMT_FP8>(p, lp, D, BS, G, s);
    case KVQ_FP8_E5M2: return dispatch_decode<FMT_E5M2>(p, lp, D, BS, 0, s);
    case KVQ_INT4: return dispatch_decode<FMT_INT4>(p, lp, D, BS, G, s);
    default: return dispatch_decode<FMT_FP16>(p, lp, D, BS, 0, s);
    }
}

}  // namespace

extern "C" {

const char *kvq_status_string(kvq_status status)
{
    switch (status) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_INVALID_ARG: return "invalid argument";
    case KVQ_ERR_UNSUPPORTED: return "unsupported format, shape or device";
    case KVQ_ERR_WORKSPACE: return "workspace too small";
    case KVQ_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

int32_t kvq_version(void) { return 100; }

static kvq_status write_impl(const void *k, const void *v, const int64_t *slot_mapping,
                             int32_t num_tokens, int32_t num_kv_heads_src,
                             const int32_t *head_ids, int32_t num_kv_heads, int32_t head_dim,
                             int32_t block_size, int32_t num_blocks, int32_t dtype,
                             int32_t group_size, void *k_pool, void *v_pool, float *k_scale,
                             float *v_scale, void *stream)
{
    if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0 || num_kv_heads_src <= 0)
        return KVQ_ERR_INVALID_ARG;
    kvq_status st = check_format(dtype, head_dim, block_size, group_size);
    if (st != KVQ_OK)
        return st;
    if (num_tokens == 0)
        return KVQ_OK;
    if (!k || !v || !slot_mapping || !k_pool || !v_pool)
        return KVQ_ERR_INVALID_ARG;
    if (dtype != KVQ_FP16 && (!k_scale || !v_scale))
        return KVQ_ERR_INVALID_ARG;
    if (!aligned16(k) || !aligned16(v) || !aligned16(k_pool) || !aligned16(v_pool) ||
        (k_scale && !aligned16(k_scale)) || (v_scale && !aligned16(v_scale)))
        return KVQ_ERR_INVALID_ARG;
    st = check_device();
    if (st != KVQ_OK)
        return st;

    WriteParams p;
    p.k = static_cast<const f16 *>(k);
    p.v = static_cast<const f16 *>(v);
    p.slots = slot_mapping;
    p.k_pool = static_cast<uint8_t *>(k_pool);
    p.v_pool = static_cast<uint8_t *>(v_pool);
    p.k_scale = k_scale;
    p.v_scale = v_scale;
    p.num_tokens = num_tokens;
    p.Hkv = num_kv_heads;
    p.block_size = block_size;
    p.num_slots = (int64_t)num_blocks * block_size;
    p.head_ids = head_ids;
    p.Hkv_src = num_kv_heads_src;
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (dtype) {
    case KVQ_INT8: return dispatch_write_d<FMT_INT8>(p, head_dim, group_size, s);
    case KVQ_FP8_E4M3: return dispatch_write_d<FMT_FP8>(p, head_dim, group_size, s);
    case KVQ_FP8_E5M2: return dispatch_write_d<FMT_E5M2>(p, head_dim, 0, s);
    case KVQ_INT4: return dispatch_write_d<FMT_INT4>(p, head_dim, group_size, s);
    default: return dispatch_write_d<FMT_FP16>(p, head_dim, 0, s);
    }
}

kvq_status kvq_cache_write(const void *k, const void *v, const int64_t *slot_mapping,
                           int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int32_t num_blocks, int32_t dtype,
                           int32_t group_size, void *k_pool, void *v_pool, float *k_scale,
                           float *v_scale, void *stream)
{
    return write_impl(k, v, slot_mapping, num_tokens, num_kv_heads, nullptr, num_kv_heads,
                      head_dim, block_size, num_blocks, dtype, group_size, k_pool, v_pool,
                      k_scale, v_scale, stream);
}

kvq_status kvq_cache_write_heads(const void *k, const void *v, const int64_t *slot_mapping,
                                 int32_t num_tokens, int32_t num_kv_heads_src,
                                 const int32_t *kv_head_ids, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                 int32_t dtype, int32_t group_size, void *k_pool, void *v_pool,
                                 float *k_scale, float *v_scale, void *stream)
{
    if (!kv_head_ids && num_tokens > 0)
        return KVQ_ERR_INVALID_ARG;
    return write_impl(k, v, slot_mapping, num_tokens, num_kv_heads_src, kv_head_ids,
                      num_kv_heads, head_dim, block_size, num_blocks, dtype, group_size,
                      k_pool, v_pool, k_scale, v_scale, stream);
}

size_t kvq_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size,
                                 int32_t max_context_len, int32_t split_tokens)
{
    (void)block_size;
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
        num_q_heads % num_kv_heads != 0 || head_dim <= 0 || max_context_len < 1 ||
        !valid_split(split_tokens))
        return SIZE_MAX;
    const int64_t balanced = (int64_t)device_cus() * kMaxWavesPerCU;
    const int64_t runs = runs_bound(num_seqs, num_kv_heads, max_context_len, split_tokens,
                                    balanced);
    WsLayout w;
    if (!workspace_layout(num_seqs, num_q_heads / num_kv_heads, head_dim, runs, w))
        return SIZE_MAX;
    return w.total;
}

// How kvq_paged_prefill cuts the work.
//   walk:    one workgroup of four wavefronts per (sequence, KV head, block
//            of 128 / r chunk tokens) walks the tokens it needs, staging
//            each 32-key step in LDS once for its 128 rows (the prefill
//            kernel);
//   short:   chunks of at most 32 / r tokens (up to 32 MFMA columns of chunk
//            tokens x query heads, one or two column groups per wavefront)
//            go through the decode partition: balanced runs over every
//            resident wavefront and the merge of cut units;
//   virtual: longer chunks are cut into virtual sequences of 32 / r tokens
//            (virtual_chunks_kernel), which the decode partition then walks.
// Automatic choice: short chunks always split; longer ones split when the
// walk would launch fewer wavefronts than the GPU holds (few sequences and
// chunk tokens over long contexts), else walk (e.g. whole prompts).
enum PrefillPath { kPathWalk, kPathShort, kPathVirtual };
struct PrefillCut {
    PrefillPath path;
    int32_t qpg;    // chunk tokens per virtual sequence
    int32_t J;      // virtual sequences per sequence
    int32_t cols;   // MFMA columns per unit
    int64_t V;      // sequences the decode partition sees
};

static bool valid_prefill_mode(int32_t mode)
{
    return mode == KVQ_PREFILL_AUTO || mode == KVQ_PREFILL_WALK || mode == KVQ_PREFILL_SPLIT;
}

static PrefillCut prefill_cut(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t max_query_len, int32_t mode)
{
    const int32_t r = num_q_heads / num_kv_heads;
    PrefillCut c{kPathWalk, 0, 1, r, num_seqs};
    if (max_query_len < 1 || mode == KVQ_PREFILL_WALK)
        return c;
    const bool fits = (int64_t)max_query_len * r <= 32;
    if (mode == KVQ_PREFILL_AUTO && !fits) {
        const int64_t tokens_per_group = prefill_tokens_per_group(r);
        const int64_t walk_waves = (int64_t)num_seqs * num_kv_heads * kPfWaves *
                                   ((max_query_len + tokens_per_group - 1) / tokens_per_group);
        if (walk_waves >= (int64_t)device_cus() * run_waves_per_cu(FMT_INT8))
            return c;
    }
    if (fits) {
        c.path = kPathShort;
        c.cols = max_query_len * r;
        return c;
    }
    c.path = kPathVirtual;
    c.qpg = 32 / r;
    c.J = (max_query_len + c.qpg - 1) / c.qpg;
    c.cols = c.qpg * r;
    c.V = (int64_t)num_seqs * c.J;
    return c;
}

// Workspace of a split prefill: the virtual-sequence arrays (virtual path),
// then the decode workspace for the sequences the partition sees.
struct PrefillWs {
    size_t vctx_off, vrow_off, vqs_off, decode_off, total;
};

static bool prefill_ws(const PrefillCut &c, int32_t num_kv_heads, int32_t head_dim,
                       int32_t max_context_len, PrefillWs &w)
{
    auto up256 = [](size_t x) { return (x + 255) / 256 * 256; };
    const int64_t nv = c.path == kPathVirtual ? c.V : 0;
    w.vctx_off = 0;
    w.vrow_off = up256((size_t)nv * 4);
    w.vqs_off = w.vrow_off + up256((size_t)nv * 4);
    w.decode_off = c.path == kPathVirtual ? w.vqs_off + up256((size_t)(nv + 1) * 4) : 0;
    const int64_t balanced = (int64_t)device_cus() * kMaxWavesPerCU;
    const int64_t runs = runs_bound((int32_t)c.V, num_kv_heads, max_context_len, 0, balanced);
    WsLayout d;
    if (!workspace_layout((int32_t)c.V, c.cols, head_dim, runs, d))
        return false;
    w.total = w.decode_off + d.total;
    return true;
}

size_t kvq_prefill_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t block_size,
                                  int32_t max_context_len, int32_t max_query_len,
                                  int32_t split_mode)
{
    (void)block_size;
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
        num_q_heads % num_kv_heads != 0 || head_dim <= 0 || max_query_len < 0 ||
        max_context_len < max_query_len || !valid_prefill_mode(split_mode) ||
        num_q_heads / num_kv_heads > 16)
        return SIZE_MAX;
    const PrefillCut c =
        prefill_cut(num_seqs, num_q_heads, num_kv_heads, max_query_len, split_mode);
    if (c.path == kPathWalk || num_seqs == 0)
        return 0;
    if (c.V > INT32_MAX)
        return SIZE_MAX;
    PrefillWs w;
    if (!prefill_ws(c, num_kv_heads, head_dim, max_context_len, w))
        return SIZE_MAX;
    return w.total;
}

// num_q_heads / num_kv_heads: the model's heads (q and out rows, GQA ratio);
// head_ids: the pool's heads as model KV heads (null: the pool holds all
// num_kv_heads); pool_heads: heads in the pool.
static kvq_status decode_impl(const void *q, const void *k_pool, const void *v_pool,
                              const float *k_scale, const float *v_scale,
                              const int32_t *block_tables, int32_t max_blocks_per_seq,
                              const int32_t *context_lens, int32_t max_context_len,
                              int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                              const int32_t *head_ids, int32_t pool_heads, int32_t head_dim,
                              int32_t block_size, int32_t num_blocks, int32_t dtype,
                              int32_t group_size, float softmax_scale, int32_t split_tokens,
                              void *out, void *workspace, size_t workspace_bytes, void *stream)
{
    kvq_status st = check_format(dtype, head_dim, block_size, group_size);
    if (st != KVQ_OK)
        return st;
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 ||
        max_blocks_per_seq <= 0 || num_blocks > kBlockIdMask + 1 || pool_heads <= 0 ||
        pool_heads > num_kv_heads)
        return KVQ_ERR_INVALID_ARG;
    if (num_q_heads % num_kv_heads != 0)
        return KVQ_ERR_INVALID_ARG;
    const int32_t r = num_q_heads / num_kv_heads;
    if (r > 16)
        return KVQ_ERR_UNSUPPORTED;
    if (num_seqs == 0)
        return KVQ_OK;
    if (max_context_len < 1 || (int64_t)max_blocks_per_seq * block_size < max_context_len)
        return KVQ_ERR_INVALID_ARG;
    if (!valid_split(split_tokens))
        return KVQ_ERR_INVALID_ARG;
    if (max_tiles(num_seqs, pool_heads, max_context_len) >= (int64_t)1 << 30)
        return KVQ_ERR_UNSUPPORTED;
    if (!(softmax_scale >= 0.0f) || std::isinf(softmax_scale))
        return KVQ_ERR_INVALID_ARG;
    if (!q || !k_pool || !v_pool || !block_tables || !context_lens || !out)
        return KVQ_ERR_INVALID_ARG;
    if (dtype != KVQ_FP16 && (!k_scale || !v_scale))
        return KVQ_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(out) || !aligned16(k_pool) || !aligned16(v_pool) ||
        (workspace && !aligned16(workspace)) || (k_scale && !aligned16(k_scale)) ||
        (v_scale && !aligned16(v_scale)))
        return KVQ_ERR_INVALID_ARG;
    if (!workspace)
        return KVQ_ERR_WORKSPACE;
    st = check_device();
    if (st != KVQ_OK)
        return st;

    DecodeParams p = {};
    p.q = static_cast<const f16 *>(q);
    p.k_pool = static_cast<const uint8_t *>(k_pool);
    p.v_pool = static_cast<const uint8_t *>(v_pool);
    p.k_scale = k_scale;
    p.v_scale = v_scale;
    p.block_tables = block_tables;
    p.context_lens = context_lens;
    p.out = static_cast<f16 *>(out);
    p.B = num_seqs;
    p.max_blocks = max_blocks_per_seq;
    p.max_ctx = max_context_len;
    p.num_blocks = num_blocks;
    p.Hq = num_q_heads;
    p.Hkv = pool_heads;
    p.r = r;
    p.cols = r;
    p.head_ids = head_ids;
    const float sm = softmax_scale > 0.0f ? softmax_scale : 1.0f / std::sqrt((float)head_dim);
    p.score_scale = sm * 1.4426950408889634f;  // log2(e): softmax in base 2
    LaunchPlan lp;
    lp.groups = 1;
    lp.split_tokens = split_tokens;
    lp.max_ctx = max_context_len;
    lp.ws_bytes = workspace_bytes;
    lp.ws = static_cast<uint8_t *>(workspace);
    return dispatch_attention(p, &lp, dtype, head_dim, block_size, group_size,
                              static_cast<hipStream_t>(stream));
}

kvq_status kvq_paged_decode(const void *q, const void *k_pool, const void *v_pool,
                            const float *k_scale, const float *v_scale,
                            const int32_t *block_tables, int32_t max_blocks_per_seq,
                            const int32_t *context_lens, int32_t max_context_len,
                            int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t block_size, int32_t num_blocks,
                            int32_t dtype, int32_t group_size, float softmax_scale,
                            int32_t split_tokens, void *out, void *workspace,
                            size_t workspace_bytes, void *stream)
{
    return decode_impl(q, k_pool, v_pool, k_scale, v_scale, block_tables, max_blocks_per_seq,
                       context_lens, max_context_len, num_seqs, num_q_heads, num_kv_heads,
                       nullptr, num_kv_heads, head_dim, block_size, num_blocks, dtype,
                       group_size, softmax_scale, split_tokens, out, workspace,
                       workspace_bytes, stream);
}

kvq_status kvq_paged_decode_heads(const void *q, const void *k_pool, const void *v_pool,
                                  const float *k_scale, const float *v_scale,
                                  const int32_t *block_tables, int32_t max_blocks_per_seq,
                                  const int32_t *context_lens, int32_t max_context_len,
                                  int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                  const int32_t *kv_head_ids, int32_t pool_heads,
                                  int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                  int32_t dtype, int32_t group_size, float softmax_scale,
                                  int32_t split_tokens, void *out, void *workspace,
                                  size_t workspace_bytes, void *stream)
{
    if (!kv_head_ids && num_seqs > 0)
        return KVQ_ERR_INVALID_ARG;
    return decode_impl(q, k_pool, v_pool, k_scale, v_scale, block_tables, max_blocks_per_seq,
                       context_lens, max_context_len, num_seqs, num_q_heads, num_kv_heads,
                       kv_head_ids, pool_heads, head_dim, block_size, num_blocks, dtype,
                       group_size, softmax_scale, split_tokens, out, workspace,
                       workspace_bytes, stream);
}

kvq_status kvq_paged_decode_noalloc(const void *q, const void *k_pool, const void *v_pool,
                                    const float *k_scale, const float *v_scale,
                                    const int32_t *block_tables, int32_t max_blocks_per_seq,
                                    const int32_t *context_lens, int32_t max_context_len,
                                    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                    int32_t dtype, int32_t group_size, float softmax_scale,
                                    int32_t split_tokens, void *out, void *stream)
{
    int dev = 0;
    const kvq_status st = check_device(&dev);
    if (st != KVQ_OK)
        return st;
    void *ws = scratch_address(dev);
    if (!ws)
        return KVQ_ERR_HIP;
    // the plan's exact need is checked against the array's size at launch
    return decode_impl(q, k_pool, v_pool, k_scale, v_scale, block_tables, max_blocks_per_seq,
                       context_lens, max_context_len, num_seqs, num_q_heads, num_kv_heads,
                       nullptr, num_kv_heads, head_dim, block_size, num_blocks, dtype,
                       group_size, softmax_scale, split_tokens, out, ws,
                       KVQ_NOALLOC_SCRATCH_BYTES, stream);
}

kvq_status kvq_paged_prefill(const void *q, const int32_t *query_start, int32_t max_query_len,
                             const void *k_pool, const void *v_pool, const float *k_scale,
                             const float *v_scale, const int32_t *block_tables,
                             int32_t max_blocks_per_seq, const int32_t *context_lens,
                             int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int32_t num_blocks, int32_t dtype, int32_t group_size,
                             float softmax_scale, int32_t split_mode, void *out,
                             void *workspace, size_t workspace_bytes, void *stream)
{
    kvq_status st = check_format(dtype, head_dim, block_size, group_size);
    if (st != KVQ_OK)
        return st;
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 ||
        max_blocks_per_seq <= 0 || num_blocks > kBlockIdMask + 1 || max_query_len < 0)
        return KVQ_ERR_INVALID_ARG;
    if (num_q_heads % num_kv_heads != 0)
        return KVQ_ERR_INVALID_ARG;
    const int32_t r = num_q_heads / num_kv_heads;
    if (r > 16)
        return KVQ_ERR_UNSUPPORTED;
    if (num_seqs == 0 || max_query_len == 0)
        return KVQ_OK;
    if (max_context_len < max_query_len ||
        (int64_t)max_blocks_per_seq * block_size < max_context_len)
        return KVQ_ERR_INVALID_ARG;
    if (!(softmax_scale >= 0.0f) || std::isinf(softmax_scale) || !valid_prefill_mode(split_mode))
        return KVQ_ERR_INVALID_ARG;
    if (!q || !query_start || !k_pool || !v_pool || !block_tables || !context_lens || !out)
        return KVQ_ERR_INVALID_ARG;
    if (dtype != KVQ_FP16 && (!k_scale || !v_scale))
        return KVQ_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(out) || !aligned16(k_pool) || !aligned16(v_pool) ||
        (k_scale && !aligned16(k_scale)) || (v_scale && !aligned16(v_scale)) ||
        (workspace && !aligned16(workspace)))
        return KVQ_ERR_INVALID_ARG;
    const PrefillCut cut =
        prefill_cut(num_seqs, num_q_heads, num_kv_heads, max_query_len, split_mode);
    PrefillWs pw{};
    if (cut.path != kPathWalk) {
        if (cut.V > INT32_MAX ||
            max_tiles((int32_t)cut.V, num_kv_heads, max_context_len) >= (int64_t)1 << 30)
            return KVQ_ERR_UNSUPPORTED;
        if (!prefill_ws(cut, num_kv_heads, head_dim, max_context_len, pw))
            return KVQ_ERR_INVALID_ARG;
        if (!workspace || workspace_bytes < pw.total)
            return KVQ_ERR_WORKSPACE;
    }
    st = check_device();
    if (st != KVQ_OK)
        return st;

    DecodeParams p = {};
    p.q = static_cast<const f16 *>(q);
    p.k_pool = static_cast<const uint8_t *>(k_pool);
    p.v_pool = static_cast<const uint8_t *>(v_pool);
    p.k_scale = k_scale;
    p.v_scale = v_scale;
    p.block_tables = block_tables;
    p.context_lens = context_lens;
    p.out = static_cast<f16 *>(out);
    p.B = num_seqs;
    p.max_blocks = max_blocks_per_seq;
    p.max_ctx = max_context_len;
    p.num_blocks = num_blocks;
    p.Hq = num_q_heads;
    p.Hkv = num_kv_heads;
    p.r = r;
    const float sm = softmax_scale > 0.0f ? softmax_scale : 1.0f / std::sqrt((float)head_dim);
    p.score_scale = sm * 1.4426950408889634f;
    p.q_start = query_start;
    p.groups = (max_query_len + prefill_tokens_per_group(r) - 1) / prefill_tokens_per_group(r);
    if (cut.path != kPathWalk) {  // the decode partition, columns = (chunk token, query head)
        hipStream_t s = static_cast<hipStream_t>(stream);
        uint8_t *ws = static_cast<uint8_t *>(workspace);
        if (cut.path == kPathVirtual) {
            VirtualParams vp;
            vp.q_start = query_start;
            vp.context_lens = context_lens;
            vp.vctx = reinterpret_cast<int32_t *>(ws + pw.vctx_off);
            vp.vrow = reinterpret_cast<int32_t *>(ws + pw.vrow_off);
            vp.vqs = reinterpret_cast<int32_t *>(ws + pw.vqs_off);
            vp.B = num_seqs;
            vp.J = cut.J;
            vp.qpg = cut.qpg;
            vp.max_ctx = max_context_len;
            const int64_t threads = cut.V + 1;
            hipLaunchKernelGGL(virtual_chunks_kernel, dim3((unsigned)((threads + 255) / 256)),
                               dim3(256), 0, s, vp);
            p.B = (int32_t)cut.V;
            p.context_lens = vp.vctx;
            p.q_start = vp.vqs;
            p.seq_row = vp.vrow;
        }
        p.cols = cut.cols;
        LaunchPlan lp;
        lp.groups = p.cols > 16 ? 2 : 1;
        lp.split_tokens = 0;
        lp.max_ctx = max_context_len;
        lp.ws_bytes = workspace_bytes - pw.decode_off;
        lp.ws = ws + pw.decode_off;
        return dispatch_attention(p, &lp, dtype, head_dim, block_size, group_size, s);
    }
    p.cols = r;
    return dispatch_attention(p, nullptr, dtype, head_dim, block_size, group_size,
                              static_cast<hipStream_t>(stream));
}

kvq_status kvq_copy_blocks(const int32_t *block_pairs, int32_t num_pairs, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, int32_t num_blocks,
                           int32_t dtype, int32_t group_size, void *k_pool, void *v_pool,
                           float *k_scale, float *v_scale, void *stream)
{
    kvq_status st = check_format(dtype, head_dim, block_size, group_size);
    if (st != KVQ_OK)
        return st;
    if (num_pairs < 0 || num_kv_heads <= 0 || num_blocks <= 0)
        return KVQ_ERR_INVALID_ARG;
    if (num_pairs == 0)
        return KVQ_OK;
    if (!block_pairs || !k_pool || !v_pool || !aligned16(k_pool) || !aligned16(v_pool))
        return KVQ_ERR_INVALID_ARG;
    const bool group_scales = has_group_scales(dtype, group_size);
    if (group_scales && (!k_scale || !v_scale))
        return KVQ_ERR_INVALID_ARG;
    st = check_device();
    if (st != KVQ_OK)
        return st;
    CopyParams p;
    p.pairs = block_pairs;
    p.k_pool = static_cast<uint8_t *>(k_pool);
    p.v_pool = static_cast<uint8_t *>(v_pool);
    p.k_scale = k_scale;
    p.v_scale = v_scale;
    p.block_bytes = block_code_bytes(dtype, num_kv_heads, block_size, head_dim);
    p.scale_block_floats =
        group_scales ? (int64_t)num_kv_heads * block_size * (head_dim / group_size) : 0;
    p.num_blocks = num_blocks;
    const unsigned chunks = (unsigned)((p.block_bytes / 16 + 255) / 256);
    hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)num_pairs, chunks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), p);
    return launch_status();
}

size_t kvq_swap_block_bytes(int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            int32_t dtype, int32_t group_size)
{
    if (num_kv_heads <= 0 || check_format(dtype, head_dim, block_size, group_size) != KVQ_OK)
        return SIZE_MAX;
    const bool group_scales = has_group_scales(dtype, group_size);
    const size_t codes = (size_t)block_code_bytes(dtype, num_kv_heads, block_size, head_dim);
    const size_t scales =
        group_scales ? (size_t)num_kv_heads * block_size * (head_dim / group_size) * 4 : 0;
    return (2 * codes + 2 * scales + 255) / 256 * 256;
}

namespace {

kvq_status swap_blocks(const int32_t *pairs, int32_t num_pairs, int32_t num_kv_heads,
                       int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t dtype,
                       int32_t group_size, void *k_pool, void *v_pool, float *k_scale,
                       float *v_scale, void *buffer, int64_t num_slots, int to_buffer,
                       void *stream)
{
    kvq_status st = check_format(dtype, head_dim, block_size, group_size);
    if (st != KVQ_OK)
        return st;
    if (num_pairs < 0 || num_kv_heads <= 0 || num_blocks <= 0 || num_slots < 0)
        return KVQ_ERR_INVALID_ARG;
    if (num_pairs == 0)
        return KVQ_OK;
    const bool group_scales = has_group_scales(dtype, group_size);
    if (!pairs || !k_pool || !v_pool || !buffer || (group_scales && (!k_scale || !v_scale)))
        return KVQ_ERR_INVALID_ARG;
    if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(buffer) ||
        (group_scales && (!aligned16(k_scale) || !aligned16(v_scale))))
        return KVQ_ERR_INVALID_ARG;
    st = check_device();
    if (st != KVQ_OK)
        return st;
    SwapParams p;
    p.pairs = pairs;
    p.k_pool = static_cast<uint8_t *>(k_pool);
    p.v_pool = static_cast<uint8_t *>(v_pool);
    p.k_scale = group_scales ? reinterpret_cast<uint8_t *>(k_scale) : nullptr;
    p.v_scale = group_scales ? reinterpret_cast<uint8_t *>(v_scale) : nullptr;
    p.buf = static_cast<uint8_t *>(buffer);
    p.block_bytes = block_code_bytes(dtype, num_kv_heads, block_size, head_dim);
    p.scale_bytes =
        group_scales ? (int64_t)num_kv_heads * block_size * (head_dim / group_size) * 4 : 0;
    p.slot_bytes = (int64_t)kvq_swap_block_bytes(num_kv_heads, head_dim, block_size, dtype,
                                                 group_size);
    p.num_slots = num_slots;
    p.num_blocks = num_blocks;
    p.to_buffer = to_buffer;
    const unsigned chunks = (unsigned)((p.block_bytes / 16 + 255) / 256);
    hipLaunchKernelGGL(swap_blocks_kernel, dim3((unsigned)num_pairs, chunks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), p);
    return launch_status();
}

}  // namespace

kvq_status kvq_swap_out(const int32_t *block_slot_pairs, int32_t num_pairs,
                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                        int32_t num_blocks, int32_t dtype, int32_t group_size,
                        const void *k_pool, const void *v_pool, const float *k_scale,
                        const float *v_scale, void *dst, int64_t num_slots, void *stream)
{
    return swap_blocks(block_slot_pairs, num_pairs, num_kv_heads, head_dim, block_size,
                       num_blocks, dtype, group_size, const_cast<void *>(k_pool),
                       const_cast<void *>(v_pool), const_cast<float *>(k_scale),
                       const_cast<float *>(v_scale), dst, num_slots, 1, stream);
}

kvq_status kvq_swap_in(const int32_t *block_slot_pairs, int32_t num_pairs, int32_t num_kv_heads,
                       int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t dtype,
                       int32_t group_size, const void *src, int64_t num_slots, void *k_pool,
                       void *v_pool, float *k_scale, float *v_scale, void *stream)
{
    return swap_blocks(block_slot_pairs, num_pairs, num_kv_heads, head_dim, block_size,
                       num_blocks, dtype, group_size, k_pool, v_pool, k_scale, v_scale,
                       const_cast<void *>(src), num_slots, 0, stream);
}

}  // extern "C"
