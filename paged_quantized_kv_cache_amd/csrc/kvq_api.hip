// kvq_api.hip -- C ABI of libkvq.so (declared in include/kvq.h).
//
// Host side only: argument checks, the split planner, template dispatch and
// launches on the caller's stream.  No allocation, no synchronization, no
// printing, no fallback to another format or path.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "kvq.h"
#include "kvq_decode.hpp"
#include "kvq_device.hpp"
#include "kvq_write.hpp"

namespace {

using namespace kvq;

constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, 2 = other device
std::atomic<int> g_arch_ok[kMaxDevices];

kvq_status check_device()
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
        g_arch_ok[dev].store(state, std::memory_order_relaxed);
    }
    return state == 1 ? KVQ_OK : KVQ_ERR_UNSUPPORTED;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

kvq_status check_format(int32_t dtype, int32_t head_dim, int32_t block_size,
                        int32_t group_size)
{
    if (dtype != KVQ_FP16 && dtype != KVQ_INT8 && dtype != KVQ_FP8_E4M3)
        return KVQ_ERR_UNSUPPORTED;
    if (head_dim != 64 && head_dim != 128)
        return KVQ_ERR_UNSUPPORTED;
    if (block_size != 16 && block_size != 32)
        return KVQ_ERR_UNSUPPORTED;
    if (dtype == KVQ_INT8) {
        if (group_size != 64 && group_size != 128)
            return KVQ_ERR_UNSUPPORTED;
        if (group_size > head_dim || head_dim % group_size != 0)
            return KVQ_ERR_UNSUPPORTED;
    }
    return KVQ_OK;
}

kvq_status launch_status()
{
    return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

// ---------------------------------------------------------------- split plan
// Tokens per split.  Splits are spans of logical tokens (multiples of 16), so
// they never depend on where blocks sit in the pool.  The automatic choice
// cuts long contexts into spans of at most 1024 tokens (bounded per-item work
// keeps skewed length mixes balanced across the 256 CUs) and shortens spans
// when there are too few (sequence, KV head) units to occupy the GPU.
constexpr int kAutoMaxSpan = 1024;
constexpr int kAutoMinSpan = 256;
constexpr int kTargetItems = 2048;

// A split covers at most kMaxSplitBlocks blocks (one block id per lane).
constexpr int kMaxSplitBlocks = 64;

int32_t plan_span(int32_t num_seqs, int32_t num_kv_heads, int32_t block_size,
                  int32_t max_ctx, int32_t split_tokens)
{
    if (split_tokens > 0)
        return split_tokens;
    const int64_t units = (int64_t)num_seqs * num_kv_heads;
    int64_t want = (kTargetItems + units - 1) / units;  // splits per unit
    if (want < 1)
        want = 1;
    int64_t span = (max_ctx + want - 1) / want;
    span = (span + 15) / 16 * 16;
    if (span > kAutoMaxSpan)
        span = kAutoMaxSpan;
    if (span < kAutoMinSpan)
        span = kAutoMinSpan;
    if (span >= max_ctx)
        span = (max_ctx + 15) / 16 * 16;  // one split
    if (span > (int64_t)kMaxSplitBlocks * block_size)
        span = (int64_t)kMaxSplitBlocks * block_size;
    return (int32_t)span;
}

struct WsLayout {
    size_t ml_off, acc_off, total;
    int32_t span, max_splits;
};

bool valid_split(int32_t block_size, int32_t split_tokens)
{
    return split_tokens >= 0 && split_tokens % 16 == 0 &&
           split_tokens <= kMaxSplitBlocks * block_size;
}

bool workspace_layout(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, int32_t block_size, int32_t max_ctx,
                      int32_t split_tokens, WsLayout &w)
{
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        max_ctx < 1 || (block_size != 16 && block_size != 32) ||
        !valid_split(block_size, split_tokens))
        return false;
    w.span = plan_span(num_seqs, num_kv_heads, block_size, max_ctx, split_tokens);
    w.max_splits = (max_ctx + w.span - 1) / w.span;
    if (w.max_splits <= 1 || num_seqs == 0) {
        w.ml_off = w.acc_off = w.total = 0;
        return true;
    }
    auto up256 = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t items = (size_t)num_seqs * num_q_heads * w.max_splits;
    w.ml_off = 0;
    w.acc_off = w.ml_off + up256(items * 2 * sizeof(float));
    w.total = w.acc_off + up256(items * head_dim * sizeof(float));
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
    if constexpr (FMT == FMT_INT8) {
        if (G == 64)
            launch_write<FMT, D, 64>(p, s);
        else if constexpr (D >= 128)
            launch_write<FMT, D, 128>(p, s);
        else
            return KVQ_ERR_UNSUPPORTED;
    } else {
        launch_write<FMT, D, D>(p, s);
    }
    return launch_status();
}

template <int FMT>
kvq_status dispatch_write_d(const WriteParams &p, int D, int G, hipStream_t s)
{
    return D == 64 ? dispatch_write_g<FMT, 64>(p, G, s) : dispatch_write_g<FMT, 128>(p, G, s);
}

template <int FMT, int D, int BS, int NG>
void launch_decode(const DecodeParams &p, int B, int Hkv, int splits, hipStream_t s)
{
    const int64_t items = (int64_t)splits * Hkv * B;
    hipLaunchKernelGGL((paged_decode_kernel<FMT, D, BS, NG>), dim3((unsigned)items),
                       dim3(64), 0, s, p);
    if (splits > 1)
        hipLaunchKernelGGL((merge_splits_kernel<D>), dim3((unsigned)p.Hq, (unsigned)B),
                           dim3(64), 0, s, p);
}

template <int FMT, int D, int BS>
kvq_status dispatch_decode_ng(const DecodeParams &p, int B, int Hkv, int splits, int G,
                              hipStream_t s)
{
    if constexpr (FMT == FMT_INT8) {
        const int NG = D / G;
        if (NG == 1)
            launch_decode<FMT, D, BS, 1>(p, B, Hkv, splits, s);
        else if constexpr (D == 128)
            launch_decode<FMT, D, BS, 2>(p, B, Hkv, splits, s);
        else
            return KVQ_ERR_UNSUPPORTED;
    } else {
        launch_decode<FMT, D, BS, 1>(p, B, Hkv, splits, s);
    }
    return launch_status();
}

template <int FMT>
kvq_status dispatch_decode(const DecodeParams &p, int B, int Hkv, int splits, int D,
                           int BS, int G, hipStream_t s)
{
    if (D == 64)
        return BS == 16 ? dispatch_decode_ng<FMT, 64, 16>(p, B, Hkv, splits, G, s)
                        : dispatch_decode_ng<FMT, 64, 32>(p, B, Hkv, splits, G, s);
    return BS == 16 ? dispatch_decode_ng<FMT, 128, 16>(p, B, Hkv, splits, G, s)
                    : dispatch_decode_ng<FMT, 128, 32>(p, B, Hkv, splits, G, s);
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

kvq_status kvq_cache_write(const void *k, const void *v, const int64_t *slot_mapping,
                           int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int32_t num_blocks, int32_t dtype,
                           int32_t group_size, void *k_pool, void *v_pool, float *k_scale,
                           float *v_scale, void *stream)
{
    if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0)
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
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (dtype) {
    case KVQ_INT8: return dispatch_write_d<FMT_INT8>(p, head_dim, group_size, s);
    case KVQ_FP8_E4M3: return dispatch_write_d<FMT_FP8>(p, head_dim, group_size, s);
    default: return dispatch_write_d<FMT_FP16>(p, head_dim, group_size, s);
    }
}

int32_t kvq_decode_split_tokens(int32_t num_seqs, int32_t num_kv_heads, int32_t block_size,
                                int32_t max_context_len, int32_t split_tokens)
{
    if (num_seqs < 0 || num_kv_heads <= 0 || max_context_len < 1 ||
        (block_size != 16 && block_size != 32) || !valid_split(block_size, split_tokens))
        return -1;
    return plan_span(num_seqs, num_kv_heads, block_size, max_context_len, split_tokens);
}

size_t kvq_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size,
                                 int32_t max_context_len, int32_t split_tokens)
{
    WsLayout w;
    if (!workspace_layout(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                          max_context_len, split_tokens, w))
        return SIZE_MAX;
    return w.total;
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
    kvq_status st = check_format(dtype, head_dim, block_size, group_size);
    if (st != KVQ_OK)
        return st;
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 ||
        max_blocks_per_seq <= 0)
        return KVQ_ERR_INVALID_ARG;
    if (num_q_heads % num_kv_heads != 0)
        return KVQ_ERR_INVALID_ARG;
    const int32_t r = num_q_heads / num_kv_heads;
    if (r > 16)
        return KVQ_ERR_UNSUPPORTED;
    if (num_seqs > 65535 || (int64_t)num_seqs * num_kv_heads > (1 << 24))
        return KVQ_ERR_UNSUPPORTED;
    if (num_seqs == 0)
        return KVQ_OK;
    if (max_context_len < 1 || (int64_t)max_blocks_per_seq * block_size < max_context_len)
        return KVQ_ERR_INVALID_ARG;
    if (!valid_split(block_size, split_tokens))
        return KVQ_ERR_INVALID_ARG;
    if (!(softmax_scale >= 0.0f) || std::isinf(softmax_scale))
        return KVQ_ERR_INVALID_ARG;
    if (!q || !k_pool || !v_pool || !block_tables || !context_lens || !out)
        return KVQ_ERR_INVALID_ARG;
    if (dtype != KVQ_FP16 && (!k_scale || !v_scale))
        return KVQ_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(out) || !aligned16(k_pool) || !aligned16(v_pool) ||
        (dtype == KVQ_INT8 && (!aligned16(k_scale) || !aligned16(v_scale))))
        return KVQ_ERR_INVALID_ARG;

    WsLayout w;
    if (!workspace_layout(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                          max_context_len, split_tokens, w))
        return KVQ_ERR_INVALID_ARG;
    if (w.total > 0 && (!workspace || workspace_bytes < w.total || !aligned16(workspace)))
        return KVQ_ERR_WORKSPACE;
    st = check_device();
    if (st != KVQ_OK)
        return st;

    DecodeParams p;
    p.q = static_cast<const f16 *>(q);
    p.k_pool = static_cast<const uint8_t *>(k_pool);
    p.v_pool = static_cast<const uint8_t *>(v_pool);
    p.k_scale = k_scale;
    p.v_scale = v_scale;
    p.block_tables = block_tables;
    p.context_lens = context_lens;
    p.out = static_cast<f16 *>(out);
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    p.ws_ml = w.total ? reinterpret_cast<float *>(ws + w.ml_off) : nullptr;
    p.ws_acc = w.total ? reinterpret_cast<float *>(ws + w.acc_off) : nullptr;
    p.B = num_seqs;
    p.max_blocks = max_blocks_per_seq;
    p.max_ctx = max_context_len;
    p.num_blocks = num_blocks;
    p.Hq = num_q_heads;
    p.Hkv = num_kv_heads;
    p.r = r;
    p.span = w.span;
    p.max_splits = w.max_splits;
    const float sm = softmax_scale > 0.0f ? softmax_scale : 1.0f / std::sqrt((float)head_dim);
    p.score_scale = sm * 1.4426950408889634f;  // log2(e): softmax in base 2
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (dtype) {
    case KVQ_INT8:
        return dispatch_decode<FMT_INT8>(p, num_seqs, num_kv_heads, w.max_splits, head_dim,
                                         block_size, group_size, s);
    case KVQ_FP8_E4M3:
        return dispatch_decode<FMT_FP8>(p, num_seqs, num_kv_heads, w.max_splits, head_dim,
                                        block_size, group_size, s);
    default:
        return dispatch_decode<FMT_FP16>(p, num_seqs, num_kv_heads, w.max_splits, head_dim,
                                         block_size, group_size, s);
    }
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
    if (dtype == KVQ_INT8 && (!k_scale || !v_scale))
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
    const int eb = dtype == KVQ_FP16 ? 2 : 1;
    p.block_bytes = (int64_t)num_kv_heads * block_size * head_dim * eb;
    p.scale_block_floats =
        dtype == KVQ_INT8 ? (int64_t)num_kv_heads * block_size * (head_dim / group_size) : 0;
    p.num_blocks = num_blocks;
    const unsigned chunks = (unsigned)((p.block_bytes / 16 + 255) / 256);
    hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)num_pairs, chunks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), p);
    return launch_status();
}

}  // extern "C"
