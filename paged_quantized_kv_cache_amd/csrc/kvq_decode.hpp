// kvq_decode.hpp -- paged decode attention with fused dequantization (gfx950).
//
// Computes, for one decode step ("KV Cache优化实战" s1.1: the current query
// attends over every cached K/V; s2.1: the query heads of a group share one
// KV head; s2.2: tokens live in blocks found through a block table; s4.3:
// dequantization fused into attention):
//     out[b][g] = sum_t softmax_t(sm * q[b][g] . Khat[t]) Vhat[t]
//
// Work decomposition.  One wavefront owns one (sequence b, KV head h, split)
// item: a span of `span` logical tokens (all of them when the sequence is not
// split).  It walks the span in tiles of 16 tokens (a 16-token block, or half
// of a 32-token block), gathering each tile through the block table.
//
// Both contractions run on 16x16x16 fp16 MFMA with the head_dim / token axes
// laid out so that no data moves between lanes except for softmax maxima.
// Lane (col, grp) = (lane % 16, lane / 16):
//   S^T[token][head] = K_tile (16 x D) * Q^T (D x 16)
//       A operand: token `col`, 4 head dims per k-step; B operand: q of query
//       head `col` (zero for col >= r), same dims.  Output: the scores of
//       query head `col` for the tile's tokens 4*grp .. 4*grp+3.
//   O^T[d][head] += V_tile^T (16 dims x 16 tokens) * P^T (16 tokens x 16 heads)
//       B operand = P^T, exactly the softmaxed S^T output already in the
//       lane; A operand: 4 consecutive tokens of one dim, which the V
//       micro-tile layout stores next to each other.
// The head_dim order inside an MFMA k-step is a permutation chosen so that
// each lane's K bytes are contiguous; q is loaded with the same permutation.
// Codes are converted to exact fp16 (INT8 c, or E4M3 value * 2^-8) right
// before the MFMA; K group scales multiply the per-group partial dot products
// (one accumulator per group); V group scales are folded into P (rounded to
// fp16 once) so the token sum stays a single MFMA chain.
//
// Online softmax in base 2 (the log2(e) factor rides on the score scale), with
// a rescale of the running output only when some head's maximum grows.
// Splits of one (b, h) write (m, l, acc) partials that a second, small launch
// merges with a log-sum-exp; a sequence that fits one split is finished by
// the split kernel itself.
#pragma once

#include "kvq_device.hpp"

namespace kvq {

struct DecodeParams {
    const f16 *q;
    const uint8_t *k_pool;
    const uint8_t *v_pool;
    const float *k_scale;
    const float *v_scale;
    const int32_t *block_tables;
    const int32_t *context_lens;
    f16 *out;
    float *ws_acc;    // [B][Hq][max_splits][D]
    float *ws_ml;     // [B][Hq][max_splits][2]
    int32_t B;
    int32_t max_blocks;
    int32_t max_ctx;     // host bound on context_lens (<= max_blocks * BS)
    int32_t num_blocks;
    int32_t Hq;
    int32_t Hkv;
    int32_t r;
    int32_t span;
    int32_t max_splits;
    float score_scale;  // softmax_scale * log2(e)
};

// Per-lane registers of one 16-token tile.
template <int FMT, int D>
struct TileData {
    static constexpr int EB = FMT == FMT_FP16 ? 2 : 1;
    static constexpr int NL = D * EB / 64;  // 16-byte K loads (= V loads) per lane
    uint32_t k[4 * NL];
    uint32_t v[4 * NL];
    // INT8: one scale per lane.  Row grp (lanes 16 grp .. 16 grp + 15) holds
    // the scales of the tile's tokens 4 grp .. 4 grp + 3: entry e of the row
    // is K (e < 4 NG) or V, token 4 grp + (e % 4NG) / NG, group e % NG.
    float sc;
};

// Broadcast entry `idx` of each 16-lane row to the whole row (ds_swizzle in
// bit mode: source lane = (lane & 0x10) | idx within each 32-lane half).
template <int idx>
__device__ __forceinline__ float row_bcast(float x)
{
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x10 | (idx << 5)));
}

template <int FMT, int D, int BS, int NG>
__device__ __forceinline__ void load_tile(const DecodeParams &p, TileData<FMT, D> &t,
                                          int phys, int h, int toff, int col, int grp)
{
    constexpr int EB = TileData<FMT, D>::EB;
    constexpr int NL = TileData<FMT, D>::NL;
    const int64_t tile = (int64_t)phys * p.Hkv + h;
    const uint8_t *kb = p.k_pool + tile * (BS * D * EB);
    const uint8_t *vb = p.v_pool + tile * (BS * D * EB);
    // K/V codes are read once per step: nontemporal loads keep them from
    // displacing reusable lines (block tables, scales, q) in the caches.
#pragma unroll
    for (int x = 0; x < NL; ++x) {
        // K chunk x of token toff + col: bytes [16 grp, 16 grp + 16) of its row
        const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(kb + (x * BS + toff + col) * 64 + 16 * grp));
        t.k[4 * x + 0] = w.x;
        t.k[4 * x + 1] = w.y;
        t.k[4 * x + 2] = w.z;
        t.k[4 * x + 3] = w.w;
    }
#pragma unroll
    for (int x = 0; x < NL; ++x) {
        // V micro-tile: part e, dim quad col + 16 * g4, token quad toff/4 + grp
        const int e = x % EB, g4 = x / EB;
        const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
            vb + ((((toff / 16) * EB + e) * (D / 4) + col + 16 * g4) * 4 + grp) * 16));
        t.v[4 * x + 0] = w.x;
        t.v[4 * x + 1] = w.y;
        t.v[4 * x + 2] = w.z;
        t.v[4 * x + 3] = w.w;
    }
    if constexpr (FMT == FMT_INT8) {
        const int e = col % (8 * NG);
        const float *arr = e < 4 * NG ? p.k_scale : p.v_scale;
        const int w = e % (4 * NG);
        t.sc = arr[(tile * BS + toff + 4 * grp + w / NG) * NG + w % NG];
    }
}

template <int FMT, int D, int BS, int NG>
__global__ __launch_bounds__(64) void paged_decode_kernel(DecodeParams p)
{
    constexpr int KS = D / 16;   // MFMA k-steps over head_dim
    constexpr int DT = D / 16;   // 16-dim output tiles
    constexpr int EB = TileData<FMT, D>::EB;
    constexpr int G = D / NG;    // INT8 group size
    static_assert(FMT != FMT_INT8 || G >= 64, "groups must cover a 64-dim chunk");

    // Work-item order: split index slowest, then sequence, then KV head.
    // Consecutive workgroups are dealt round-robin to the 8 XCDs, so every
    // XCD receives an equal share of each split index (the first split of
    // every sequence exists; later ones only for long sequences).
    const int units = p.B * p.Hkv;
    const int split = blockIdx.x / units;
    const int unit = blockIdx.x - split * units;
    const int b = unit / p.Hkv;
    const int h = unit - b * p.Hkv;
    const int lane = threadIdx.x;
    const int col = lane & 15;
    const int grp = lane >> 4;

    // Device lengths beyond the host bound are clamped so that no table entry
    // or workspace slot outside the caller's buffers is ever addressed.
    const int ctx = min(p.context_lens[b], p.max_ctx);
    const int t_begin = split * p.span;
    if (t_begin >= ctx)
        return;
    const int t_end = min(ctx, t_begin + p.span);
    const int nsplit = (ctx + p.span - 1) / p.span;
    const int ntiles = (t_end - t_begin + 15) >> 4;
    const bool head_ok = col < p.r;
    const int qhead = h * p.r + col;

    // ---- query operand, in the k-step dim order of the K loads:
    //   1-byte codes: k-step s, lane group grp, element v -> dim
    //       64 (s/4) + 16 grp + 4 (s%4) + v
    //   fp16:   32 (s/2) + 8 grp + 4 (s%2) + v
    f16x4 qop[KS];
    {
        const f16 *qrow = p.q + ((int64_t)b * p.Hq + (head_ok ? qhead : h * p.r)) * D;
        if constexpr (EB == 1) {
#pragma unroll
            for (int c = 0; c < D / 64; ++c) {
                const uint4 w0 = *reinterpret_cast<const uint4 *>(qrow + 64 * c + 16 * grp);
                const uint4 w1 = *reinterpret_cast<const uint4 *>(qrow + 64 * c + 16 * grp + 8);
                qop[4 * c + 0] = f16x4_from_u2(w0.x, w0.y);
                qop[4 * c + 1] = f16x4_from_u2(w0.z, w0.w);
                qop[4 * c + 2] = f16x4_from_u2(w1.x, w1.y);
                qop[4 * c + 3] = f16x4_from_u2(w1.z, w1.w);
            }
        } else {
#pragma unroll
            for (int c = 0; c < D / 32; ++c) {
                const uint4 w = *reinterpret_cast<const uint4 *>(qrow + 32 * c + 8 * grp);
                qop[2 * c + 0] = f16x4_from_u2(w.x, w.y);
                qop[2 * c + 1] = f16x4_from_u2(w.z, w.w);
            }
        }
        if (!head_ok) {
#pragma unroll
            for (int s = 0; s < KS; ++s)
                qop[s] = f16x4{0, 0, 0, 0};
        }
    }

    float score_scale = p.score_scale;
    float out_scale = 1.0f;
    if constexpr (FMT == FMT_FP8) {
        score_scale *= 256.0f * p.k_scale[h];
        out_scale = 256.0f * p.v_scale[h];
    }

    // ---- block table: the split's (at most 64) logical blocks, one per lane
    const int32_t *bt = p.block_tables + (int64_t)b * p.max_blocks;
    const int blk0 = t_begin / BS;
    const int blk_last = (t_end - 1) / BS;
    const int win = (blk0 + lane <= blk_last) ? bt[blk0 + lane] : 0;
    auto tile_phys = [&](int it) -> int {
        const int id = __builtin_amdgcn_readlane(win, (t_begin + 16 * it) / BS - blk0);
        return min(max(id, 0), p.num_blocks - 1);  // never leave the pool
    };
    auto tile_off = [&](int it) -> int { return (t_begin + 16 * it) % BS; };

    // o[tau][v]: output dim 64 (tau / 4) + 16 grp + 4 v + tau % 4, head col
    f32x4 o[DT];
#pragma unroll
    for (int i = 0; i < DT; ++i)
        o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY;
    float l = 0.0f;

    // One tile of 16 tokens starting at logical token ts, data in `cur`.
    auto process = [&](const TileData<FMT, D> &cur, const int ts) {
        // ---- this lane's scales: sk[v][j], sv[v][j] of tokens 4 grp + v
        float sk[4][NG], sv[4][NG];
        if constexpr (FMT == FMT_INT8) {
            static_for<0, 4 * NG>([&](auto I) {
                constexpr int i = decltype(I)::value;
                sk[i / NG][i % NG] = row_bcast<i>(cur.sc);
                sv[i / NG][i % NG] = row_bcast<4 * NG + i>(cur.sc);
            });
        }

        // ---- S^T = K Q^T, one accumulator per INT8 group
        f32x4 sacc[NG];
#pragma unroll
        for (int i = 0; i < NG; ++i)
            sacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            f16x4 a;
            if constexpr (FMT == FMT_INT8) {
                a = int8x4_to_f16x4(cur.k[s]);
            } else if constexpr (FMT == FMT_FP8) {
                a = fp8x4_to_f16x4_scaled(cur.k[s]);
            } else {
                a = f16x4_from_u2(cur.k[2 * s], cur.k[2 * s + 1]);
            }
            const int gi = (FMT == FMT_INT8 && NG == 2) ? (s >> 2) : 0;
            sacc[gi] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, qop[s], sacc[gi], 0, 0, 0);
        }

        // ---- scores of tokens ts + 4 grp + v for query head col (base 2)
        const int tok0 = ts + 4 * grp;
        float z[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            float acc;
            if constexpr (FMT == FMT_INT8) {
                acc = sacc[0][v] * sk[v][0];
                if constexpr (NG == 2)
                    acc += sacc[1][v] * sk[v][1];
            } else {
                acc = sacc[0][v];
            }
            z[v] = (tok0 + v < t_end) ? acc * score_scale : -INFINITY;
        }

        // ---- online softmax
        float mt = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
        mt = fmaxf(mt, __shfl_xor(mt, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        if (__builtin_amdgcn_ballot_w64(mt > m)) {
            const float mn = fmaxf(m, mt);
            const float alpha = __builtin_amdgcn_exp2f(m - mn);
            l *= alpha;
#pragma unroll
            for (int i = 0; i < DT; ++i)
                o[i] *= alpha;
            m = mn;
        }
        float pr[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            pr[v] = __builtin_amdgcn_exp2f(z[v] - m);
            l += pr[v];
        }

        // ---- P^T operands (V group scales folded in for INT8)
        f16x4 pop[NG];
        if constexpr (FMT == FMT_INT8) {
#pragma unroll
            for (int j = 0; j < NG; ++j) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    pop[j][v] = (f16)((tok0 + v < t_end) ? pr[v] * sv[v][j] : 0.0f);
                }
            }
        } else {
#pragma unroll
            for (int v = 0; v < 4; ++v)
                pop[0][v] = (f16)pr[v];
        }

        // ---- O^T += V^T P^T; d-tile tau covers dims 64 (tau/4) + 4 m + tau%4
        const bool partial = ts + 16 > t_end;
#pragma unroll
        for (int tau = 0; tau < DT; ++tau) {
            const int g4 = tau >> 2, i = tau & 3;
            f16x4 a;
            if constexpr (FMT == FMT_INT8) {
                a = int8x4_to_f16x4(cur.v[4 * g4 + i]);
            } else if constexpr (FMT == FMT_FP8) {
                a = fp8x4_to_f16x4_scaled(cur.v[4 * g4 + i]);
            } else {
                // fp16 micro-tiles hold 2 dims x 4 tokens: part i/2 of quad g4
                const int x = 2 * g4 + (i >> 1), w = 2 * (i & 1);
                a = f16x4_from_u2(cur.v[4 * x + w], cur.v[4 * x + w + 1]);
                if (partial) {  // stale fp16 slots may hold non-finite values
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        if (tok0 + v >= t_end)
                            a[v] = (f16)0.0f;
                }
            }
            const int gi = (FMT == FMT_INT8 && NG == 2) ? (64 * g4) / G : 0;
            o[tau] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, pop[gi], o[tau], 0, 0, 0);
        }
    };

    // Ping-pong over two tile buffers: the loads of tile i+1 are in flight
    // while tile i is computed.  Loads are issued unconditionally (past the
    // end they repeat the last tile) so the wait counts stay static.
    TileData<FMT, D> buf0, buf1;
    load_tile<FMT, D, BS, NG>(p, buf0, tile_phys(0), h, tile_off(0), col, grp);
    for (int it = 0; it < ntiles; it += 2) {
        const int i1 = min(it + 1, ntiles - 1);
        load_tile<FMT, D, BS, NG>(p, buf1, tile_phys(i1), h, tile_off(i1), col, grp);
        process(buf0, t_begin + 16 * it);
        const int i2 = min(it + 2, ntiles - 1);
        load_tile<FMT, D, BS, NG>(p, buf0, tile_phys(i2), h, tile_off(i2), col, grp);
        if (it + 1 < ntiles)
            process(buf1, t_begin + 16 * (it + 1));
    }

    // ---- epilogue: lane holds dims 64 g4 + 16 grp + (0..15) of head col
    float lt = l + __shfl_xor(l, 16);
    lt += __shfl_xor(lt, 32);
    if (!head_ok)
        return;
    if (nsplit == 1) {
        const float inv = out_scale / lt;
        f16 *orow = p.out + ((int64_t)b * p.Hq + qhead) * D + 16 * grp;
#pragma unroll
        for (int g4 = 0; g4 < D / 64; ++g4) {
            f16x4 hv[4];
#pragma unroll
            for (int v = 0; v < 4; ++v)
                hv[v] = f16x4{(f16)(o[4 * g4 + 0][v] * inv), (f16)(o[4 * g4 + 1][v] * inv),
                              (f16)(o[4 * g4 + 2][v] * inv), (f16)(o[4 * g4 + 3][v] * inv)};
#pragma unroll
            for (int v = 0; v < 4; ++v)
                *reinterpret_cast<f16x4 *>(orow + 64 * g4 + 4 * v) = hv[v];
        }
        return;
    }
    const int64_t idx = ((int64_t)b * p.Hq + qhead) * p.max_splits + split;
    float *wacc = p.ws_acc + idx * D + 16 * grp;
#pragma unroll
    for (int g4 = 0; g4 < D / 64; ++g4)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const f32x4 w = {o[4 * g4 + 0][v] * out_scale, o[4 * g4 + 1][v] * out_scale,
                             o[4 * g4 + 2][v] * out_scale, o[4 * g4 + 3][v] * out_scale};
            *reinterpret_cast<f32x4 *>(wacc + 64 * g4 + 4 * v) = w;
        }
    if (grp == 0)
        *reinterpret_cast<float2 *>(p.ws_ml + 2 * idx) = make_float2(m, lt);
}

// Log-sum-exp merge of the split partials of one (sequence, query head):
//   M = max_i m_i,  L = sum_i l_i 2^(m_i - M),  out = sum_i acc_i 2^(m_i - M) / L.
// Runs as its own launch after the split kernel, so the partials written by
// wavefronts on any XCD are visible without device-wide fences inside the
// split kernel.  Sequences that were not split were finished by that kernel.
template <int D>
__global__ __launch_bounds__(64) void merge_splits_kernel(DecodeParams p)
{
    const int g = blockIdx.x;
    const int b = blockIdx.y;
    const int lane = threadIdx.x;
    const int ctx = min(p.context_lens[b], p.max_ctx);
    const int nsplit = (ctx + p.span - 1) / p.span;
    if (nsplit <= 1)
        return;
    const int64_t base = ((int64_t)b * p.Hq + g) * p.max_splits;
    float mx = -INFINITY;
    for (int i = lane; i < nsplit; i += 64)
        mx = fmaxf(mx, p.ws_ml[2 * (base + i)]);
    mx = wave_max(mx);
    float ls = 0.0f;
    for (int i = lane; i < nsplit; i += 64)
        ls += p.ws_ml[2 * (base + i) + 1] * __builtin_amdgcn_exp2f(p.ws_ml[2 * (base + i)] - mx);
    ls = wave_sum(ls);
    const float inv = 1.0f / ls;
    constexpr int PER = D / 64;
    float acc[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j)
        acc[j] = 0.0f;
    for (int i = 0; i < nsplit; ++i) {
        const float w = __builtin_amdgcn_exp2f(p.ws_ml[2 * (base + i)] - mx);
        const float *a = p.ws_acc + (base + i) * D + PER * lane;
#pragma unroll
        for (int j = 0; j < PER; ++j)
            acc[j] += a[j] * w;
    }
    f16 *orow = p.out + ((int64_t)b * p.Hq + g) * D + PER * lane;
#pragma unroll
    for (int j = 0; j < PER; ++j)
        orow[j] = (f16)(acc[j] * inv);
}

}  // namespace kvq
