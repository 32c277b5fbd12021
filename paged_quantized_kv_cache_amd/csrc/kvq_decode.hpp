// kvq_decode.hpp -- paged decode attention with fused dequantization (gfx950).
//
// Computes, for one decode step ("KV Cache优化实战" s1.1: the current query
// attends over every cached K/V; s2.1: the query heads of a group share one
// KV head; s2.2: tokens live in blocks found through a block table; s4.3:
// dequantization fused into attention):
//     out[b][g] = sum_t softmax_t(sm * q[b][g] . Khat[t]) Vhat[t]
//
// Work decomposition (details at PlanRecord).  The batch's 16-token tiles,
// unit by unit ((sequence b, KV head h) units), are dealt in contiguous runs,
// one per wavefront.  A wavefront walks its run's tiles, gathering each
// through the block table (a 16-token block, or half of a 32-token block),
// with the next tile's loads in flight while the current one is computed.
//
// Both contractions run on fp16 MFMA (S^T on 16x16x32, which gfx950 issues
// at the rate of the older 16x16x16) with the head_dim / token axes laid
// out so that no data moves between lanes except for softmax maxima.
// Lane (col, grp) = (lane % 16, lane / 16):
//   S^T[token][head] = K_tile (16 x D) * Q^T (D x 16)
//       A operand: token `col`, 8 head dims per MFMA (two 4-dim k-steps);
//       B operand: q of query head `col` (zero for col >= r), same dims.
//       Output: the scores of query head `col` for the tile's tokens
//       4*grp .. 4*grp+3.
//   O^T[d][head] += V_tile^T (16 dims x 16 tokens) * P^T (16 tokens x 16 heads)
//       B operand = P^T, exactly the softmaxed S^T output already in the
//       lane, as an fp16 pair hi + lo; A operand: 4 consecutive tokens of
//       one dim (which the V micro-tile layout stores next to each other),
//       taken once against hi and once against lo (16x16x16 MFMAs).
// The head_dim order inside an MFMA k-step is a permutation chosen so that
// each lane's K bytes are contiguous; q is loaded with the same permutation.
// Codes are converted to exact fp16 (INT8 / INT4 code c, E4M3 and
// E5M2 value) right before the MFMA; K group scales multiply the per-group partial dot
// products (one accumulator per group); V group scales are folded into P
// (kept to ~2^-22 relative by the hi + lo pair) so the token sum stays a
// single MFMA chain.
//
// Online softmax in base 2 (the log2(e) factor rides on the score scale), with
// a rescale of the running output only when some head's maximum exceeds the
// reference by more than a few units (P stays below 2^slack).
// Pieces of a unit cut by run boundaries write (m, l, acc) partials that a
// second, small launch merges with a log-sum-exp; a unit that lies inside one
// run is finished by the decode kernel itself.  A run's results are stored
// only once its loads are done (see kDefer): a store among the loads would
// hold up every later wait for them.
#pragma once

#include "kvq_device.hpp"

namespace kvq {

// Work partition.  The batch is viewed as one sequence of 16-token tiles:
// units (sequence b, KV head h) in order b-major, h-minor, each unit holding
// n_b = ceil(ctx_b / 16) tiles.  A plan kernel scans the lengths and gives
// every launched wavefront one contiguous run [g0, g1) of this sequence:
//   balanced:   W runs of equal length (T / W tiles each, T = total tiles),
//               W = the number of wavefronts the GPU holds at once, so every
//               wavefront gets the same work whatever the length mix;
//   fixed span: one run per span of `span` tokens of every unit.
// A run may cover the end of one unit, whole units, and the start of
// another.  A unit finished inside one run is written out directly; a unit
// cut by run boundaries leaves (m, l, acc) partials that the boundary merge
// kernel combines.  The partition depends only on the lengths, never on
// where blocks sit in the pool.
// Block-table entries: bits 0..29 hold the physical block id; bit 30 is a
// caching hint set by the caller for blocks shared by several sequences.
constexpr int kBlockIdMask = 0x3fffffff;
// Buffer descriptor word 3 for raw (untyped) buffer loads on gfx9-class GPUs.
constexpr int kBufferConfig = 0x00020000;
constexpr int kSharedBlock = 0x40000000;
// Initial running maximum of the online softmax: finite, so that a column
// whose tokens in a piece are all masked (a short chunk's causal bound) gets
// P = 2^(-inf - kNoMax) = 0 rather than NaN, and its partial (m = kNoMax,
// l = 0, acc = 0) weighs 0 in the merge.
constexpr float kNoMax = -3.0e38f;

struct PlanRecord {
    int32_t b;     // sequence holding tile g0
    int32_t g0;    // first tile of the run
    int32_t g1;    // one past the last tile
    int32_t base;  // first tile of sequence b (Hkv * tiles before b)
    int32_t us;    // first tile of the unit holding g0
    int32_t ue;    // one past its last tile
    int32_t pad[2];
};

// Batches of at most 64 * kInlineSeqs sequences are planned inside the
// decode kernel (each wavefront scans the lengths itself); larger ones by
// plan_kernel.
constexpr int kInlineSeqs = 16;

struct DecodeParams {
    const f16 *q;
    const uint8_t *k_pool;
    const uint8_t *v_pool;
    const float *k_scale;
    const float *v_scale;
    const int32_t *block_tables;
    const int32_t *context_lens;
    f16 *out;
    PlanRecord *plan_rec;        // [W] (written here when planned inline)
    int32_t *plan_meta;          // [0] = runs in use
    int32_t inline_plan;         // 1: plan inside the decode kernel
    float *ws_acc;               // [W][2 slots][r][D]
    float *ws_ml;                // [W][2 slots][r][2]
    int32_t B;
    int32_t max_blocks;
    int32_t max_ctx;     // host bound on context_lens (<= max_blocks * BS)
    int32_t num_blocks;
    int32_t Hq;
    int32_t Hkv;
    int32_t r;
    int32_t cols;        // MFMA columns per unit (partials, merge): r, or chunk x r
    int32_t W;           // wavefronts launched
    float score_scale;   // softmax_scale * log2(e)
    // KV-head subset (per-head mixed precision): the pool's head h is KV
    // head head_ids[h] of the model; q / out rows have Hq query heads, of
    // which KV head g serves g * r .. g * r + r - 1.  Null: the identity.
    const int32_t *head_ids;
    // chunks: [B + 1] offsets in q / out (chunked prefill, and short chunks
    // walked by the decode partition); null for decode
    const int32_t *q_start;
    // [B] table row of each (virtual) sequence when the chunks of longer
    // prompts are cut into virtual sequences; null: row b is sequence b
    const int32_t *seq_row;
    int32_t groups;          // chunked prefill: query blocks per (sequence, KV head)
};

struct PlanParams {
    const int32_t *context_lens;
    int32_t *S;
    PlanRecord *rec;
    int32_t *meta;
    int32_t B;
    int32_t Hkv;
    int32_t max_ctx;
    int32_t W;            // balanced: runs wanted; fixed span: runs launched
    int32_t span_tiles;   // 0: balanced; else tiles per span
};

// Wavefront priority from the share of its run still ahead: 3 while more
// than half is left, then 2, 1, and 0 for the last eighth.  Without it the
// SIMD's arbiter favours its oldest wavefront: of the three wavefronts on a
// SIMD, the first finishes an equal run ~1.4x sooner than the third, and the
// launch ends with few wavefronts left.  With the priority falling as a run
// progresses, the wavefronts that are behind issue first and the runs of a
// SIMD end closer together.
__device__ __forceinline__ void set_run_priority(int left, int len)
{
    if (2 * left > len)
        __builtin_amdgcn_s_setprio(3);
    else if (4 * left > len)
        __builtin_amdgcn_s_setprio(2);
    else if (8 * left > len)
        __builtin_amdgcn_s_setprio(1);
    else
        __builtin_amdgcn_s_setprio(0);
}

__device__ __forceinline__ int model_head(const DecodeParams &p, int h)
{
    return p.head_ids ? p.head_ids[h] : h;
}

__device__ __forceinline__ int ctx_tiles(const int32_t *lens, int b, int max_ctx)
{
    const int ctx = min(max(lens[b], 0), max_ctx);
    return (ctx + 15) >> 4;
}

constexpr int kPlanThreads = 1024;
constexpr int kPlanLdsSeqs = 8192;  // sequences whose tile prefix fits in LDS

// One workgroup: exclusive scan of the tile counts, then the run records.
__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanParams p)
{
    __shared__ int32_t sc_t[kPlanThreads];
    __shared__ int32_t sc_i[kPlanThreads];
    __shared__ int32_t s_S[kPlanLdsSeqs + 1];
    const int tid = threadIdx.x;
    const int per = (p.B + kPlanThreads - 1) / kPlanThreads;
    const int b0 = min(p.B, tid * per), b1 = min(p.B, b0 + per);
    int st = 0, si = 0;
    for (int b = b0; b < b1; ++b) {
        const int n = ctx_tiles(p.context_lens, b, p.max_ctx);
        st += n;
        if (p.span_tiles)
            si += (n + p.span_tiles - 1) / p.span_tiles;
    }
    sc_t[tid] = st;
    sc_i[tid] = si;
    __syncthreads();
    for (int o = 1; o < kPlanThreads; o <<= 1) {  // inclusive scans
        const int at = tid >= o ? sc_t[tid - o] : 0;
        const int ai = tid >= o ? sc_i[tid - o] : 0;
        __syncthreads();
        sc_t[tid] += at;
        sc_i[tid] += ai;
        __syncthreads();
    }
    const int tot_t = sc_t[kPlanThreads - 1];
    const int tot_i = sc_i[kPlanThreads - 1];
    const int T = p.Hkv * tot_t;
    const int W = p.span_tiles ? p.Hkv * tot_i : min(p.W, T);
    const bool lds = p.B <= kPlanLdsSeqs;
    int off_t = sc_t[tid] - st, off_i = sc_i[tid] - si;
    for (int b = b0; b < b1; ++b) {
        const int n = ctx_tiles(p.context_lens, b, p.max_ctx);
        p.S[b] = off_t;
        if (lds)
            s_S[b] = off_t;
        if (p.span_tiles) {
            const int lo = p.Hkv * off_t;
            const int m = (n + p.span_tiles - 1) / p.span_tiles;
            for (int h = 0; h < p.Hkv; ++h)
                for (int k = 0; k < m; ++k) {
                    const int g0 = lo + h * n + k * p.span_tiles;
                    p.rec[p.Hkv * off_i + h * m + k] =
                        PlanRecord{b, g0, min(lo + (h + 1) * n, g0 + p.span_tiles), lo,
                                   lo + h * n, lo + (h + 1) * n, {0, 0}};
                }
            off_i += m;
        }
        off_t += n;
    }
    if (tid == kPlanThreads - 1) {
        p.S[p.B] = tot_t;
        if (lds)
            s_S[p.B] = tot_t;
        p.meta[0] = W;
    }
    if (p.span_tiles || T == 0)
        return;
    __syncthreads();
    __threadfence_block();
    // balanced runs: run w = [w T / W, (w + 1) T / W); its sequence is the
    // last b with Hkv * S[b] <= g0 (binary search over the prefix)
    const int32_t *S = lds ? s_S : p.S;
    for (int w = tid; w < W; w += kPlanThreads) {
        const int g0 = (int)((int64_t)w * T / W);
        const int g1 = (int)((int64_t)(w + 1) * T / W);
        int lo = 0, hi = p.B;  // invariant: Hkv * S[lo] <= g0 < Hkv * S[hi + 1]
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (p.Hkv * S[mid] <= g0)
                lo = mid;
            else
                hi = mid - 1;
        }
        const int base = p.Hkv * S[lo];
        const int n = S[lo + 1] - S[lo];  // > 0: tile g0 lies in sequence lo
        const int us = base + (g0 - base) / n * n;
        p.rec[w] = PlanRecord{lo, g0, g1, base, us, us + n, {0, 0}};
    }
}

// Virtual sequences for chunks longer than one wavefront's columns: chunk
// j of sequence b (tokens [j qpg, (j + 1) qpg) of its chunk, qpg = 32 / r)
// becomes virtual sequence v = b J + j, whose context ends at its last chunk
// token (so the causal bounds come out as for the whole chunk) and whose
// chunk is those qpg tokens; chunks past the end of b's are empty (context
// 0, no tiles).  The decode partition then runs over the B J virtual
// sequences with seq_row[v] = b choosing the block-table row.
struct VirtualParams {
    const int32_t *q_start;       // [B + 1]
    const int32_t *context_lens;  // [B]
    int32_t *vctx;                // [B J]
    int32_t *vrow;                // [B J]
    int32_t *vqs;                 // [B J + 1]
    int32_t B;
    int32_t J;
    int32_t qpg;
    int32_t max_ctx;
};

__global__ __launch_bounds__(256) void virtual_chunks_kernel(VirtualParams p)
{
    const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t nv = (int64_t)p.B * p.J;
    if (v > nv)
        return;
    if (v == nv) {
        p.vqs[v] = p.q_start[p.B];
        return;
    }
    const int b = (int)(v / p.J), j = (int)(v % p.J);
    const int ctx = min(max(p.context_lens[b], 0), p.max_ctx);
    const int qs = p.q_start[b];
    const int nb = max(min(p.q_start[b + 1] - qs, ctx), 0);
    const int lo = j * p.qpg;
    p.vrow[v] = b;
    if (lo < nb) {
        p.vctx[v] = ctx - nb + min(lo + p.qpg, nb);
        p.vqs[v] = qs + lo;
    } else {
        p.vctx[v] = 0;
        p.vqs[v] = qs + nb;
    }
}

// Per-lane registers of one 16-token tile.
template <int FMT, int D>
struct TileData {
    static constexpr int EB = FMT == FMT_FP16 ? 2 : 1;  // INT4: q / output dim order as 1 byte
    static constexpr int TB = FMT == FMT_INT4 ? D / 2 : D * EB;  // tile bytes per token
    static constexpr int NL = TB / 64;      // 16-byte K loads (= V loads) per lane
    uint32_t k[4 * NL];
    uint32_t v[4 * NL];
    // INT8: one scale per lane.  Row grp (lanes 16 grp .. 16 grp + 15) holds
    // the scales of the tile's tokens 4 grp .. 4 grp + 3: entry e of the row
    // is K (e < 4 NG) or V, token 4 grp + (e % 4NG) / NG, group e % NG.
    float sc;
};

// Broadcast entry `idx` of each 16-lane row to the whole row (ds_swizzle in
// bit mode: source lane = (lane & 0x10) | idx within each 32-lane half).  It
// runs on the LDS pipe; a DPP row_newbcast move, one VALU instruction, was
// measured 4-6 % slower on INT4 (whose tiles leave the VALU the busier unit)
// and no faster elsewhere.
template <int idx>
__device__ __forceinline__ float row_bcast(float x)
{
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x10 | (idx << 5)));
}

template <int FMT, int D, int BS, int NG, bool kNT>
__device__ __forceinline__ void load_codes(const DecodeParams &p, TileData<FMT, D> &t,
                                           const uint8_t *kb, const uint8_t *vb, int toff,
                                           int col, int grp)
{
    constexpr int EB = TileData<FMT, D>::EB;
    constexpr int TB = TileData<FMT, D>::TB;
    constexpr int NL = TileData<FMT, D>::NL;
    // Buffer loads on a descriptor spanning one tile: the cache policy is an
    // immediate of each load (nt = bit 1 of the aux field on gfx950), and
    // offsets past the tile read zeros instead of faulting.
    constexpr int kAux = kNT ? 2 : 0;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(kb), 0, BS * TB, kBufferConfig);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(vb), 0, BS * TB, kBufferConfig);
#pragma unroll
    for (int x = 0; x < NL; ++x) {
        // K chunk x of token toff + col: bytes [16 grp, 16 grp + 16) of its row
        const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(
            rk, (x * BS + toff + col) * 64 + 16 * grp, 0, kAux);
        t.k[4 * x + 0] = w.x;
        t.k[4 * x + 1] = w.y;
        t.k[4 * x + 2] = w.z;
        t.k[4 * x + 3] = w.w;
    }
#pragma unroll
    for (int x = 0; x < NL; ++x) {
        // V micro-tile: part e, dim quad col + 16 * g4, token quad toff/4 + grp
        const int e = x % EB, g4 = x / EB;
        // INT4: one 16-byte slice per lane, dim quad col x token quad grp
        const int voff = FMT == FMT_INT4
                             ? ((toff / 16) * 64 + col * 4 + grp) * 16
                             : ((((toff / 16) * EB + e) * (D / 4) + col + 16 * g4) * 4 + grp) * 16;
        const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(rv, voff, 0, kAux);
        t.v[4 * x + 0] = w.x;
        t.v[4 * x + 1] = w.y;
        t.v[4 * x + 2] = w.z;
        t.v[4 * x + 3] = w.w;
    }
}

// Loads one 16-token tile.  kNT selects nontemporal loads (see the window
// walk in the decode kernel for when).
template <int FMT, int D, int BS, int NG, bool kNT>
__device__ __forceinline__ void load_tile(const DecodeParams &p, TileData<FMT, D> &t,
                                          int phys, int h, int toff, int col, int grp)
{
    constexpr int TB = TileData<FMT, D>::TB;
    const int64_t tile = (int64_t)phys * p.Hkv + h;
    const uint8_t *kb = p.k_pool + tile * (BS * TB);
    const uint8_t *vb = p.v_pool + tile * (BS * TB);
    load_codes<FMT, D, BS, NG, kNT>(p, t, kb, vb, toff, col, grp);
    if constexpr (NG > 0) {  // per-group scales
        const int e = col % (8 * NG);
        const float *arr = e < 4 * NG ? p.k_scale : p.v_scale;
        const int w = e % (4 * NG);
        t.sc = arr[(tile * BS + toff + 4 * grp + w / NG) * NG + w % NG];
    }
}

// Query columns of one MFMA column group: this lane's query row (active) or
// a harmless row (inactive: q is zeroed, nothing is written), its output
// row, and the column's token bound (causal limit in prefill).
struct Cols {
    const f16 *qrow;
    f16 *orow;
    int tcol;
    bool active;
};

// kDecodeGroups: MFMA column groups per wavefront in the decode walk (2 for
// short chunks of more than 16 columns: chunk tokens x query heads).
// The INT4 decode instance runs four wavefronts per SIMD (its tiles carry
// half the bytes, so more of them must be in flight), which needs it to fit
// in 128 VGPRs (with 32-token blocks that would spill; it runs three).
template <int FMT, int D, int BS, int NG, int kDecodeGroups = 1>
__global__ __launch_bounds__(64, (FMT == FMT_INT4 && BS == 16 && kDecodeGroups == 1) ? 4 : 1)
void paged_decode_kernel(DecodeParams p)
{
    constexpr int KS = D / 16;   // MFMA k-steps over head_dim
    constexpr int DT = D / 16;   // 16-dim output tiles
    constexpr int EB = TileData<FMT, D>::EB;
    // Scales: NG > 0 -- one per (token, group of G dims) in arrays beside
    // the pools (INT8 or E4M3); NG == 0 -- static: one per KV head (FP8),
    // one per (KV head, channel) (INT8), none (fp16).
    constexpr bool kGroup = NG > 0;
    constexpr int NA = kGroup ? NG : 1;        // score accumulators per tile
    constexpr int NQ = kDecodeGroups;          // column groups per wavefront
    constexpr int G = kGroup ? D / NG : D;     // group size
    constexpr bool kChannel = FMT == FMT_INT8 && !kGroup;
    static_assert(FMT != FMT_INT4 || (D == 128 && kGroup), "INT4: head_dim 128, group scales");
    // PV precision.  P enters the PV MFMA as fp16, rounded with relative
    // error <= 2^-11, so a single fp16 P moves an output by up to 2^-11 times
    // the largest |V| the softmax weighs (the weights sum to 1): inside an
    // absolute 2e-3 only while |V| <= 4.  Outlier channels in V reach ~30.
    // P is therefore split into hi = fp16(P) and lo = fp16(P - hi), which
    // leaves ~2^-22 relative; the codes meet hi and lo in two 16x16x16
    // MFMAs per d-tile (one column group) or in one 16x16x32 MFMA that holds
    // them twice (two column groups).
    static_assert(!kGroup || G >= 64, "groups must cover a 64-dim chunk");

    // Vector memory operations complete in issue order, so a store issued
    // between a run's tile loads holds up every later wait for those loads
    // until the store is done (microseconds with HBM busy).  With one column
    // group the results of a piece therefore wait in registers while the
    // run continues, up to two pieces' (a third piece stores the oldest),
    // and are stored once the run's last piece is done; a run of up to three
    // pieces then stores nothing before its last load, and the inline
    // plan's record for the merge launch is stored after the walk too.
    // (Two column groups, or INT4's four wavefronts per SIMD, have no
    // registers to spare; they store as they go.)
    constexpr bool kDefer = NQ == 1 && FMT != FMT_INT4;

    // run index: workgroups go round-robin to the 8 XCDs (w to XCD w % 8);
    // XCD x takes the runs x G / 8 .. (x + 1) G / 8 - 1, so the heads of a
    // sequence (consecutive runs) share an XCD and start together
    const int G8 = gridDim.x;
    const int w = (G8 & 7) == 0 ? (int)(blockIdx.x & 7) * (G8 >> 3) + (int)(blockIdx.x >> 3)
                                : (int)blockIdx.x;
    const int lane = threadIdx.x;
    const int col = lane & 15;
    const int grp = lane >> 4;
    PlanRecord rec{};
    // this wavefront's run of tiles
    if (p.inline_plan) {
        // every wavefront scans the lengths: lane i holds sequences
        // per*i .. per*i + per - 1
        const int per = (p.B + 63) >> 6;
        int tl[kInlineSeqs];
        int sum = 0;
#pragma unroll
        for (int j = 0; j < kInlineSeqs; ++j) {
            const int bb = lane * per + j;
            tl[j] = (j < per && bb < p.B) ? ctx_tiles(p.context_lens, bb, p.max_ctx) : 0;
            sum += tl[j];
        }
        int incl = sum;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(incl, o);
            if (lane >= o)
                incl += y;
        }
        // (readfirstlane: the values are wave-uniform; keep them scalar)
        const int T = p.Hkv * __builtin_amdgcn_readfirstlane(__shfl(incl, 63));
        const int W = min(p.W, T);
        if (w == 0 && lane == 0)
            p.plan_meta[0] = W;  // runs in use, for the merge launch
        if (w >= W)
            return;
        const int g0 = (int)((int64_t)w * T / W);
        const int g1 = (int)((int64_t)(w + 1) * T / W);
        int s0 = incl - sum, found = -1, fbase = 0, fn = 1;
#pragma unroll
        for (int j = 0; j < kInlineSeqs; ++j) {
            if (p.Hkv * s0 <= g0 && g0 < p.Hkv * (s0 + tl[j])) {
                found = lane * per + j;
                fbase = p.Hkv * s0;
                fn = tl[j];
            }
            s0 += tl[j];
        }
        const int src = __builtin_ctzll(__builtin_amdgcn_ballot_w64(found >= 0));
        const int base = __builtin_amdgcn_readlane(fbase, src);
        const int n0 = __builtin_amdgcn_readlane(fn, src);
        const int us = base + (g0 - base) / n0 * n0;
        rec = PlanRecord{__builtin_amdgcn_readlane(found, src), g0, g1, base, us, us + n0,
                         {0, 0}};
        if constexpr (!kDefer) {
            if (lane == 0)
                p.plan_rec[w] = rec;  // for the merge launch
        }
    } else {
        if (w >= p.plan_meta[0])
            return;
        rec = p.plan_rec[w];
    }

    float score_scale0 = p.score_scale;

    // decode: tiles of the run, and those after the piece being walked
    int run_len = 0, run_after = 0;

    // Attend over tiles [t0, t1) of unit (b, h); ctx clamped to the host
    // bound.  cg[q]: the columns of group q (see Cols); every loaded tile
    // serves all NQ groups.
    // A piece's results: the final fp16 output of a whole unit (kind 1) or
    // the fp32 partial (out_scale-scaled acc, then (m, l)) of a cut one
    // (kind 2) in its workspace slot.
    auto emit = [&](const f32x4 (&oq)[DT], const float mq, const float lq, const float osc,
                    const int kind, f16 *orow, const int64_t idx) {
        if (kind == 1) {
            const float inv = osc / lq;
            orow += 16 * grp;
#pragma unroll
            for (int g4 = 0; g4 < D / 64; ++g4) {
                f16x4 hv[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const f32x4 *t = &oq[4 * g4];
                    hv[v] = f16x4{(f16)(t[0][v] * inv), (f16)(t[1][v] * inv),
                                  (f16)(t[2][v] * inv), (f16)(t[3][v] * inv)};
                }
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    *reinterpret_cast<f16x4 *>(orow + 64 * g4 + 4 * v) = hv[v];
            }
        } else if (kind == 2) {
            float *wacc = p.ws_acc + idx * D + 16 * grp;
#pragma unroll
            for (int g4 = 0; g4 < D / 64; ++g4)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const f32x4 *t = &oq[4 * g4];
                    const f32x4 wv = {t[0][v] * osc, t[1][v] * osc, t[2][v] * osc, t[3][v] * osc};
                    *reinterpret_cast<f32x4 *>(wacc + 64 * g4 + 4 * v) = wv;
                }
            if (grp == 0)
                *reinterpret_cast<float2 *>(p.ws_ml + 2 * idx) = make_float2(mq, lq);
        }
    };
    constexpr int kHeld = kDefer ? 2 : 1;   // pieces whose results can wait
    struct Held {
        f32x4 o[DT];
        float m, l, s;
        int kind;       // 0: nothing held
        f16 *orow;
        int64_t idx;
    };
    Held held[kHeld];
#pragma unroll
    for (int i = 0; i < kHeld; ++i)
        held[i].kind = 0;
    auto emit_held = [&](const Held &x) {
        if (x.kind != 0)
            emit(x.o, x.m, x.l, x.s, x.kind, x.orow, x.idx);
    };

    auto attend = [&](const int b, const int h, const int ctx, const int n, const int t0,
                      const int t1, const Cols (&cg)[NQ], const bool last) {
        const int t_end = min(ctx, 16 * t1);  // token bound of this run (data)
        int t_col[NQ];                        // score bound of this lane's columns
#pragma unroll
        for (int q = 0; q < NQ; ++q)
            t_col[q] = min(t_end, cg[q].tcol);

        // ---- query operand, in the k-step dim order of the K loads:
        //   1-byte codes: k-step s, lane group grp, element v -> dim
        //       64 (s/4) + 16 grp + 4 (s%4) + v
        //   fp16:   32 (s/2) + 8 grp + 4 (s%2) + v
        f16x4 qop[NQ][KS];
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const f16 *qrow = cg[q].qrow;
            if constexpr (EB == 1) {
#pragma unroll
                for (int c = 0; c < D / 64; ++c) {
                    const uint4 w0 = *reinterpret_cast<const uint4 *>(qrow + 64 * c + 16 * grp);
                    const uint4 w1 = *reinterpret_cast<const uint4 *>(qrow + 64 * c + 16 * grp + 8);
                    qop[q][4 * c + 0] = f16x4_from_u2(w0.x, w0.y);
                    qop[q][4 * c + 1] = f16x4_from_u2(w0.z, w0.w);
                    qop[q][4 * c + 2] = f16x4_from_u2(w1.x, w1.y);
                    qop[q][4 * c + 3] = f16x4_from_u2(w1.z, w1.w);
                }
            } else {
#pragma unroll
                for (int c = 0; c < D / 32; ++c) {
                    const uint4 w4 = *reinterpret_cast<const uint4 *>(qrow + 32 * c + 8 * grp);
                    qop[q][2 * c + 0] = f16x4_from_u2(w4.x, w4.y);
                    qop[q][2 * c + 1] = f16x4_from_u2(w4.z, w4.w);
                }
            }
            if (!cg[q].active) {
#pragma unroll
                for (int s = 0; s < KS; ++s)
                    qop[q][s] = f16x4{0, 0, 0, 0};
            }
        }
        // INT8 per channel: K's channel scales ride on q, q' = q * s_d, as an
        // fp16 pair hi + lo (hi = fp16(q'), lo = fp16(q' - hi)) so the dot
        // products keep ~22 bits of q'; both halves go through the MFMA.
        f16x4 qlo[NQ][kChannel ? KS : 1];
        if constexpr (kChannel) {
            const float *srow = p.k_scale + (int64_t)h * D;
#pragma unroll
            for (int c = 0; c < D / 64; ++c) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {  // dims 64 c + 16 grp + 4 u + (0..3)
                    const float4 sc4 = *reinterpret_cast<const float4 *>(srow + 64 * c + 16 * grp + 4 * u);
                    const float scv[4] = {sc4.x, sc4.y, sc4.z, sc4.w};
#pragma unroll
                    for (int q = 0; q < NQ; ++q) {
                        f16x4 &hi = qop[q][4 * c + u];
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const float qs = (float)hi[v] * scv[v];
                            const f16 h16 = (f16)qs;
                            hi[v] = h16;
                            qlo[q][4 * c + u][v] = (f16)(qs - (float)h16);
                        }
                    }
                }
            }
        }
        float score_scale = score_scale0;
        float out_scale = 1.0f;
        if constexpr ((FMT == FMT_FP8 || FMT == FMT_E5M2) && !kGroup) {
            score_scale *= p.k_scale[h];
            out_scale = p.v_scale[h];
        }
        // Per-group scales: this lane's scale entry (see TileData) is token
        // lane_tok of the tile; K entries carry the score scale, so the
        // scores need no further multiply.  Entries of tokens past t_end
        // become 0.
        float lane_fac = 1.0f;
        int lane_tok = 0;
        if constexpr (kGroup) {
            const int e = col % (8 * NG);
            lane_fac = e < 4 * NG ? score_scale : 1.0f;
            lane_tok = 4 * grp + (e % (4 * NG)) / NG;
        }
        // o[q][tau][v]: output dim 64 (tau / 4) + 16 grp + 4 v + tau % 4 of
        // column col of group q; m, l likewise per group
        f32x4 o[NQ][DT];
        float m[NQ], l[NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
#pragma unroll
            for (int i = 0; i < DT; ++i)
                o[q][i] = f32x4{0.f, 0.f, 0.f, 0.f};
            m[q] = kNoMax;
            l[q] = 0.0f;
        }

        // One tile of 16 tokens starting at logical token ts, data in `cur`.
        auto process = [&](const TileData<FMT, D> &cur, const int ts) {
            // ---- this lane's scales: sk[v][j], sv[v][j] of tokens 4 grp + v
            float sk[4][NA], sv[4][NA];
            if constexpr (kGroup) {
                const float sc = ts + lane_tok < t_end ? cur.sc * lane_fac : 0.0f;
                static_for<0, 4 * NG>([&](auto I) {
                    constexpr int i = decltype(I)::value;
                    sk[i / NG][i % NG] = row_bcast<i>(sc);
                    sv[i / NG][i % NG] = row_bcast<4 * NG + i>(sc);
                });
            }
            // ---- S^T = K Q^T, one accumulator per scale group (and column group)
            f32x4 sacc[NQ][NA];
#pragma unroll
            for (int q = 0; q < NQ; ++q)
#pragma unroll
                for (int i = 0; i < NA; ++i)
                    sacc[q][i] = f32x4{0.f, 0.f, 0.f, 0.f};
            // K operand of k-step s (4 head dims per lane, see the q order)
            auto kop = [&](int s) -> f16x4 {
                if constexpr (FMT == FMT_INT8)
                    return int8x4_to_f16x4(cur.k[s]);
                else if constexpr (FMT == FMT_FP8)
                    return fp8x4_to_f16x4(cur.k[s]);
                else if constexpr (FMT == FMT_E5M2)
                    return e5m2x4_to_f16x4(cur.k[s]);
                else
                    return f16x4_from_u2(cur.k[2 * s], cur.k[2 * s + 1]);
            };
            // two k-steps per 16x16x32 MFMA; both lie in one scale group
#pragma unroll
            for (int s2 = 0; s2 < KS / 2; ++s2) {
                f16x8 a;
                if constexpr (FMT == FMT_INT4) {  // a dword holds k-steps 2 s2, 2 s2 + 1
                    f16x4 lo, hi;
                    int4x8_to_f16x4(cur.k[s2], lo, hi);
                    a = cat8(lo, hi);
                } else {
                    a = cat8(kop(2 * s2), kop(2 * s2 + 1));
                }
                const int gi = NA == 2 ? (s2 >> 1) : 0;
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    sacc[q][gi] =
                        mfma32(a, cat8(qop[q][2 * s2], qop[q][2 * s2 + 1]), sacc[q][gi]);
                    if constexpr (kChannel)
                        sacc[q][0] =
                            mfma32(a, cat8(qlo[q][2 * s2], qlo[q][2 * s2 + 1]), sacc[q][0]);
                }
            }
            // ---- scores of tokens ts + 4 grp + v for query head col (base 2)
            const int tok0 = ts + 4 * grp;
            f16x4 pop[NQ][NA], plo[NQ][NA];
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                float z[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    float acc;
                    if constexpr (kGroup) {
                        acc = sacc[q][0][v] * sk[v][0];
                        if constexpr (NA == 2)
                            acc += sacc[q][1][v] * sk[v][1];
                    } else {
                        acc = sacc[q][0][v] * score_scale;
                    }
                    z[v] = tok0 + v < t_col[q] ? acc : -INFINITY;
                }
                // ---- online softmax, with a lazy rescale: the reference m
                // moves only when a score exceeds it by more than kSlack (base
                // 2), so P < 2^kSlack.  The P^T operands (P times a V group
                // scale) stay finite in fp16 for any fp16 input: a group scale
                // is at most 65504 / 127 (INT8), / 448 (E4M3) or / 7 (INT4).
                constexpr float kSlack = !kGroup ? 8.0f
                                       : FMT == FMT_INT8 || FMT == FMT_FP8 ? 6.0f
                                       : FMT == FMT_INT4 ? 2.0f : 0.0f;
                float mt = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
                mt = fmaxf(mt, __shfl_xor(mt, 16));
                mt = fmaxf(mt, __shfl_xor(mt, 32));
                if (__builtin_amdgcn_ballot_w64(mt > m[q] + kSlack)) {
                    const float mn = fmaxf(m[q], mt);
                    const float alpha = __builtin_amdgcn_exp2f(m[q] - mn);
                    l[q] *= alpha;
#pragma unroll
                    for (int i = 0; i < DT; ++i)
                        o[q][i] *= alpha;
                    m[q] = mn;
                }
                float pr[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    pr[v] = __builtin_amdgcn_exp2f(z[v] - m[q]);
                    l[q] += pr[v];
                }
                // ---- P^T operands (V group scales folded in; masked tokens
                // have pr = 0 and a zeroed scale): P split into fp16 hi + lo
#pragma unroll
                for (int j = 0; j < NA; ++j) {
                    f16x2 h[2], lo[2];
#pragma unroll
                    for (int v = 0; v < 4; v += 2)
                        split_f16x2(kGroup ? pr[v] * sv[v][j] : pr[v],
                                    kGroup ? pr[v + 1] * sv[v + 1][j] : pr[v + 1], h[v / 2], lo[v / 2]);
                    pop[q][j] = f16x4{h[0].x, h[0].y, h[1].x, h[1].y};
                    plo[q][j] = f16x4{lo[0].x, lo[0].y, lo[1].x, lo[1].y};
                }
            }
            // ---- O^T += V^T P^T; d-tile tau covers dims 64 (tau/4) + 4 m + tau%4
            // fp16: stale slots past t_end may hold non-finite values, which
            // a zero P entry does not cancel; the lane's V dwords hold tokens
            // (0, 1) or (2, 3) of its quad and are masked per token.
            // E5M2 and E4M3 likewise: their conversions are exact, so stale
            // NaN / inf codes survive them; a V dword holds tokens 0..3 of
            // the quad, one byte each.
            uint32_t vmask01 = ~0u, vmask23 = ~0u, vmask8 = ~0u;
            if constexpr (FMT == FMT_FP16) {
                const int nv = t_end - tok0;  // valid tokens of this lane's quad (if < 4)
                vmask01 = nv >= 2 ? ~0u : (nv == 1 ? 0xffffu : 0u);
                vmask23 = nv >= 4 ? ~0u : (nv == 3 ? 0xffffu : 0u);
            } else if constexpr (FMT == FMT_E5M2 || FMT == FMT_FP8) {
                const int nv = t_end - tok0;
                vmask8 = nv >= 4 ? ~0u : (nv <= 0 ? 0u : (1u << (8 * nv)) - 1u);
            }
            // per d-tile, one column group: two 16x16x16 MFMAs, the codes
            // against hi, then against lo (a 16x16x32 one would need the
            // codes copied into both halves of its operand: 16 register moves
            // per tile, which cost more VALU time than the second MFMA costs
            // matrix time); two column groups: one 16x16x32 MFMA per group,
            // the codes twice, against hi and lo (there the matrix core is
            // the busier unit)
#pragma unroll
            for (int tau = 0; tau < DT; ++tau) {
                const int g4 = tau >> 2, i = tau & 3;
                f16x4 a;
                if constexpr (FMT == FMT_INT4) {  // a dword holds dims 4 col + i, i = 2x, 2x + 1
                    f16x4 lo, hi;
                    int4x8_to_f16x4(cur.v[2 * g4 + (i >> 1)], lo, hi);
                    a = (i & 1) ? hi : lo;
                } else if constexpr (FMT == FMT_INT8) {
                    a = int8x4_to_f16x4(cur.v[4 * g4 + i]);
                } else if constexpr (FMT == FMT_FP8) {
                    a = fp8x4_to_f16x4(cur.v[4 * g4 + i] & vmask8);
                } else if constexpr (FMT == FMT_E5M2) {
                    a = e5m2x4_to_f16x4(cur.v[4 * g4 + i] & vmask8);
                } else {
                    // fp16 micro-tiles hold 2 dims x 4 tokens: part i/2 of quad g4
                    const int x = 2 * g4 + (i >> 1), wd = 2 * (i & 1);
                    a = f16x4_from_u2(cur.v[4 * x + wd] & vmask01, cur.v[4 * x + wd + 1] & vmask23);
                }
                const int gi = NA == 2 ? (64 * g4) / G : 0;
                if constexpr (NQ == 1) {
                    o[0][tau] = mfma16(a, pop[0][gi], o[0][tau]);
                    o[0][tau] = mfma16(a, plo[0][gi], o[0][tau]);
                } else {
#pragma unroll
                    for (int q = 0; q < NQ; ++q)
                        o[q][tau] = mfma32(cat8(a, a), cat8(pop[q][gi], plo[q][gi]), o[q][tau]);
                }
            }
        };

        // ---- walk tiles [t0, t1) with two tile buffers: tile i+1's loads
        // are in flight while tile i is computed.  Loads are issued
        // unconditionally (past t1 they repeat the last tile), so the wait
        // before a tile's compute leaves the next tile's loads in flight.
        //
        // Block ids come from 64-entry windows of the table row (one entry
        // per lane, read with readlane), aligned to 64-block boundaries of
        // the sequence.  Three window registers rotate: the current window,
        // the next one (read by the loads that run ahead), and the one after,
        // whose load is issued a whole window before it is needed, so the
        // walk never waits on the table.
        //
        // Cache policy, one per piece (a per-tile choice would put the loads
        // under a branch, and the wait would then have to cover every load
        // issued): codes of private blocks are read once per step, so they
        // use nontemporal loads, which do not displace reusable lines; blocks
        // the caller marks as shared are read by several sequences in the
        // same step and use ordinary loads, so that later readers hit in L2 /
        // the last-level cache.  Shared blocks are normally a prefix of the
        // sequence: the leading windows (among the three first loaded) that
        // hold a shared block are walked with ordinary loads, the rest with
        // nontemporal ones.
        const int32_t *bt =
            p.block_tables + (int64_t)(p.seq_row ? p.seq_row[b] : b) * p.max_blocks;
        constexpr int TPB = BS / 16;                // tiles per block
        const int blk_last = (16 * t1 - 1) / BS;    // last block of the piece
        // (entries past the piece repeat its last block: never used, and the
        // load stays unconditional so no wait is needed until a use)
        auto load_win = [&](int wi) -> int { return bt[min(64 * wi + lane, blk_last)]; };
        int wi = t0 / (64 * TPB);   // window of the tile being processed
        int win_a = load_win(wi), win_b = load_win(wi + 1), win_c = load_win(wi + 2);
        auto ld = [&](TileData<FMT, D> &buf, int i, auto nt_tag) {
            const int blk = i / TPB;
            const int ea = __builtin_amdgcn_readlane(win_a, blk % 64);
            const int eb = __builtin_amdgcn_readlane(win_b, blk % 64);
            const int e = blk / 64 == wi ? ea : eb;
            const int id = min(max(e & kBlockIdMask, 0), p.num_blocks - 1);  // stay in the pool
            load_tile<FMT, D, BS, NG, decltype(nt_tag)::value>(p, buf, id, h, (16 * i) % BS, col,
                                                              grp);
        };
        // walk tiles [tb, te) with one cache policy; tile tb lies in window
        // wi or wi + 1
        auto walk = [&](const int tb, const int te, auto nt_tag) {
            auto ldw = [&](TileData<FMT, D> &buf, int i) { ld(buf, min(i, te - 1), nt_tag); };
            auto proc = [&](const TileData<FMT, D> &buf, int i) { process(buf, 16 * i); };
            auto next_window = [&](int i) {
                set_run_priority(t1 - i + run_after, run_len);
                if (i / (64 * TPB) != wi) {  // entering the next window
                    ++wi;
                    win_a = win_b;
                    win_b = win_c;
                    win_c = load_win(wi + 2);
                }
            };
            if constexpr (NQ == 2 && FMT != FMT_FP16) {
                // two column groups: twice the compute per tile at 2 waves /
                // SIMD, so three tile buffers keep two tiles' loads in flight
                // (fp16 tiles are twice the size: they stay at two)
                TileData<FMT, D> buf0, buf1, buf2;
                ldw(buf0, tb);
                ldw(buf1, tb + 1);
                // loop invariant: tile i lies in window wi, its data is in
                // buf0 and tile i + 1's in buf1
                for (int i = tb; i < te; i += 3) {
                    next_window(i);
                    ldw(buf2, i + 2);
                    proc(buf0, i);
                    ldw(buf0, i + 3);
                    if (i + 1 < te)
                        proc(buf1, i + 1);
                    ldw(buf1, i + 4);
                    if (i + 2 < te)
                        proc(buf2, i + 2);
                }
            } else {
                TileData<FMT, D> buf0, buf1;
                ldw(buf0, tb);
                // loop invariant: tile i lies in window wi and its data is in buf0
                for (int i = tb; i < te; i += 2) {
                    next_window(i);
                    ldw(buf1, i + 1);
                    proc(buf0, i);
                    ldw(buf0, i + 2);
                    if (i + 1 < te)
                        proc(buf1, i + 1);
                }
            }
        };
        auto has_shared = [&](int win) {
            return __builtin_amdgcn_ballot_w64((win & kSharedBlock) != 0) != 0;
        };
        int ts = t0;  // end of the leading windows that hold shared blocks
        if (has_shared(win_a)) {
            ts = (wi + 1) * 64 * TPB;
            if (has_shared(win_b))
                ts = has_shared(win_c) ? t1 : (wi + 2) * 64 * TPB;
        }
        ts = min(ts, t1);
        if (ts > t0)
            walk(t0, ts, std::false_type{});
        if (ts < t1)
            walk(ts, t1, std::true_type{});
    
        // ---- epilogue: lane holds dims 64 g4 + 16 grp + (0..15) of head col
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            float lt = l[q] + __shfl_xor(l[q], 16);
            lt += __shfl_xor(lt, 32);
            if (!cg[q].active)
                continue;
            if constexpr (kChannel) {
                // V channel scales: o[4 g4 + i][v] is dim 64 g4 + 16 grp + 4 v + i
                const float *srow = p.v_scale + (int64_t)h * D + 16 * grp;
#pragma unroll
                for (int g4 = 0; g4 < D / 64; ++g4)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const float4 sc4 =
                            *reinterpret_cast<const float4 *>(srow + 64 * g4 + 4 * v);
                        o[q][4 * g4 + 0][v] *= sc4.x;
                        o[q][4 * g4 + 1][v] *= sc4.y;
                        o[q][4 * g4 + 2][v] *= sc4.z;
                        o[q][4 * g4 + 3][v] *= sc4.w;
                    }
            }
            // the whole unit: final output; else a piece of a unit: slot 0
            // if it continues a unit, slot 1 if it starts one (decode walk
            // only); unit column 16 q + col
            const int kind = (t0 == 0 && t1 == n) ? 1 : 2;
            const int slot = t0 > 0 ? 0 : 1;
            const int64_t idx = ((int64_t)w * 2 + slot) * p.cols + 16 * q + col;
            if constexpr (kDefer) {
                if (last) {   // the run's loads are done: store everything
#pragma unroll
                    for (int i = 0; i < kHeld; ++i) {
                        emit_held(held[i]);
                        held[i].kind = 0;
                    }
                    emit(o[q], m[q], lt, out_scale, kind, cg[q].orow, idx);
                } else {      // hold it; when every slot is full, store the oldest
                    emit_held(held[0]);
#pragma unroll
                    for (int i = 0; i + 1 < kHeld; ++i)
                        held[i] = held[i + 1];
                    Held &x = held[kHeld - 1];
#pragma unroll
                    for (int i = 0; i < DT; ++i)
                        x.o[i] = o[q][i];
                    x.m = m[q];
                    x.l = lt;
                    x.s = out_scale;
                    x.kind = kind;
                    x.orow = cg[q].orow;
                    x.idx = idx;
                }
            } else {
                emit(o[q], m[q], lt, out_scale, kind, cg[q].orow, idx);
            }
        }
    };

    // ---- decode: walk the run [g0, g1) unit by unit (values wave-uniform).
    // Unit column c = 16 q + col (column group q) is query head c of the
    // unit's KV head; with short chunks (q_start set: every chunk at most
    // cols / r tokens, chunk token i at position ctx - nq + i) it is chunk
    // token c / r, query head c % r, and it takes the tokens at or before its
    // position.
    int b = rec.b;
    int g = rec.g0;
    int n = ctx_tiles(p.context_lens, b, p.max_ctx);
    int base = rec.base;
    run_len = rec.g1 - rec.g0;
    while (g < rec.g1) {
        if (g >= base + p.Hkv * n) {
            base += p.Hkv * n;
            ++b;
            n = ctx_tiles(p.context_lens, b, p.max_ctx);
            continue;
        }
        const int h = (g - base) / n;
        const int t0 = g - base - h * n;
        const int t1 = min(n, t0 + (rec.g1 - g));
        const int ctx = min(p.context_lens[b], p.max_ctx);
        const int gh = model_head(p, h);
        int qs = b, nq = 1, tcol = 1 << 30;  // tcol: causal bound of chunk token 0
        if (p.q_start) {
            qs = p.q_start[b];
            nq = min(p.q_start[b + 1] - qs, max(ctx, 0));
            tcol = ctx - nq + 1;
        }
        run_after = rec.g1 - g - (t1 - t0);
        if (nq > 0) {  // (an empty chunk has nothing to attend)
            Cols cg[NQ];
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const int c = 16 * q + col;
                const int ci = c / p.r, cj = c % p.r;
                const bool act = c < p.cols && ci < nq;
                const int64_t row =
                    (int64_t)(qs + (act ? ci : 0)) * p.Hq + gh * p.r + (act ? cj : 0);
                cg[q] = Cols{p.q + row * D, p.out + row * D, p.q_start ? tcol + ci : tcol, act};
            }
            attend(b, h, ctx, n, t0, t1, cg, g + (t1 - t0) >= rec.g1);
        }
        g += t1 - t0;
    }
    if constexpr (kDefer) {   // pieces before an empty last chunk, or inactive lanes'
#pragma unroll
        for (int i = 0; i < kHeld; ++i)
            emit_held(held[i]);
    }
    if constexpr (kDefer) {   // the record for the merge launch, after the loads
        if (p.inline_plan && lane == 0)
            p.plan_rec[w] = rec;
    }
}

// Log-sum-exp merge of the pieces of a unit cut by run boundaries:
//   M = max_i m_i,  L = sum_i l_i 2^(m_i - M),  out = sum_i acc_i 2^(m_i - M) / L.
// Workgroup (k, y) looks at the boundary between runs k-1 and k; when that
// boundary is the first one of the unit holding tile g0(k), its wavefront c
// merges column kMergeCols * y + c of that unit (up to kMergeCols wavefronts
// per workgroup: one per column was 20 % slower on C3, sixteen per workgroup
// made the 16-column merge of short chunks 2.6x slower).  The pieces are run
// k-1's slot 1 (the unit's start) and slot 0 of runs k, k+1, ... up to the
// unit's end.  It runs as its own launch, so the partials written by
// wavefronts on any XCD are visible without device-wide fences.  Loads come in
// two batches: the run records (each carries its unit's bounds), then every
// piece's (m, l) together with the first pieces' partial outputs.
constexpr int kMergeCols = 4;

template <int D>
__global__ __launch_bounds__(64 * kMergeCols) void merge_runs_kernel(DecodeParams p)
{
    constexpr int PER = D / 64;   // output dims per lane
    constexpr int kAhead = 8;     // pieces whose partials load with (m, l)
    const int k = blockIdx.x + 1;
    const int col = kMergeCols * blockIdx.y + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (col >= p.cols)
        return;
    // first loads: the runs in use, and the records of runs k - 1 .. k + 62
    // (lane j: run k - 1 + j; p.W records are allocated)
    const int nrec = p.plan_meta[0];
    const int rj = k - 1 + lane;
    PlanRecord rr{};
    if (rj < p.W)
        rr = p.plan_rec[rj];
    if (k >= nrec)
        return;
    const int g0k = __builtin_amdgcn_readlane(rr.g0, 1);
    const int us = __builtin_amdgcn_readlane(rr.us, 1);
    const int ue = __builtin_amdgcn_readlane(rr.ue, 1);
    if (us == g0k)
        return;                           // the boundary is a unit start
    if (__builtin_amdgcn_readlane(rr.g0, 0) > us)
        return;                           // an earlier boundary cuts this unit
    const int b = __builtin_amdgcn_readlane(rr.b, 1);
    const int base = __builtin_amdgcn_readlane(rr.base, 1);
    const int h = (us - base) / (ue - us);
    // pieces: j = 0 is run k-1 (slot 1), j >= 1 is run k-1+j (slot 0): the
    // runs from k on that start before the unit's end (a prefix of them)
    int np = 1 + __builtin_popcountll(
                     __builtin_amdgcn_ballot_w64(lane >= 1 && rj < nrec && rr.g0 < ue));
    if (np == 64) {  // a unit over more than 63 runs: count the rest
        for (int j0 = 64;; j0 += 64) {
            const int r2 = k - 1 + j0 + lane;
            const uint64_t m = __builtin_amdgcn_ballot_w64(r2 < nrec && p.plan_rec[r2].g0 < ue);
            np += __builtin_popcountll(m);
            if (m != ~0ull)
                break;
        }
    }
    auto piece = [&](int j) -> int64_t {
        return ((int64_t)(k - 1 + j) * 2 + (j == 0 ? 1 : 0)) * p.cols + col;
    };
    // output row (short chunks: column col is chunk token col / r)
    int64_t row = (int64_t)b * p.Hq + model_head(p, h) * p.r + col;
    if (p.q_start) {
        const int qs = p.q_start[b];
        const int nq = min(p.q_start[b + 1] - qs, min(max(p.context_lens[b], 0), p.max_ctx));
        if (col / p.r >= nq)
            return;
        row = (int64_t)(qs + col / p.r) * p.Hq + model_head(p, h) * p.r + col % p.r;
    }
    // second loads: (m, l) of every piece, the partials of the first kAhead
    float ahead[kAhead][PER];
#pragma unroll
    for (int j = 0; j < kAhead; ++j) {
        if (j < np) {
            const float *a = p.ws_acc + piece(j) * D + PER * lane;
#pragma unroll
            for (int i = 0; i < PER; ++i)
                ahead[j][i] = a[i];
        }
    }
    float mx = -INFINITY;
    for (int j = lane; j < np; j += 64)
        mx = fmaxf(mx, p.ws_ml[2 * piece(j)]);
    mx = wave_max(mx);
    float ls = 0.0f;
    for (int j = lane; j < np; j += 64)
        ls += p.ws_ml[2 * piece(j) + 1] * __builtin_amdgcn_exp2f(p.ws_ml[2 * piece(j)] - mx);
    ls = wave_sum(ls);
    float acc[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i)
        acc[i] = 0.0f;
#pragma unroll
    for (int j = 0; j < kAhead; ++j) {
        if (j < np) {
            const float wgt = __builtin_amdgcn_exp2f(p.ws_ml[2 * piece(j)] - mx);
#pragma unroll
            for (int i = 0; i < PER; ++i)
                acc[i] += ahead[j][i] * wgt;
        }
    }
#pragma unroll 4
    for (int j = kAhead; j < np; ++j) {
        const int64_t ix = piece(j);
        const float wgt = __builtin_amdgcn_exp2f(p.ws_ml[2 * ix] - mx);
        const float *a = p.ws_acc + ix * D + PER * lane;
#pragma unroll
        for (int i = 0; i < PER; ++i)
            acc[i] += a[i] * wgt;
    }
    const float inv = 1.0f / ls;
    f16 *orow = p.out + row * D + PER * lane;
#pragma unroll
    for (int i = 0; i < PER; ++i)
        orow[i] = (f16)(acc[i] * inv);
}

}  // namespace kvq
