// kvq_prefill.hpp -- chunked-prefill attention over the paged, quantized pool
// (gfx950).
//
// Computes, for every token i of sequence b's chunk (its last nq cached
// tokens, at position pos = ctx - nq + i) and every query head g of KV head h
// ("KV Cache优化实战" s1.1: each prompt token attends to the tokens before it;
// s2.1: the query heads of a group share one KV head; xpshop.cn article 312
// s6: long prompts go in chunks):
//     out[i][g] = sum_{t <= pos} softmax_t(sm * q[i][g] . Khat[t]) Vhat[t]
//
// A workgroup of four wavefronts takes 128 query rows of one (sequence, KV
// head): rows are (chunk token, query head) pairs, 128 / r tokens x r heads,
// and each wavefront owns 32 of them (two 16-row MFMA tiles).  The workgroup
// walks the keys its rows need in steps of 32 tokens.  For every step the
// 256 threads gather the step's K / V codes and scales through the block
// table once, convert the codes to exact fp16 and store them in LDS (three
// buffers: while step s is contracted, step s + 1's K forms the next scores
// and step s + 2's loads are in flight); every wavefront then contracts its
// rows against the step from LDS.  A tile is therefore converted once for
// 128 rows instead of once per 32-row wavefront.  What bounds the walk is
// the vector ALU: per step a wavefront issues ~290 VALU instructions (score
// scaling, softmax, the P split) against 48 MFMAs, so the VALU port, not
// the matrix core, is the busy unit.
//
// Contractions (16x16x32 fp16 MFMA, laid out as in the decode kernel so the
// softmax needs only two cross-lane exchanges per row):
//   S^T[key][row] = K (16 keys x 32 dims, from LDS) * Q^T (32 dims x 16 rows,
//       in registers); one accumulator per scale group, K group scales (with
//       the softmax scale) applied to the partial dots in fp32.
//   O^T[dim][row] += V^T (16 dims x 32 keys, from LDS) * P_hi^T, then the
//       same V^T * P_lo^T: P carried as an fp16 pair (~2^-21 relative) with
//       the V group scales folded in, as the decode kernel does.
// Online softmax in base 2 with the decode kernel's lazy rescale; the
// running maximum is subtracted inside the score FMAs.
#pragma once

#include "kvq_device.hpp"
#include "kvq_decode.hpp"

namespace kvq {

constexpr int kPfWaves = 4;                 // wavefronts per workgroup
constexpr int kPfRows = 32 * kPfWaves;      // query rows per workgroup
constexpr int kPfKeys = 32;                 // keys per step

// Query rows (chunk tokens) per workgroup for a GQA ratio r.
__host__ __device__ constexpr int prefill_tokens_per_group(int r) { return kPfRows / r; }

// Chunk tokens per workgroup: 128 / r; query blocks per (sequence, KV head):
// p.groups = ceil(max chunk length / (128 / r)).
template <int FMT, int D, int BS, int NG>
__global__ __launch_bounds__(64 * kPfWaves, 2) void prefill_kernel(DecodeParams p)
{
    constexpr int EB = FMT == FMT_FP16 ? 2 : 1;
    constexpr bool kGroup = NG > 0;
    constexpr int NA = kGroup ? NG : 1;         // score accumulators (scale groups)
    constexpr int G = kGroup ? D / NG : D;
    constexpr bool kChannel = FMT == FMT_INT8 && !kGroup;
    constexpr int KS = D / 32;                  // 16x16x32 k-steps over head_dim
    constexpr int DT = D / 16;                  // 16-dim output tiles
    constexpr int KSTR = D + 8;                 // K row stride in LDS (halves; 16 B pad)
    constexpr int VSTR = kPfKeys + 4;           // V row (one dim) stride in LDS (halves)
    // tile bytes per token in the pool, and 16-byte pieces per step
    constexpr int TB = FMT == FMT_INT4 ? D / 2 : D * EB;
    constexpr int KPIECES = kPfKeys * TB / 16;  // K pieces (one token's 16 bytes)
    constexpr int VPIECES = kPfKeys * TB / 16;  // V 16-byte units
    constexpr int NT = 64 * kPfWaves;
    constexpr int KPT = (KPIECES + NT - 1) / NT;  // per thread
    constexpr int VPT = (VPIECES + NT - 1) / NT;
    static_assert(FMT != FMT_INT4 || (D == 128 && kGroup), "INT4: head_dim 128, group scales");
    static_assert(!kGroup || G >= 64, "groups cover a 64-dim chunk");

    // three buffers: step s is contracted from one while step s + 1's K
    // feeds the next scores and step s + 2 is being stored
    __shared__ __align__(16) f16 k_lds[3][kPfKeys * KSTR];
    __shared__ __align__(16) f16 v_lds[3][D * VSTR];
    __shared__ __align__(16) float sc_lds[3][2][kPfKeys * NA];  // [buf][K, V][key * NA + g]

    const int tid = threadIdx.x;
    const int wv = tid >> 6, lane = tid & 63;
    const int col = lane & 15, grp = lane >> 4;

    // ---- workgroup -> (sequence, KV head, query block).  Workgroups go
    // round-robin to the 8 XCDs (w to XCD w % 8): XCD x takes the pairs x,
    // x + 8, ... one after another, all query blocks of a pair together
    // (longest first), so the pair's K / V stays in that XCD's L2.
    const int TQ = kPfRows / p.r;               // chunk tokens per workgroup
    const int nqb = p.groups;
    const int w = blockIdx.x;
    const int sl = w >> 3;
    const int pair = (w & 7) + 8 * (sl / nqb);
    const int qb = nqb - 1 - sl % nqb;
    if (pair >= p.B * p.Hkv)
        return;
    const int b = pair / p.Hkv;
    const int h = pair % p.Hkv;
    const int ctx = min(max(p.context_lens[b], 0), p.max_ctx);
    const int qs = p.q_start[b];
    const int nq = min(p.q_start[b + 1] - qs, ctx);
    const int i0 = qb * TQ;
    if (i0 >= nq)
        return;
    const int c0 = ctx - nq;                     // tokens cached before the chunk
    const int kend = c0 + min(i0 + TQ, nq);      // keys the last row reads
    const int nsteps = (kend + kPfKeys - 1) / kPfKeys;
    const int gh = model_head(p, h);

    // ---- this lane's query rows (row tile rt: workgroup row 32 wv + 16 rt + col)
    int pos[2];
    bool act[2];
    int64_t qrow[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const int rho = 32 * wv + 16 * rt + col;
        const int i = rho / p.r, j = rho % p.r;
        act[rt] = rho < TQ * p.r && i0 + i < nq;
        pos[rt] = act[rt] ? c0 + i0 + i : -1;
        qrow[rt] = (int64_t)(qs + (act[rt] ? i0 + i : 0)) * p.Hq + gh * p.r + (act[rt] ? j : 0);
    }
    // the wavefront's smallest and largest positions: steps wholly below the
    // first need no mask, steps wholly above the second are skipped
    int wpos = 1 << 30, wmax = -1;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
        if (act[rt]) {
            wpos = min(wpos, pos[rt]);
            wmax = max(wmax, pos[rt]);
        }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        wpos = min(wpos, __shfl_xor(wpos, o));
        wmax = max(wmax, __shfl_xor(wmax, o));
    }
    wmax = __builtin_amdgcn_readfirstlane(wmax);
    wpos = wmax < 0 ? -1 : __builtin_amdgcn_readfirstlane(wpos);  // no rows: skip every step

    // ---- Q^T operands: lane (row col, k-group grp) holds dims 32 s + 8 grp .. + 7
    f16x8 qop[2][KS];
    f16x8 qlo[2][kChannel ? KS : 1];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const f16 *qr = p.q + qrow[rt] * D;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            qop[rt][s] = *reinterpret_cast<const f16x8 *>(qr + 32 * s + 8 * grp);
            if (!act[rt])
                qop[rt][s] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
        }
    }
    if constexpr (kChannel) {  // K channel scales ride on q as an fp16 pair hi + lo
        const float *srow = p.k_scale + (int64_t)h * D;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            float sc[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                sc[e] = srow[32 * s + 8 * grp + e];
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = (float)qop[rt][s][e] * sc[e];
                    const f16 hv = (f16)x;
                    qop[rt][s][e] = hv;
                    qlo[rt][s][e] = (f16)(x - (float)hv);
                }
        }
    }
    float score_scale = p.score_scale;
    float out_scale = 1.0f;
    if constexpr ((FMT == FMT_FP8 || FMT == FMT_E5M2) && !kGroup) {
        score_scale *= p.k_scale[h];
        out_scale = p.v_scale[h];
    }

    // ---- the step loader.  A step's 32 keys span two 16-token halves, each
    // inside one block; fetch(step) reads the two block-table entries (the
    // same address in every lane, so each wavefront reads them once);
    // load() gathers that step's K / V codes (16-byte pieces) and scales
    // into registers; store() converts them and writes LDS.  Every
    // wavefront's K and V pieces lie in one half, so a piece's address is a
    // wave-uniform tile base (scalar registers) plus an offset fixed per
    // thread: the loads cost no vector address arithmetic.  The walk issues
    // fetch three steps ahead and load two steps ahead, so neither the table
    // read nor the code read it depends on waits behind compute.  Tokens at
    // or past ctx read a valid block and are written as zeros (stale slots
    // may hold non-finite fp16 / E5M2 codes).
    const int32_t *bt = p.block_tables + (int64_t)b * p.max_blocks;
    constexpr int PPT = TB / 16;                // K pieces per token
    constexpr int UPH = VPIECES / 2;            // V units per 16-token half
    static_assert(64 / PPT <= 16 && UPH % 64 == 0, "a wavefront's pieces lie in one half");
    // whether a thread's x-th piece exists (always, when the pieces fill
    // every thread: no branch then, so no wait lands inside one)
    auto has_k = [&](int x) { return KPIECES % NT == 0 || tid + NT * x < KPIECES; };
    auto has_v = [&](int x) { return VPIECES % NT == 0 || tid + NT * x < VPIECES; };
    const int wvu = __builtin_amdgcn_readfirstlane(wv);
    // per thread: byte offsets of its pieces inside their (block, head) tile
    // (a step starts on a block boundary or a block's second half, so these
    // do not change from step to step), and the half each piece lies in
    int k_off[KPT], v_off[VPT];
#pragma unroll
    for (int x = 0; x < KPT; ++x) {
        const int c = tid + NT * x;
        const int kk = c / PPT, pc = c % PPT;
        if constexpr (FMT == FMT_INT4)
            k_off[x] = (kk % BS) * 64 + 16 * pc;
        else
            k_off[x] = k_offset<D, EB>(BS, kk % BS, pc * 16 / EB);
    }
#pragma unroll
    for (int x = 0; x < VPT; ++x) {
        const int c = tid + NT * x;
        const int hf = c / UPH, u = c % UPH;
        const int hb = (16 * hf % BS) / 16;     // half of its block
        if constexpr (FMT == FMT_INT4) {
            v_off[x] = hb * 1024 + u * 16;      // (dim quad, token quad) unit
        } else {
            // unit u = (part e, dim quad dq, token quad tq)
            const int e = u / D, dq = (u % D) / 4, tq = u % 4;
            v_off[x] = (((hb * EB + e) * (D / 4) + dq) * 4 + tq) * 16;
        }
    }
    auto k_half = [&](int x) { return ((64 * wvu + NT * x) / PPT) / 16; };   // wave-uniform
    auto v_half = [&](int x) { return (64 * wvu + NT * x) / UPH; };          // wave-uniform
    // scale loads: every thread loads one (the first 2 x 32 x NG are kept)
    const int s_kind = (tid / (kPfKeys * NA)) & 1, s_idx = tid % (kPfKeys * NA);
    const int s_half = (s_idx / NA) / 16;
    const int s_off = ((s_idx / NA) % BS) * NA + s_idx % NA;
    u32x4 kraw[KPT], vraw[VPT];
    float sraw = 0.0f;
    int ent_f[2] = {0, 0}, ent_l[2] = {0, 0};   // table entries: fetched / for the next load
    auto fetch = [&](int step) {
        const int kb = step * kPfKeys;
        ent_f[0] = bt[min(kb, kend - 1) / BS];
        ent_f[1] = bt[min(kb + 16, kend - 1) / BS];
    };
    auto tile_of = [&](int half) -> int64_t {   // (block, head) tile of a half, wave-uniform
        const int e = __builtin_amdgcn_readfirstlane(ent_l[half]);
        return (int64_t)min(max(e & kBlockIdMask, 0), p.num_blocks - 1) * p.Hkv + h;
    };
    auto load = [&]() {   // the step whose entries are in ent_l
        const int64_t t0 = tile_of(0), t1 = tile_of(1);
#pragma unroll
        for (int x = 0; x < KPT; ++x)
            if (has_k(x)) {
                const uint8_t *tile = p.k_pool + (k_half(x) ? t1 : t0) * (BS * TB);
                kraw[x] = *reinterpret_cast<const u32x4 *>(tile + k_off[x]);
            }
#pragma unroll
        for (int x = 0; x < VPT; ++x)
            if (has_v(x)) {
                const uint8_t *tile = p.v_pool + (v_half(x) ? t1 : t0) * (BS * TB);
                vraw[x] = *reinterpret_cast<const u32x4 *>(tile + v_off[x]);
            }
        if constexpr (kGroup) {
            const float *arr = s_kind == 0 ? p.k_scale : p.v_scale;
            sraw = arr[(s_half ? t1 : t0) * (BS * NG) + s_off];
        }
    };
    auto cvt4 = [&](uint32_t wd) -> f16x4 {
        if constexpr (FMT == FMT_INT8)
            return int8x4_to_f16x4(wd);
        else if constexpr (FMT == FMT_FP8)
            return fp8x4_to_f16x4(wd);
        else
            return e5m2x4_to_f16x4(wd);
    };
    // kTail: the step reaches past ctx (its tokens there become zeros)
    auto store = [&](int step, int buf, auto tail_tag) {
        constexpr bool kTail = decltype(tail_tag)::value;
        const int kb = step * kPfKeys;
        const f16x4 z4 = {0, 0, 0, 0};
#pragma unroll
        for (int x = 0; x < KPT; ++x) {
            if (has_k(x)) {
                const int c = tid + NT * x;
                const int kk = c / PPT, pc = c % PPT;
                const bool ok = !kTail || kb + kk < ctx;
                f16 *dst = &k_lds[buf][kk * KSTR];
                const u32x4 r = kraw[x];
                if constexpr (FMT == FMT_INT4) {
                    // slice pc: dword q holds dims base .. base + 7,
                    // base = 64 (q / 2) + 16 pc + 8 (q % 2)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        f16x4 lo, hi;
                        int4x8_to_f16x4(r[q], lo, hi);
                        const int base = 64 * (q / 2) + 16 * pc + 8 * (q % 2);
                        *reinterpret_cast<f16x8 *>(dst + base) = ok ? cat8(lo, hi) : cat8(z4, z4);
                    }
                } else if constexpr (FMT == FMT_FP16) {
                    const f16x8 v = ok ? bit_cast<f16x8>(r) : cat8(z4, z4);
                    *reinterpret_cast<f16x8 *>(dst + 8 * pc) = v;
                } else {
                    const f16x8 a = ok ? cat8(cvt4(r[0]), cvt4(r[1])) : cat8(z4, z4);
                    const f16x8 bb = ok ? cat8(cvt4(r[2]), cvt4(r[3])) : cat8(z4, z4);
                    *reinterpret_cast<f16x8 *>(dst + 16 * pc) = a;
                    *reinterpret_cast<f16x8 *>(dst + 16 * pc + 8) = bb;
                }
            }
        }
#pragma unroll
        for (int x = 0; x < VPT; ++x) {
            if (has_v(x)) {
                const int c = tid + NT * x;
                const int hf = c / UPH, u = c % UPH;
                const u32x4 r = vraw[x];
                if constexpr (FMT == FMT_INT4) {
                    // unit (dq, tq): dword q holds dims d, d + 1 of tokens
                    // 4 tq .. 4 tq + 3, d = 64 (q / 2) + 4 dq + 2 (q % 2)
                    const int dq = u / 4, tq = u % 4;
                    const int t0 = kb + 16 * hf + 4 * tq;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        f16x4 lo, hi;
                        int4x8_to_f16x4(r[q], lo, hi);
                        if constexpr (kTail) {
#pragma unroll
                            for (int v = 0; v < 4; ++v)
                                if (t0 + v >= ctx)
                                    lo[v] = hi[v] = (f16)0.0f;
                        }
                        const int d = 64 * (q / 2) + 4 * dq + 2 * (q % 2);
                        *reinterpret_cast<f16x4 *>(&v_lds[buf][d * VSTR + 16 * hf + 4 * tq]) = lo;
                        *reinterpret_cast<f16x4 *>(&v_lds[buf][(d + 1) * VSTR + 16 * hf + 4 * tq]) = hi;
                    }
                } else {
                    const int e = u / D, dq = (u % D) / 4, tq = u % 4;
                    const int t0 = kb + 16 * hf + 4 * tq;
                    // 1-byte codes: dword m holds dim 4 dq + m of the 4 tokens;
                    // fp16: dwords (2 m', 2 m' + 1) hold dim 4 dq + 2 e + m'
                    constexpr int NDIM = 4 / EB;
#pragma unroll
                    for (int m = 0; m < NDIM; ++m) {
                        f16x4 vv;
                        if constexpr (FMT == FMT_FP16)
                            vv = f16x4_from_u2(r[2 * m], r[2 * m + 1]);
                        else
                            vv = cvt4(r[m]);
                        if constexpr (kTail) {
#pragma unroll
                            for (int v = 0; v < 4; ++v)
                                if (t0 + v >= ctx)
                                    vv[v] = (f16)0.0f;
                        }
                        const int d = 4 * dq + NDIM * e + m;
                        *reinterpret_cast<f16x4 *>(&v_lds[buf][d * VSTR + 16 * hf + 4 * tq]) = vv;
                    }
                }
            }
        }
        if constexpr (kGroup) {
            // threads past the first 2 x 32 x NG write the same value to
            // the same slot as a thread below (same load): no branch
            const bool ok = !kTail || kb + s_idx / NG < ctx;
            sc_lds[buf][s_kind][s_idx] =
                ok ? (s_kind == 0 ? sraw * score_scale : sraw) : 0.0f;
        }
    };
    auto store_step = [&](int step, int buf) {
        if ((step + 1) * kPfKeys <= ctx)
            store(step, buf, std::false_type{});
        else
            store(step, buf, std::true_type{});
    };

    // ---- accumulators
    f32x4 o[2][DT];
    float m[2], l[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
        for (int t = 0; t < DT; ++t)
            o[rt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        m[rt] = 0.0f;
        l[rt] = 0.0f;
    }

    // S^T = K Q^T of the step in LDS buffer buf, per half (16 keys), one
    // accumulator per scale group
    using SAcc = f32x4[2][2][NA];
    auto qk = [&](int buf, SAcc &sacc) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int g = 0; g < NA; ++g)
                    sacc[hf][rt][g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const f16x8 a =
                    *reinterpret_cast<const f16x8 *>(&k_lds[buf][(16 * hf + col) * KSTR + 32 * s + 8 * grp]);
                const int gi = NA == 2 ? s / (KS / 2) : 0;
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    sacc[hf][rt][gi] = mfma32(a, qop[rt][s], sacc[hf][rt][gi]);
                    if constexpr (kChannel)
                        sacc[hf][rt][0] = mfma32(a, qlo[rt][s], sacc[hf][rt][0]);
                }
            }
        }
    };

    // One step: keys kb .. kb + 31, scores in sacc, codes in LDS buffer buf.
    // Once its scores are formed, the next step's (K from buffer nbuf) go
    // into sacc, the MFMAs interleaved with the softmax VALU work.  kMask:
    // some key may lie past some row's position.  kFirst: the wavefront's
    // first step (m is not yet a running maximum).  kFuse: the step also
    // converts and stores step + 2 (whole, in range) into LDS buffer sbuf.
    auto compute = [&](int step, int buf, int nbuf, SAcc &sacc, auto mask_tag, auto first_tag,
                       auto fuse_tag, int sbuf) {
        constexpr bool kMask = decltype(mask_tag)::value;
        constexpr bool kFirst = decltype(first_tag)::value;
        constexpr bool kFuse = decltype(fuse_tag)::value;
        const int kb = step * kPfKeys;
        // scores of this lane's keys kb + 16 hf + 4 grp + v (base 2, scaled),
        // less the running maximum m (0 before the first step)
        float z[2][2][4];   // [rt][hf][v]
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            float sk[4][NA];
            if constexpr (kGroup) {
                const float *ks = &sc_lds[buf][0][(16 * hf + 4 * grp) * NA];
#pragma unroll
                for (int v = 0; v < 4; ++v)
#pragma unroll
                    for (int g = 0; g < NA; ++g)
                        sk[v][g] = ks[v * NA + g];
            }
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float base = kFirst ? 0.0f : -m[rt];
                    float acc;
                    if constexpr (kGroup) {
                        acc = __builtin_fmaf(sacc[hf][rt][0][v], sk[v][0], base);
                        if constexpr (NA == 2)
                            acc = __builtin_fmaf(sacc[hf][rt][1][v], sk[v][1], acc);
                    } else {
                        acc = __builtin_fmaf(sacc[hf][rt][0][v], score_scale, base);
                    }
                    const int t = kb + 16 * hf + 4 * grp + v;
                    z[rt][hf][v] = (!kMask || t <= pos[rt]) ? acc : -INFINITY;
                }
        }
        // online softmax: the maximum moves only when a score passes it by
        // more than kSlack (in log2 units), and always on the first step
        constexpr float kSlack = !kGroup ? 8.0f
                               : FMT == FMT_INT8 || FMT == FMT_FP8 ? 6.0f
                               : FMT == FMT_INT4 ? 2.0f : 0.0f;
        // the next step's S^T MFMAs (sacc is free now that z holds this
        // step's scores) run beside the softmax VALU work below
        qk(nbuf, sacc);
        float mt[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {   // a chain, so it folds into 3-input maxima
            mt[rt] = z[rt][0][0];
#pragma unroll
            for (int x = 1; x < 8; ++x)
                mt[rt] = fmaxf(mt[rt], z[rt][x / 4][x % 4]);
        }
        max_over_groups2(mt[0], mt[1]);
        // one branch for both row tiles: a row whose scores stay at or below
        // its maximum shifts by 0 (alpha 1) when the other tile moves
        if (kFirst || __builtin_amdgcn_ballot_w64(fmaxf(mt[0], mt[1]) > kSlack)) {
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                // a row with every key masked (mt = -inf) keeps its maximum
                const float shift = kFirst ? (mt[rt] > -INFINITY ? mt[rt] : 0.0f) : fmaxf(mt[rt], 0.0f);
                if constexpr (!kFirst) {
                    const float alpha = __builtin_amdgcn_exp2f(-shift);
                    l[rt] *= alpha;
#pragma unroll
                    for (int t = 0; t < DT; ++t)
                        o[rt][t] *= alpha;
                }
                m[rt] += shift;
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        z[rt][hf][v] -= shift;
            }
        }
        // O^T += V^T P^T per scale group, P (with the group's V scales)
        // split into fp16 hi + lo: a lane's 8 k-slots are its 8 keys (4 grp
        // .. + 3 of each half), so one read of the V codes serves the hi and
        // the lo product
        f16x8 phi[NA][2], plo[NA][2];   // [group][rt]
        auto make_p = [&](int g) {
            float sv[2][4];
            if constexpr (kGroup) {
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const float *vs = &sc_lds[buf][1][(16 * hf + 4 * grp) * NA];
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        sv[hf][v] = vs[v * NA + g];
                }
            }
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                f16x2 h[4], lo[4];
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int v = 0; v < 4; v += 2) {
                        const float P0 = kGroup ? z[rt][hf][v] * sv[hf][v] : z[rt][hf][v];
                        const float P1 = kGroup ? z[rt][hf][v + 1] * sv[hf][v + 1] : z[rt][hf][v + 1];
                        split_f16x2(P0, P1, h[2 * hf + v / 2], lo[2 * hf + v / 2]);
                    }
                phi[g][rt] = f16x8{h[0].x, h[0].y, h[1].x, h[1].y, h[2].x, h[2].y, h[3].x, h[3].y};
                plo[g][rt] = f16x8{lo[0].x, lo[0].y, lo[1].x, lo[1].y, lo[2].x, lo[2].y, lo[3].x, lo[3].y};
            }
        };
        auto pv = [&](int g) {
#pragma unroll
            for (int t = g * DT / NA; t < (g + 1) * DT / NA; ++t) {
                const f16 *vr = &v_lds[buf][(16 * t + col) * VSTR + 4 * grp];
                const f16x8 a = cat8(*reinterpret_cast<const f16x4 *>(vr),
                                     *reinterpret_cast<const f16x4 *>(vr + 16));
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    o[rt][t] = mfma32(a, phi[g][rt], o[rt][t]);
                    o[rt][t] = mfma32(a, plo[g][rt], o[rt][t]);
                }
            }
        };
        // exp2, the sums and the first group's P (VALU)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    z[rt][hf][v] = __builtin_amdgcn_exp2f(z[rt][hf][v]);
                    l[rt] += z[rt][hf][v];
                }
        make_p(0);

        if constexpr (NA == 2) {
            // the second group's P rides between the first group's MFMAs
            make_p(1);
            pv(0);

            pv(1);
        } else {
            pv(0);
        }
        if constexpr (kFuse) {
            // step s + 2's conversion and LDS stores fill the VALU slots
            // beside this step's last MFMAs
            store(step + 2, sbuf, std::false_type{});
        }
    };

    // ---- the walk: the codes of step s + 2 and the blocks of step s + 3 in
    // flight while step s is computed (and step s + 1's scores formed).  The
    // wavefront's steps fall in three runs: below every row's position (no
    // mask), then up to its last position (masked), then none of its keys
    // (loads and barriers only); one loop per run keeps each loop's
    // accumulators in place.
    fetch(0);
    ent_l[0] = ent_f[0];
    ent_l[1] = ent_f[1];
    load();
    if (nsteps > 1)
        fetch(1);
    store_step(0, 0);
    if (nsteps > 1) {
        ent_l[0] = ent_f[0];
        ent_l[1] = ent_f[1];
        load();
        if (nsteps > 2)
            fetch(2);
        store_step(1, 1);
    }
    __syncthreads();
    auto advance = [&](int step) {   // before a step's compute
        ent_l[0] = ent_f[0];
        ent_l[1] = ent_f[1];
        if (step + 2 < nsteps)
            load();
        if (step + 3 < nsteps)
            fetch(step + 3);
    };
    auto finish = [&](int step, int b2) {    // after it; b2: buffer of step + 2
        if (step + 2 < nsteps)
            store_step(step + 2, b2);
        __syncthreads();
    };
    const int n_free = wpos < 0 ? 0 : min((wpos + 1) / kPfKeys, nsteps);
    const int n_any = wmax < 0 ? 0 : min(wmax / kPfKeys + 1, nsteps);
    SAcc sacc;
    int step = 0, b0 = 0, b1 = 1, b2 = 2;   // buffers of steps s, s + 1, s + 2
    auto rotate = [&]() {
        const int t = b0;
        b0 = b1;
        b1 = b2;
        b2 = t;
    };
    // the next step's buffer; the last step re-forms its own scores instead
    // (a spare contraction, but no branch around the MFMAs)
    auto nb = [&](int s) { return s + 1 < nsteps ? b1 : b0; };
    if (n_any > 0) {   // step 0, every row's first
        qk(0, sacc);
        advance(0);
        if (n_free > 0)
            compute(0, b0, nb(0), sacc, std::false_type{}, std::true_type{}, std::false_type{}, 0);
        else
            compute(0, b0, nb(0), sacc, std::true_type{}, std::true_type{}, std::false_type{}, 0);
        finish(0, b2);
        rotate();
        step = 1;
    }
    // steps whose loads, table reads and store are all in range and whole:
    // the store of step s + 2 goes inside the compute, between its MFMAs
    const int n_fast = min(n_free, min(nsteps - 3, ctx / kPfKeys - 2));
    for (; step < n_fast; ++step) {
        ent_l[0] = ent_f[0];
        ent_l[1] = ent_f[1];
        load();
        fetch(step + 3);
        compute(step, b0, b1, sacc, std::false_type{}, std::false_type{}, std::true_type{}, b2);
        __syncthreads();
        rotate();
    }
    for (; step < n_free; ++step) {
        advance(step);
        compute(step, b0, nb(step), sacc, std::false_type{}, std::false_type{}, std::false_type{}, 0);
        finish(step, b2);
        rotate();
    }
    for (; step < n_any; ++step) {
        advance(step);
        compute(step, b0, nb(step), sacc, std::true_type{}, std::false_type{}, std::false_type{}, 0);
        finish(step, b2);
        rotate();
    }
    for (; step < nsteps; ++step) {
        advance(step);
        finish(step, b2);
        rotate();
    }

    // ---- epilogue: lane holds dims 16 t + 4 grp .. + 3 of its rows
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        float lt = l[rt] + __shfl_xor(l[rt], 16);
        lt += __shfl_xor(lt, 32);
        if (!act[rt])
            continue;
        const float inv = out_scale / lt;
        f16 *orow = p.out + qrow[rt] * D;
#pragma unroll
        for (int t = 0; t < DT; ++t) {
            f32x4 v = o[rt][t] * inv;
            if constexpr (kChannel) {
                const float4 sc4 =
                    *reinterpret_cast<const float4 *>(p.v_scale + (int64_t)h * D + 16 * t + 4 * grp);
                v[0] *= sc4.x;
                v[1] *= sc4.y;
                v[2] *= sc4.z;
                v[3] *= sc4.w;
            }
            *reinterpret_cast<f16x4 *>(orow + 16 * t + 4 * grp) =
                f16x4{(f16)v[0], (f16)v[1], (f16)v[2], (f16)v[3]};
        }
    }
}

}  // namespace kvq
