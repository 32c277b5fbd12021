// kvq_write.hpp -- quantizing cache-write kernel and block-copy kernel.
//
// Cache write ("KV Cache优化实战" s1.1: the new token's K/V is appended to the
// cache; s2.3 / s3.3: INT8 absmax symmetric per group of 64 or 128 elements,
// with a stored scale, or per channel; xpshop.cn article 312 s3: FP8 KV, as
// E4M3 or E5M2).
//
// G > 0: a scale per (token, head, group of G elements) computed here (INT8
// or FP8); G == 0: static scales given by the caller (FP8: one per KV head;
// INT8: one per (KV head, channel)); fp16 is copied.
//
// One wavefront per (token, KV head): lanes 0..31 take K, lanes 32..63 take V,
// each lane D/32 consecutive elements of the head.  A group of G elements is
// spread over G/(D/32) neighbouring lanes; its absmax is reduced across them
// with xor shuffles, so the scale and the codes come out in one pass.  INT8
// codes are stored as excess-128 bytes (c + 128), which the decode kernel
// turns into fp16 with two byte permutes per four codes.  K codes
// go to 64-byte token rows (one dword per lane), V codes to 4x4 micro-tiles
// (the layouts the decode kernel reads, see k_offset / v_offset), scales to
// the slot's entry of the scale arrays.
#pragma once

#include "kvq_device.hpp"

namespace kvq {

struct WriteParams {
    const f16 *k;
    const f16 *v;
    const int64_t *slots;
    uint8_t *k_pool;
    uint8_t *v_pool;
    float *k_scale;
    float *v_scale;
    int32_t num_tokens;
    int32_t Hkv;        // heads in the pools
    int32_t block_size;
    int64_t num_slots;  // num_blocks * block_size
    const int32_t *head_ids;  // pool head h is input head head_ids[h] (null: h)
    int32_t Hkv_src;          // heads per token in k / v
};

constexpr int kWriteWaves = 4;

template <int FMT, int D, int G>
__global__ __launch_bounds__(64 * kWriteWaves) void cache_write_kernel(WriteParams p)
{
#pragma clang fp contract(off)
    constexpr int EPL = D / 32;               // elements per lane
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int64_t pair = (int64_t)blockIdx.x * kWriteWaves + wave;
    if (pair >= (int64_t)p.num_tokens * p.Hkv)
        return;
    const int t = (int)(pair / p.Hkv);
    const int h = (int)(pair % p.Hkv);
    const bool is_v = lane >= 32;
    const int e0 = (lane & 31) * EPL;

    // The slot and the token's values are read together (the values' address
    // does not depend on the slot); the empty asm uses both before the slot
    // check, which keeps the compiler from moving the value load below it.
    const int gh = p.head_ids ? p.head_ids[h] : h;
    const f16 *src = (is_v ? p.v : p.k) + ((int64_t)t * p.Hkv_src + gh) * D + e0;
    int64_t slot = p.slots[t];
    uint32_t raw[EPL / 2];
    if constexpr (EPL == 4) {
        const uint2 r2 = *reinterpret_cast<const uint2 *>(src);
        raw[0] = r2.x;
        raw[1] = r2.y;
    } else {
        raw[0] = *reinterpret_cast<const uint32_t *>(src);
    }
#pragma unroll
    for (int i = 0; i < EPL / 2; ++i)
        __asm__ __volatile__("" : "+v"(raw[i]), "+v"(slot));
    if (slot < 0 || slot >= p.num_slots)
        return;
    float x[EPL];
#pragma unroll
    for (int i = 0; i < EPL / 2; ++i) {
        const f16x2 hv = bit_cast<f16x2>(raw[i]);
        x[2 * i] = (float)hv.x;
        x[2 * i + 1] = (float)hv.y;
    }
    const int BS = p.block_size;
    const int64_t blk = slot / BS;
    const int off = (int)(slot % BS);

    const int64_t head_base = blk * p.Hkv + h;  // (block, head) tile index
    uint32_t code[EPL];

    if constexpr (G > 0) {
        // dynamic per-group scale (INT8, or either FP8 format): s = absmax /
        // (largest code value), one fp32 scale per (slot, group)
        constexpr int LPG = G / EPL;            // lanes per group
        constexpr int NG = D / G;
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            a = fmaxf(a, __builtin_fabsf(x[i]));
#pragma unroll
        for (int o = 1; o < LPG; o <<= 1)
            a = fmaxf(a, __shfl_xor(a, o));
        constexpr float kMaxCode =
            FMT == FMT_INT8 ? 127.0f : (FMT == FMT_INT4 ? 7.0f : fp8_max<FMT>());
        const float s = a / kMaxCode;           // IEEE division (correctly rounded)
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            if constexpr (FMT == FMT_INT8 || FMT == FMT_INT4) {
                float q = 0.0f;
                if (s != 0.0f) {
                    q = __builtin_rintf(x[i] / s);  // round half to even
                    q = fminf(fmaxf(q, -kMaxCode), kMaxCode);
                }
                // stored in excess-128 (INT8) / excess-8 (INT4) form
                code[i] = (uint32_t)((int32_t)q + (FMT == FMT_INT8 ? 128 : 8));
            } else {
                code[i] = s != 0.0f ? fp8_rne_sat<FMT>(x[i] / s) : 0u;
            }
        }
        if ((lane & (LPG - 1)) == 0) {
            float *sc = is_v ? p.v_scale : p.k_scale;
            sc[(head_base * BS + off) * NG + (e0 / G)] = s;
        }
    } else if constexpr (FMT == FMT_INT8) {
        // static per-channel scales [Hkv][D]; a zero scale gives code 0
        const float *S = (is_v ? p.v_scale : p.k_scale) + (int64_t)h * D + e0;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            float q = 0.0f;
            if (S[i] != 0.0f) {
                q = __builtin_rintf(x[i] / S[i]);
                q = fminf(fmaxf(q, -127.0f), 127.0f);
            }
            code[i] = (uint32_t)((int32_t)q + 128);
        }
    } else if constexpr (FMT == FMT_FP8 || FMT == FMT_E5M2) {
        // static per-head scale
        const float S = (is_v ? p.v_scale : p.k_scale)[h];
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            code[i] = S != 0.0f ? fp8_rne_sat<FMT>(x[i] / S) : 0u;  // zero scale: code 0
    }

    if constexpr (FMT == FMT_INT4) {
        // nibble layouts: see int4_k_byte / int4_v_byte (kvq_device.hpp).  A
        // K dword holds the 4 low-nibble dims of the even lane of a pair and
        // the 4 high-nibble dims of the odd one; a V byte holds two dims of
        // this token.
        static_assert(D == 128 && EPL == 4, "INT4 tiles are laid out for head_dim 128");
        uint8_t *tile = (is_v ? p.v_pool : p.k_pool) + head_base * ((int64_t)BS * 64);
        uint32_t pc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            pc[i] = (uint32_t)__shfl_xor((int)code[i], 1);
        if (!is_v) {
            if ((lane & 1) == 0) {
                uint32_t wv = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    wv |= (code[j] | (pc[j] << 4)) << (8 * j);
                *reinterpret_cast<uint32_t *>(tile + int4_k_byte(off, e0)) = wv;
            }
        } else {
            tile[int4_v_byte(off, e0)] = (uint8_t)(code[0] | (code[1] << 4));
            tile[int4_v_byte(off, e0 + 2)] = (uint8_t)(code[2] | (code[3] << 4));
        }
        return;
    }

    // Tile layouts: see k_offset / v_offset (kvq_device.hpp).
    constexpr int EB = FMT == FMT_FP16 ? 2 : 1;
    uint8_t *tile = (is_v ? p.v_pool : p.k_pool) + head_base * ((int64_t)BS * D * EB);
    if (!is_v) {
        // EPL consecutive dims of one token are contiguous in a K row
        uint8_t *dst = tile + k_offset<D, EB>(BS, off, e0);
        if constexpr (FMT == FMT_FP16) {
            if constexpr (EPL == 4)
                *reinterpret_cast<uint2 *>(dst) = make_uint2(raw[0], raw[1]);
            else
                *reinterpret_cast<uint32_t *>(dst) = raw[0];
        } else if constexpr (EPL == 4) {
            *reinterpret_cast<uint32_t *>(dst) =
                code[0] | (code[1] << 8) | (code[2] << 16) | (code[3] << 24);
        } else {
            *reinterpret_cast<uint16_t *>(dst) = (uint16_t)(code[0] | (code[1] << 8));
        }
    } else {
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            uint8_t *dst = tile + v_offset<D, EB>(BS, off, e0 + i);
            if constexpr (FMT == FMT_FP16)
                *reinterpret_cast<f16 *>(dst) = bit_cast<f16x2>(raw[i / 2])[i % 2];
            else
                *dst = (uint8_t)code[i];
        }
    }
}

// Whole-block copy for copy-on-write: codes of every slot (K and V) and, for
// INT8, the scales of every slot.  blockIdx.x = pair, grid-stride over bytes.
struct CopyParams {
    const int32_t *pairs;
    uint8_t *k_pool;
    uint8_t *v_pool;
    float *k_scale;
    float *v_scale;
    int64_t block_bytes;        // bytes of one block in one pool
    int64_t scale_block_floats; // floats of one block in one scale array (0: none)
    int32_t num_blocks;
};

__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyParams p)
{
    const int32_t src = p.pairs[2 * blockIdx.x];
    const int32_t dst = p.pairs[2 * blockIdx.x + 1];
    if (src < 0 || dst < 0 || src >= p.num_blocks || dst >= p.num_blocks || src == dst)
        return;
    const int64_t n16 = p.block_bytes / 16;
    const int64_t stride = (int64_t)blockDim.x * gridDim.y;
    for (int64_t i = (int64_t)blockIdx.y * blockDim.x + threadIdx.x; i < n16; i += stride) {
        const uint4 *ks = reinterpret_cast<const uint4 *>(p.k_pool + src * p.block_bytes);
        uint4 *kd = reinterpret_cast<uint4 *>(p.k_pool + dst * p.block_bytes);
        const uint4 *vs = reinterpret_cast<const uint4 *>(p.v_pool + src * p.block_bytes);
        uint4 *vd = reinterpret_cast<uint4 *>(p.v_pool + dst * p.block_bytes);
        kd[i] = ks[i];
        vd[i] = vs[i];
    }
    for (int64_t i = (int64_t)blockIdx.y * blockDim.x + threadIdx.x; i < p.scale_block_floats; i += stride) {
        p.k_scale[dst * p.scale_block_floats + i] = p.k_scale[src * p.scale_block_floats + i];
        p.v_scale[dst * p.scale_block_floats + i] = p.v_scale[src * p.scale_block_floats + i];
    }
}

// Swap of whole blocks between the pools and a caller-owned staging buffer
// (device memory, or pinned host memory the GPU writes and reads across the
// bus): preemption moves a sequence's blocks out and back in, possibly to
// other physical blocks (xpshop.cn article 312, s3 and s6: under memory
// pressure a low-priority request is preempted, its KV swapped out and
// brought back later).
// One swap slot holds [K codes][V codes][K scales][V scales] of one block
// (scales only for per-group formats).  pairs[2i] = pool block, pairs[2i+1]
// = swap slot; blockIdx.x = pair, grid-stride over 16-byte units.
struct SwapParams {
    const int32_t *pairs;
    uint8_t *k_pool;
    uint8_t *v_pool;
    uint8_t *k_scale;           // per-group scale arrays as bytes (or null)
    uint8_t *v_scale;
    uint8_t *buf;
    int64_t block_bytes;        // codes of one block in one pool
    int64_t scale_bytes;        // scales of one block in one scale array
    int64_t slot_bytes;         // one swap slot
    int64_t num_slots;
    int32_t num_blocks;
    int32_t to_buffer;          // 1: pools -> buffer, 0: buffer -> pools
};

__global__ __launch_bounds__(256) void swap_blocks_kernel(SwapParams p)
{
    const int32_t blk = p.pairs[2 * blockIdx.x];
    const int32_t slot = p.pairs[2 * blockIdx.x + 1];
    if (blk < 0 || blk >= p.num_blocks || slot < 0 || slot >= p.num_slots)
        return;
    uint8_t *base = p.buf + (int64_t)slot * p.slot_bytes;
    uint8_t *pool_ptr[4] = {p.k_pool + blk * p.block_bytes, p.v_pool + blk * p.block_bytes,
                            p.k_scale ? p.k_scale + blk * p.scale_bytes : nullptr,
                            p.v_scale ? p.v_scale + blk * p.scale_bytes : nullptr};
    const int64_t len[4] = {p.block_bytes, p.block_bytes, p.k_scale ? p.scale_bytes : 0,
                            p.v_scale ? p.scale_bytes : 0};
    int64_t off = 0;
    const int64_t stride = (int64_t)blockDim.x * gridDim.y;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        uint4 *pool16 = reinterpret_cast<uint4 *>(pool_ptr[r]);
        uint4 *buf16 = reinterpret_cast<uint4 *>(base + off);
        for (int64_t i = (int64_t)blockIdx.y * blockDim.x + threadIdx.x; i < len[r] / 16;
             i += stride) {
            if (p.to_buffer)
                buf16[i] = pool16[i];
            else
                pool16[i] = buf16[i];
        }
        off += len[r];
    }
}

}  // namespace kvq
