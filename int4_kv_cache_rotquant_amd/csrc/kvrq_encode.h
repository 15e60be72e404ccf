// Row encoder of the rotated INT4 cache, shared by the write kernel and the fused decode
// step: block Walsh-Hadamard rotation + token-wise INT4 quantisation of one 128-channel
// (token, head) row held by a quad of lanes (32 channels each), stored into its page
// (SAW-INT4: K~ = quant(K H_blk), V~ = quant(V H_blk); wispaper.ai blog, section 3 core
// formula, and section 2 for the block-diagonal matrix).
//
// Bit-exactness: every step runs in IEEE binary32 in a fixed order -- butterfly widths
// 1, 2, 4, ... with (u+w, u-w), then * fp32(1/sqrt b); exact min/max; correctly rounded
// (mx-mn)/15 and 1/scale; round-to-nearest-even binary16 parameters; codes from the
// stored parameters.  The compiler contracts nothing here; the explicit multiply-adds are
// exact (a product by +-1 in the butterflies) or the correction step of the division.
#pragma once

#include <hip/hip_runtime.h>

#include "kvrq_internal.h"

namespace kvrq {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// fp32 value of 1/sqrt(b), the rotation's normalisation.
template <int B> struct InvSqrt;
template <> struct InvSqrt<16> { static constexpr float value = 0x1p-2f; };
template <> struct InvSqrt<32> { static constexpr float value = 0x1.6a09e6p-3f; };
template <> struct InvSqrt<64> { static constexpr float value = 0x1p-3f; };
template <> struct InvSqrt<128> { static constexpr float value = 0x1.6a09e6p-4f; };

// DPP quad permutes: value of lane ql^1 / ql^2 within the quad.
__device__ __forceinline__ float quad_swap1(float x)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float quad_swap2(float x)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
}

__device__ __forceinline__ void bf16x8_to_f32(const u32x4 &w, float *x)
{
    const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        x[2 * m] = __uint_as_float(d[m] << 16);
        x[2 * m + 1] = __uint_as_float(d[m] & 0xFFFF0000u);
    }
}

// Block Walsh-Hadamard transform of a row, this lane's 32 channels.
template <int B>
__device__ __forceinline__ void rotate_row(float (&x)[32], int ql)
{
#pragma clang fp contract(off)
    if constexpr (B > 1) {
        constexpr int in_lane = B < 32 ? B : 32;
#pragma unroll
        for (int h = 1; h < in_lane; h <<= 1) {
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                if (i & h)
                    continue;
                const float u = x[i];
                const float w = x[i + h];
                x[i] = u + w;
                x[i + h] = u - w;
            }
        }
        if constexpr (B >= 64) {
            // width 32: the lower lane keeps u + w, the upper lane u - w (= partner - self)
            const float sgn = (ql & 1) ? -1.0f : 1.0f;
#pragma unroll
            for (int i = 0; i < 32; ++i)
                x[i] = __builtin_fmaf(x[i], sgn, quad_swap1(x[i]));
        }
        if constexpr (B >= 128) {
            const float sgn = (ql & 2) ? -1.0f : 1.0f;
#pragma unroll
            for (int i = 0; i < 32; ++i)
                x[i] = __builtin_fmaf(x[i], sgn, quad_swap2(x[i]));
        }
#pragma unroll
        for (int i = 0; i < 32; ++i)
            x[i] = x[i] * InvSqrt<B>::value;
    }
}

// Stores of the encoded rows: non-temporal (NT) for the write kernel, whose output is not
// read back by it (measured on MI355X: the 32k-token chunk write 37.7 -> 35.6 us, and the
// 1M-token decode that follows 64 such writes 234 -> 205 us, since the fill no longer leaves
// the Infinity Cache full of dirty lines); plain for the fused decode step, whose workgroup
// reads its rows back.
template <bool NT, typename T>
__device__ __forceinline__ void store_row(T *p, const T &v)
{
    if constexpr (NT)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

// One staged tile of 16 rows (the write kernel's LDS staging): each lane's code piece (16
// bytes; 8 at 2 bits), and per row the parameter word and the destination cell
// (0xFFFFFFFF: nothing to store; no real cell has that index, since a pool of 2^32 cells
// would need 256 GiB for one tensor's 4-bit codes alone).
struct StageSlot {
    u32x4 piece[64];
    uint32_t par[16];
    uint32_t cell[16];
};

// Rotate, quantise and store one row held in x; called by all four lanes of the quad.
// 4 bits: 15 levels, two codes per byte, 64-byte rows; 2 bits: 3 levels, four codes per
// byte (channel d at bit 2 (d % 4) of byte d / 4), 32-byte rows.  BITS fixes the width at
// compile time (4 or 2); BITS = 0 takes it from `bits` at run time.  NT: non-temporal code
// stores (the parameter words are always stored plainly).  With `stage`, nothing is stored:
// the encoded tile goes to that LDS slot, and the caller stores it later.
template <int B, int BITS = 4, bool NT = false>
__device__ __forceinline__ void encode_row(float (&x)[32], int32_t slot, uint8_t *__restrict__ codes,
                                           uint32_t *__restrict__ params, int64_t num_slots,
                                           int num_kv_heads, int page_log2, int h, int ql,
                                           int bits = 4, StageSlot *stage = nullptr)
{
#pragma clang fp contract(off)
    static_assert(BITS == 4 || BITS == 2 || BITS == 0, "code widths: 4, 2, or run time");
    const bool two = BITS == 2 || (BITS == 0 && bits == 2);
    rotate_row<B>(x, ql);

    float mn = x[0], mx = x[0];
#pragma unroll
    for (int i = 1; i < 32; ++i) {
        mn = fminf(mn, x[i]);
        mx = fmaxf(mx, x[i]);
    }
    mn = fminf(mn, quad_swap1(mn));
    mx = fmaxf(mx, quad_swap1(mx));
    mn = fminf(mn, quad_swap2(mn));
    mx = fmaxf(mx, quad_swap2(mx));
    mn = mn + 0.0f;  // a zero minimum is stored as +0
    mx = mx + 0.0f;

    // scale32 = (mx - mn) / levels correctly rounded, as q0 = x r plus one FMA correction
    // step (r = fp32(1 / levels)): three instructions instead of a full IEEE division, and
    // equal to the division for every non-negative finite binary32 x at levels 15 and 3
    // (checked exhaustively, all 2^31 values of x, by tests/test_write_arithmetic.py)
    const float levels = two ? 3.0f : 15.0f;
    const float rlev = two ? 0x1.555556p-2f : 0x1.111112p-4f;
    const float range = mx - mn;
    const float q0 = range * rlev;
    float scale32 = __builtin_fmaf(__builtin_fmaf(-q0, levels, range), rlev, q0);
    // keep the binary32 rounding of the scale: the compiler would otherwise fold the
    // conversion below into the multiply-add (v_fma_mixlo_f16, one rounding to fp16 instead
    // of fp32 then fp16)
    asm volatile("" : "+v"(scale32));
    const _Float16 s16 = (_Float16)scale32;
    const _Float16 z16 = (_Float16)mn;
    const uint32_t s_bits = __builtin_bit_cast(uint16_t, s16);
    const uint32_t z_bits = __builtin_bit_cast(uint16_t, z16);

    const bool store = slot >= 0 && slot < num_slots;
    const int64_t page = slot >> page_log2;
    const int64_t off = slot & ((1 << page_log2) - 1);
    const int64_t cell = ((page * num_kv_heads + h) << page_log2) + off;
    if (two) {
        uint32_t out[2] = {0u, 0u};
        if (s_bits != 0u) {
            const float zf = (float)z16;
            const float inv = 1.0f / (float)s16;
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                uint32_t byte[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    uint32_t acc = 0u;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float v = (x[16 * k + 4 * m + e] - zf) * inv;
                        // clamp to [0, 3], then round half to even as for 4 bits; the
                        // integer sits in bits 0..1, bits 2..21 are zero
                        const float c = __builtin_amdgcn_fmed3f(v, 0.0f, 3.0f) + 12582912.0f;
                        acc |= __float_as_uint(c) << (2 * e);
                    }
                    byte[m] = acc;
                }
                const uint32_t lo = __builtin_amdgcn_perm(byte[1], byte[0], 0x0C0C0400u);
                const uint32_t hi = __builtin_amdgcn_perm(byte[3], byte[2], 0x0C0C0400u);
                out[k] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
            }
        }
        if (stage != nullptr) {
            const int ln = threadIdx.x & 63;
            stage->piece[ln] = u32x4{out[0], out[1], 0u, 0u};
            if (ql == 0) {
                stage->par[ln >> 2] = s_bits | (z_bits << 16);
                stage->cell[ln >> 2] = store ? (uint32_t)cell : 0xFFFFFFFFu;
            }
            return;
        }
        if (store) {
            u32x2 *dst = reinterpret_cast<u32x2 *>(codes + cell * (kRowCodeBytes / 2)) + ql;
            store_row<NT>(dst, u32x2{out[0], out[1]});
            if (ql == 0)
                store_row<false>(params + cell, s_bits | (z_bits << 16));
        }
        return;
    }
    uint32_t out[4] = {0u, 0u, 0u, 0u};
    if (s_bits != 0u) {
        const float zf = (float)z16;
        const float inv = 1.0f / (float)s16;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            // clamp to [0, 15], then v_cvt_pk_u8_f32 rounds half to even (saturating at 0)
            // into byte m: the even channels' codes go to `ev`, the odd channels' to `od`,
            // and byte m of the word is code(2m) | code(2m + 1) << 4
            uint32_t ev = 0u, od = 0u;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const float v0 = (x[8 * k + 2 * m] - zf) * inv;
                const float v1 = (x[8 * k + 2 * m + 1] - zf) * inv;
                ev = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_amdgcn_fmed3f(v0, 0.0f, 15.0f), m, ev);
                od = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_amdgcn_fmed3f(v1, 0.0f, 15.0f), m, od);
            }
            out[k] = ev | (od << 4);
        }
    }
    if (stage != nullptr) {
        const int ln = threadIdx.x & 63;
        stage->piece[ln] = u32x4{out[0], out[1], out[2], out[3]};
        if (ql == 0) {
            stage->par[ln >> 2] = s_bits | (z_bits << 16);
            stage->cell[ln >> 2] = store ? (uint32_t)cell : 0xFFFFFFFFu;
        }
        return;
    }
    if (store) {
        u32x4 *dst = reinterpret_cast<u32x4 *>(codes + cell * kRowCodeBytes) + ql;
        store_row<NT>(dst, u32x4{out[0], out[1], out[2], out[3]});
        // the parameters always as plain stores: a tile's 16 words fill half a 128-byte line
        // whose other half a neighbouring wave writes, and the L2 merges the two halves
        // before the line goes to memory (the Qwen3-4B-like write, page 16: -4%)
        if (ql == 0)
            store_row<false>(params + cell, s_bits | (z_bits << 16));
    }
}

}  // namespace
}  // namespace kvrq
