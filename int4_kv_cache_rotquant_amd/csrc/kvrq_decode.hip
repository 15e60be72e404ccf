// Split-K paged decode attention over the rotated INT4 cache, for gfx950.
//
// SAW-INT4 keeps attention fused over the paged cache (fugumt.com abstract:
// fused attention execution is one of the serving constraints; wispaper.ai
// blog, section 1: decode relies on FlashAttention-style kernels and extra
// per-element decoding work costs registers and speed).  The query is rotated
// with the K block matrix so its dot product with the rotated keys is the
// original one (wispaper.ai blog, section 3, third consequence); V is stored
// rotated, so the output is rotated back once at the end (H is symmetric and
// orthonormal, hence its own inverse).
//
// Launch 1 -- decode_split_kernel, one 64-lane wave per (split, KV head,
// sequence).  The wave walks its token range in 32-token tiles:
//   QK^T  S[t][g] = sum_d (code_K[t][d] - 8) q''[d][g] on MFMA 16x16x32 (f16
//         in, f32 accumulate): A = the INT4 codes of 16 tokens turned into
//         exact centred f16 integers, B = the G (<= 16) rotated queries split
//         into f16 high and low parts (two MFMAs) so the product keeps ~22
//         mantissa bits; score = scale_t * S + (zero_t + 8 scale_t) * sum(q')
//         (de-quantisation factored out of the dot product);
//   softmax online, in base 2 (log2 e is folded into q');
//   PV    O'[d][g] += sum_t (code_V[t][d] - 8) (p_t scale_t), plus
//         sum_t p_t (zero_t + 8 scale_t), again on MFMA with the weights split
//         into f16 high and low parts.
// Each lane keeps one query head g = lane % 16, so the softmax state and the
// 32 output channels a lane accumulates never need a cross-lane exchange
// except for the per-tile maximum.
// Launch 2 -- decode_combine_kernel, one wave per (query head, sequence):
// log-sum-exp combine of the splits, then the inverse V rotation.
#include <hip/hip_runtime.h>

#include "kvrq_internal.h"

namespace kvrq {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int B> struct InvSqrtF;
template <> struct InvSqrtF<16> { static constexpr float value = 0x1p-2f; };
template <> struct InvSqrtF<32> { static constexpr float value = 0x1.6a09e6p-3f; };
template <> struct InvSqrtF<64> { static constexpr float value = 0x1p-3f; };
template <> struct InvSqrtF<128> { static constexpr float value = 0x1.6a09e6p-4f; };

__device__ __forceinline__ float dpp_quad_swap1(float x)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_quad_swap2(float x)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
}

// Query rotation: a quad holds one query row, lane ql the channels
// [32 ql, 32 ql + 32); widths up to 16 in-lane, 32 and 64 across the quad.
template <int B>
__device__ __forceinline__ void rotate_query(float (&x)[32], int ql)
{
    if constexpr (B > 1) {
        constexpr int in_lane = B < 32 ? B : 32;
#pragma unroll
        for (int h = 1; h < in_lane; h <<= 1) {
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                if (i & h)
                    continue;
                const float u = x[i], w = x[i + h];
                x[i] = u + w;
                x[i + h] = u - w;
            }
        }
        if constexpr (B >= 64) {
            const float sgn = (ql & 1) ? -1.0f : 1.0f;
#pragma unroll
            for (int i = 0; i < 32; ++i)
                x[i] = __builtin_fmaf(x[i], sgn, dpp_quad_swap1(x[i]));
        }
        if constexpr (B >= 128) {
            const float sgn = (ql & 2) ? -1.0f : 1.0f;
#pragma unroll
            for (int i = 0; i < 32; ++i)
                x[i] = __builtin_fmaf(x[i], sgn, dpp_quad_swap2(x[i]));
        }
#pragma unroll
        for (int i = 0; i < 32; ++i)
            x[i] *= InvSqrtF<B>::value;
    }
}

// Two codes n as centred f16 integers n - 8: OR-ing a nibble into 0x6400 gives the f16
// value 1024 + n, and subtracting 1032 is exact.  Centring keeps the code sums small, so
// code * scale and the zero term do not cancel in the fp32 accumulators; the zero point
// moves to zero + 8 * scale.
__device__ __forceinline__ uint32_t nibbles_to_f16x2(uint32_t masked)
{
    const f16x2 v = __builtin_bit_cast(f16x2, masked | 0x64006400u);
    const f16x2 r = v - f16x2{(_Float16)1032.0f, (_Float16)1032.0f};
    return __builtin_bit_cast(uint32_t, r);
}

// 8 K codes of one dword (channels c..c+7) as MFMA operand elements in the
// order (c, c+4, c+1, c+5, c+2, c+6, c+3, c+7).
__device__ __forceinline__ f16x8 k_operand(uint32_t w)
{
    u32x4 r;
    r.x = nibbles_to_f16x2(w & 0x000F000Fu);
    r.y = nibbles_to_f16x2((w >> 4) & 0x000F000Fu);
    r.z = nibbles_to_f16x2((w >> 8) & 0x000F000Fu);
    r.w = nibbles_to_f16x2((w >> 12) & 0x000F000Fu);
    return __builtin_bit_cast(f16x8, r);
}

__device__ __forceinline__ f32x4 mfma16x16x32(const f16x8 &a, const f16x8 &b, const f32x4 &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float wave_xor(float x, int m)
{
    return __shfl_xor(x, m, 64);
}

template <int BK>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeArgs a)
{
    const int split = blockIdx.x;
    const int h = blockIdx.y;
    const int s = blockIdx.z;
    const int L = min(a.seq_lens[s], a.max_seq_len);
    const int t_begin = split * a.split_tokens;
    if (t_begin >= L)
        return;
    const int t_end = min(L, t_begin + a.split_tokens);
    const int lane = threadIdx.x;
    const int G = a.group;

    __shared__ float q_lds[kMaxGroup][kHeadDim + 4];
    __shared__ float qsum_lds[kMaxGroup];
    __shared__ float qinv_lds[kMaxGroup];

    // ---- a6: rotate the G queries of this KV head, fold sm_scale * log2(e) -------------
    {
        const int g = lane >> 2, ql = lane & 3;
        float x[32];
        if (g < G) {
            const u32x4 *src = reinterpret_cast<const u32x4 *>(
                a.q + ((int64_t)s * a.num_q_heads + h * G + g) * kHeadDim + 32 * ql);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const u32x4 w = src[j];
                const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    x[8 * j + 2 * m] = __uint_as_float(d[m] << 16);
                    x[8 * j + 2 * m + 1] = __uint_as_float(d[m] & 0xFFFF0000u);
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < 32; ++i)
                x[i] = 0.0f;
        }
        rotate_query<BK>(x, ql);
        float amax = 0.0f, sum = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            x[i] *= a.q_scale;
            amax = fmaxf(amax, fabsf(x[i]));
            sum += x[i];
        }
        amax = fmaxf(amax, dpp_quad_swap1(amax));
        amax = fmaxf(amax, dpp_quad_swap2(amax));
        sum += dpp_quad_swap1(sum);
        sum += dpp_quad_swap2(sum);
        // power-of-two factor placing the largest |q''| in [2^14, 2^15): the f16 high part
        // then has full precision and the low part stays out of the f16 subnormal range
        float f = 1.0f;
        if (amax > 0.0f) {
            int e;
            frexpf(amax, &e);
            f = ldexpf(1.0f, 15 - e);
        }
#pragma unroll
        for (int i = 0; i < 32; ++i)
            q_lds[g][32 * ql + i] = x[i] * f;
        if (ql == 0) {
            qsum_lds[g] = sum;
            qinv_lds[g] = 1.0f / f;
        }
    }
    __syncthreads();

    const int n16 = lane & 15;  // MFMA row/column owned by this lane: query head g, token, or channel row
    const int kq = lane >> 4;   // MFMA k-slice of this lane
    f16x8 qb_hi[4], qb_lo[4];
    {
        const int perm[8] = {0, 4, 1, 5, 2, 6, 3, 7};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v = q_lds[n16][32 * kq + 8 * ks + perm[e]];
                const _Float16 hi = (_Float16)v;
                qb_hi[ks][e] = hi;
                qb_lo[ks][e] = (_Float16)(v - (float)hi);
            }
        }
    }
    const float qsum = qsum_lds[n16];
    const float qinv = qinv_lds[n16];

    float m_run = -INFINITY, l_run = 0.0f, z_run = 0.0f;
    f32x4 acc[8];
#pragma unroll
    for (int b = 0; b < 8; ++b)
        acc[b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    const int P = 1 << a.page_log2;
    const int32_t *ptab = a.page_table + (int64_t)s * a.max_pages;

    for (int t0 = t_begin; t0 < t_end; t0 += kTile) {
        // ---- a7: page walk, this tile's codes and parameters -----------------------------
        u32x4 kc[2];
        uint32_t vc[8];
        u32x4 kp[2], vp[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int tb = t0 + 16 * hf;
            if (tb < t_end) {
                int page = ptab[tb >> a.page_log2];
                page = (unsigned)page < (unsigned)a.num_pages ? page : 0;
                const int64_t cell0 = ((int64_t)page * a.num_kv_heads + h) * P + (tb & (P - 1));
                kc[hf] = *reinterpret_cast<const u32x4 *>(a.k_codes + (cell0 + n16) * kRowCodeBytes + 16 * kq);
                kp[hf] = *reinterpret_cast<const u32x4 *>(a.k_params + cell0 + 4 * kq);
                vp[hf] = *reinterpret_cast<const u32x4 *>(a.v_params + cell0 + 4 * kq);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    vc[4 * hf + r] = *reinterpret_cast<const uint32_t *>(
                        a.v_codes + (cell0 + 4 * kq + r) * kRowCodeBytes + 4 * n16);
            } else {
                kc[hf] = u32x4{0u, 0u, 0u, 0u};
                kp[hf] = u32x4{0u, 0u, 0u, 0u};
                vp[hf] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    vc[4 * hf + r] = 0u;
            }
        }

        // ---- a8: scores of tokens t0 + 16 hf + 4 kq + r for query head g = n16 -----------
        float sc[8], sv[8], zv[8];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            f32x4 d = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            const uint32_t kw[4] = {kc[hf].x, kc[hf].y, kc[hf].z, kc[hf].w};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const f16x8 ka = k_operand(kw[ks]);
                d = mfma16x16x32(ka, qb_hi[ks], d);
                d = mfma16x16x32(ka, qb_lo[ks], d);
            }
            const uint32_t kpw[4] = {kp[hf].x, kp[hf].y, kp[hf].z, kp[hf].w};
            const uint32_t vpw[4] = {vp[hf].x, vp[hf].y, vp[hf].z, vp[hf].w};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tok = t0 + 16 * hf + 4 * kq + r;
                const f16x2 kpar = __builtin_bit_cast(f16x2, kpw[r]);
                const f16x2 vpar = __builtin_bit_cast(f16x2, vpw[r]);
                const float ks_ = (float)kpar.x, vs_ = (float)vpar.x;
                const float score = d[r] * (ks_ * qinv) + ((float)kpar.y + 8.0f * ks_) * qsum;
                const bool ok = tok < t_end;
                sc[4 * hf + r] = ok ? score : -INFINITY;
                sv[4 * hf + r] = ok ? vs_ : 0.0f;
                zv[4 * hf + r] = ok ? (float)vpar.y + 8.0f * vs_ : 0.0f;
            }
        }

        // ---- a9: online softmax (base 2) ----------------------------------------------
        float tmax = sc[0];
#pragma unroll
        for (int i = 1; i < 8; ++i)
            tmax = fmaxf(tmax, sc[i]);
        tmax = fmaxf(tmax, wave_xor(tmax, 16));
        tmax = fmaxf(tmax, wave_xor(tmax, 32));
        const float m_new = fmaxf(m_run, tmax);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        float psum = 0.0f, pz = 0.0f;
        f16x8 pb_hi, pb_lo;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float p = __builtin_amdgcn_exp2f(sc[i] - m_new);
            psum += p;
            pz += p * zv[i];
            const float w = p * sv[i];
            const _Float16 hi = (_Float16)w;
            pb_hi[i] = hi;
            pb_lo[i] = (_Float16)(w - (float)hi);
        }
        l_run = l_run * alpha + psum;
        z_run = z_run * alpha + pz;
#pragma unroll
        for (int b = 0; b < 8; ++b)
            acc[b] *= alpha;

        // ---- PV: A = V codes (rows: channel 8 n16 + b, k: tokens), B = p * scale ----------
        uint32_t lo4[4], hi4[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            lo4[p] = __builtin_amdgcn_perm(vc[2 * p + 1], vc[2 * p], 0x05040100u);
            hi4[p] = __builtin_amdgcn_perm(vc[2 * p + 1], vc[2 * p], 0x07060302u);
        }
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const int sh = 4 * (b & 3);
            u32x4 r;
            const uint32_t *src = b < 4 ? lo4 : hi4;
            r.x = nibbles_to_f16x2((src[0] >> sh) & 0x000F000Fu);
            r.y = nibbles_to_f16x2((src[1] >> sh) & 0x000F000Fu);
            r.z = nibbles_to_f16x2((src[2] >> sh) & 0x000F000Fu);
            r.w = nibbles_to_f16x2((src[3] >> sh) & 0x000F000Fu);
            const f16x8 va = __builtin_bit_cast(f16x8, r);
            acc[b] = mfma16x16x32(va, pb_hi, acc[b]);
            acc[b] = mfma16x16x32(va, pb_lo, acc[b]);
        }
    }

    // ---- partials: o'[d] (d = 8 (4 kq + r) + b), running max and sum ----------------------
    l_run += wave_xor(l_run, 16);
    l_run += wave_xor(l_run, 32);
    z_run += wave_xor(z_run, 16);
    z_run += wave_xor(z_run, 32);
    if (n16 < G) {
        const int64_t row = ((int64_t)s * a.num_q_heads + h * G + n16) * a.max_splits + split;
        float *dst = a.part_o + row * kHeadDim + 32 * kq;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            f32x4 lo = f32x4{acc[0][r], acc[1][r], acc[2][r], acc[3][r]} + z_run;
            f32x4 hi = f32x4{acc[4][r], acc[5][r], acc[6][r], acc[7][r]} + z_run;
            *reinterpret_cast<f32x4 *>(dst + 8 * r) = lo;
            *reinterpret_cast<f32x4 *>(dst + 8 * r + 4) = hi;
        }
        if (kq == 0) {
            a.part_ml[2 * row] = m_run;
            a.part_ml[2 * row + 1] = l_run;
        }
    }
}

// ---- a10: combine the splits of one (sequence, query head), undo the V rotation ---------
template <int BV>
__global__ __launch_bounds__(64) void decode_combine_kernel(DecodeArgs a)
{
    const int g = blockIdx.x;
    const int s = blockIdx.y;
    const int lane = threadIdx.x;
    const int L = min(a.seq_lens[s], a.max_seq_len);
    float *out = a.out + ((int64_t)s * a.num_q_heads + g) * kHeadDim;
    if (L <= 0) {
        out[2 * lane] = 0.0f;
        out[2 * lane + 1] = 0.0f;
        return;
    }
    const int n = (L + a.split_tokens - 1) / a.split_tokens;
    const int64_t row0 = ((int64_t)s * a.num_q_heads + g) * a.max_splits;
    const float *ml = a.part_ml + 2 * row0;

    float M = -INFINITY;
    for (int i = lane; i < n; i += 64)
        M = fmaxf(M, ml[2 * i]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        M = fmaxf(M, wave_xor(M, o));
    float l = 0.0f;
    for (int i = lane; i < n; i += 64)
        l += __builtin_amdgcn_exp2f(ml[2 * i] - M) * ml[2 * i + 1];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        l += wave_xor(l, o);

    float o0 = 0.0f, o1 = 0.0f;
    const float *po = a.part_o + row0 * kHeadDim + 2 * lane;
    for (int i = 0; i < n; ++i) {
        const float w = __builtin_amdgcn_exp2f(ml[2 * i] - M);
        const float2 v = *reinterpret_cast<const float2 *>(po + (int64_t)i * kHeadDim);
        o0 += w * v.x;
        o1 += w * v.y;
    }
    const float inv_l = 1.0f / l;
    o0 *= inv_l;
    o1 *= inv_l;

    if constexpr (BV > 1) {
        // lane holds channels 2 lane, 2 lane + 1: width 1 in-lane, widths 2.. across lanes
        float u = o0 + o1, w = o0 - o1;
        o0 = u;
        o1 = w;
#pragma unroll
        for (int hw = 2; hw < BV; hw <<= 1) {
            const int m = hw >> 1;
            const float p0 = wave_xor(o0, m), p1 = wave_xor(o1, m);
            const bool upper = lane & m;
            o0 = upper ? p0 - o0 : o0 + p0;
            o1 = upper ? p1 - o1 : o1 + p1;
        }
        o0 *= InvSqrtF<BV>::value;
        o1 *= InvSqrtF<BV>::value;
    }
    *reinterpret_cast<float2 *>(out + 2 * lane) = make_float2(o0, o1);
}

template <int BK>
hipError_t launch_split(const DecodeArgs &a, hipStream_t s)
{
    const dim3 grid((unsigned)a.max_splits, (unsigned)a.num_kv_heads, (unsigned)a.num_seqs);
    hipLaunchKernelGGL(decode_split_kernel<BK>, grid, dim3(64), 0, s, a);
    return hipGetLastError();
}

template <int BV>
hipError_t launch_combine(const DecodeArgs &a, hipStream_t s)
{
    const dim3 grid((unsigned)a.num_q_heads, (unsigned)a.num_seqs);
    hipLaunchKernelGGL(decode_combine_kernel<BV>, grid, dim3(64), 0, s, a);
    return hipGetLastError();
}

}  // namespace

int launch_decode(int k_block, int v_block, const DecodeArgs &a, void *stream)
{
    if (a.num_seqs == 0)
        return 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    switch (k_block) {
    case 0: e = launch_split<0>(a, s); break;
    case 16: e = launch_split<16>(a, s); break;
    case 32: e = launch_split<32>(a, s); break;
    case 64: e = launch_split<64>(a, s); break;
    case 128: e = launch_split<128>(a, s); break;
    default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess)
        return e;
    switch (v_block) {
    case 0: return launch_combine<0>(a, s);
    case 16: return launch_combine<16>(a, s);
    case 32: return launch_combine<32>(a, s);
    case 64: return launch_combine<64>(a, s);
    case 128: return launch_combine<128>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace kvrq
