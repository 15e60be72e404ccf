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
// Launch 1 -- decode_split_kernel, one workgroup of four 64-lane waves per
// (split, KV head, sequence); each wave walks a quarter of the split's tokens
// in 32-token tiles, the next tile's loads in flight while one is consumed:
//   QK^T  S[t][g] = sum_d code_K[t][d] q[d][g] on int8 MFMA 16x16x64: A = the
//         INT4 codes as bytes, B = the G (<= 16) rotated queries rounded to a
//         21-bit integer grid and cut into three int8 digits, so the products
//         are exact integers; score = scale_t * 2^-f * S + zero_t * sum(q')
//         (de-quantisation factored out of the dot product);
//   softmax online, in base 2 (log2 e is folded into q'), with a lazy maximum;
//   PV    O'[d][g] += sum_t (code_V[t][d] - 8) (p_t scale_t), plus
//         sum_t p_t (zero_t + 8 scale_t), on f16 MFMA 16x16x32 with the codes
//         as exact centred f16 integers and the weights split into f16 high
//         and low parts.
// Lane (n16, kq) keeps query head g = n16, so the softmax state needs no
// cross-lane exchange except for the per-tile maxima.  The four waves' states
// are merged in LDS into one split partial (o, m, l).
// Launch 2 -- decode_combine_kernel, one workgroup per (query head, sequence):
// log-sum-exp combine of the splits, then the inverse V rotation.
#include <hip/hip_runtime.h>

#include "kvrq_internal.h"

namespace kvrq {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

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

// V codes become f16 MFMA operands: a nibble masked in place and OR-ed into the
// f16 pattern 0x6400 (= 1024) is the exact f16 integer 1024 + code (bits 0-3) or
// 1024 + 16 code (bits 4-7); one packed subtraction centres it to code - 8 (times
// 16 for the upper nibble).  Normal f16 operands keep the matrix cores' full
// accumulation precision, and centred codes keep the weighted sums small.
constexpr uint32_t kLoNib = 0x000F000Fu;
constexpr uint32_t kHiNib = 0x00F000F0u;

__device__ __forceinline__ uint32_t centred_codes(uint32_t masked, bool upper)
{
    const f16x2 v = __builtin_bit_cast(f16x2, masked | 0x64006400u);
    const _Float16 c = upper ? (_Float16)1152.0f : (_Float16)1032.0f;
    return __builtin_bit_cast(uint32_t, v - f16x2{c, c});
}

// K codes become int8 MFMA operands: the even and the odd nibbles of a dword, masked
// in place, are four bytes each.  Scores are integer dot products of codes with the
// query quantised to 22 bits (three int8 slices), exact in the int32 accumulators.
constexpr uint32_t kNibBytes = 0x0F0F0F0Fu;

// Lazy softmax maximum (base 2): weights exp2(score - m) may grow to 2^kLazyMax before
// the reference max m moves and the accumulators are rescaled.
constexpr float kLazyMax = 8.0f;

__device__ __forceinline__ i32x4 mfma_i8(const i32x4 &a, const i32x4 &b, const i32x4 &c)
{
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16x16x32(const f16x8 &a, const f16x8 &b, const f32x4 &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float wave_xor(float x, int m)
{
    return __shfl_xor(x, m, 64);
}

// One 32-token tile of one (sequence, KV head) as this lane loads it.
//   kc[hf]  16 code bytes of token t0 + 16 hf + n16, channels [32 kq, 32 kq + 32)
//   vc      code dword n16 (channels 8 n16 .. 8 n16 + 7) of tokens t0 + 16 hf + 4 kq + r
//   par     lanes 0..31: (scale, zero) of K for token t0 + lane; lanes 32..63: the same
//           for V (token t0 + lane - 32); redistributed through LDS when the tile is used
struct Tile {
    u32x4 kc[2];
    uint32_t vc[8];
    uint32_t par;
};

// Lane byte offsets inside one 16-token half tile of a (page, head): constant for the
// whole loop, so the loads are a scalar (uniform) base plus a 32-bit lane offset.
struct LaneOffsets {
    uint32_t kc;   // n16 * 64 + 16 kq into the K codes
    uint32_t vc;   // 4 kq * 64 + 4 n16 into the V codes; + 64 r for token 4 kq + r
    uint32_t par;  // 4 (lane % 16) into the parameters of the lane's half tile
};

__device__ __forceinline__ void load_tile(Tile &T, const DecodeArgs &a, const int32_t *ptab, int h,
                                          int t0, int t_end, const LaneOffsets &o, int lane)
{
    const int P = 1 << a.page_log2;
    const bool v_lane = lane >= 32;
    const int my_half = (lane >> 4) & 1;
    T.par = 0u;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        const int tb = t0 + 16 * hf;
        if (tb < t_end) {
            int page = ptab[tb >> a.page_log2];
            page = (unsigned)page < (unsigned)a.num_pages ? page : 0;
            const int64_t cell0 = ((int64_t)page * a.num_kv_heads + h) * P + (tb & (P - 1));
            const uint8_t *kc = a.k_codes + cell0 * kRowCodeBytes;
            const uint8_t *vc = a.v_codes + cell0 * kRowCodeBytes;
            T.kc[hf] = *reinterpret_cast<const u32x4 *>(kc + o.kc);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                T.vc[4 * hf + r] = *reinterpret_cast<const uint32_t *>(vc + o.vc + 64 * r);
            if (my_half == hf) {
                const uint32_t *pp = v_lane ? a.v_params + cell0 : a.k_params + cell0;
                T.par = *reinterpret_cast<const uint32_t *>(reinterpret_cast<const uint8_t *>(pp) + o.par);
            }
        } else {
            T.kc[hf] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int r = 0; r < 4; ++r)
                T.vc[4 * hf + r] = 0u;
        }
    }
}

// B operand of QK^T in lane order: the query quantised to int32 q = round(q' * 2^f)
// (|q| < 2^21) and cut into int8 digits q = 2^16 hi + 2^8 mid + lo.  Element e of
// k-step ks for lane (n16, kq) is the digit of channel 32 kq + 8 (e / 4) + 2 (e % 4) + ks.
struct QOperand {
    i32x4 v[2][3][64];   // [k-step][hi, mid, lo][lane]
};

// Online-softmax state of one wave: lane (n16, kq) keeps query head g = n16.
struct WaveState {
    float kscale;               // 2^-f: integer dot products back to the query's scale
    float qsum;                 // sum of the rotated, scaled query (for the zero points)
    float m, l, z;              // running max (base 2), partial sums of p and p * zero_V
    int E;                      // weights enter the PV product as p * scale_V * 2^E
    f32x4 acc[8];               // O'[d][g] * 2^E, d = 8 (4 kq + r) + b, centred codes
                                // (x16 for odd b)

    __device__ __forceinline__ void consume(const Tile &T, int t0, int t_end, int lane,
                                            const QOperand &qop, uint32_t *par_lds)
    {
        const int kq = lane >> 4;
        const bool full = t0 + kTile <= t_end;   // uniform: no masking inside full tiles
        // parameters of the lane's 8 tokens, K then V: [0..31] K of tokens 0..31, [32..63] V
        // (lanes of one wave exchange through LDS; LDS operations of a wave complete in order)
        par_lds[lane] = T.par;
        __builtin_amdgcn_wave_barrier();
        const u32x4 kp0 = *reinterpret_cast<const u32x4 *>(par_lds + 4 * kq);
        const u32x4 kp1 = *reinterpret_cast<const u32x4 *>(par_lds + 16 + 4 * kq);
        const u32x4 vp0 = *reinterpret_cast<const u32x4 *>(par_lds + 32 + 4 * kq);
        const u32x4 vp1 = *reinterpret_cast<const u32x4 *>(par_lds + 48 + 4 * kq);

        // ---- a8: scores of tokens t0 + 16 hf + 4 kq + r ---------------------------------
        float Sd[8];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const u32x4 w = T.kc[hf];
            const i32x4 ev = {int32_t(w.x & kNibBytes), int32_t(w.y & kNibBytes),
                              int32_t(w.z & kNibBytes), int32_t(w.w & kNibBytes)};
            const i32x4 od = {int32_t((w.x >> 4) & kNibBytes), int32_t((w.y >> 4) & kNibBytes),
                              int32_t((w.z >> 4) & kNibBytes), int32_t((w.w >> 4) & kNibBytes)};
            i32x4 dg[3];
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                dg[j] = mfma_i8(ev, qop.v[0][j][lane], i32x4{0, 0, 0, 0});
                dg[j] = mfma_i8(od, qop.v[1][j][lane], dg[j]);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Sd[4 * hf + r] = (float)(dg[0][r] * 256 + dg[1][r]) * 256.0f + (float)dg[2][r];
        }
        float sc[8], sv[8], zv[8];
        const uint32_t kpw[8] = {kp0.x, kp0.y, kp0.z, kp0.w, kp1.x, kp1.y, kp1.z, kp1.w};
        const uint32_t vpw[8] = {vp0.x, vp0.y, vp0.z, vp0.w, vp1.x, vp1.y, vp1.z, vp1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const f16x2 kpar = __builtin_bit_cast(f16x2, kpw[i]);
            const f16x2 vpar = __builtin_bit_cast(f16x2, vpw[i]);
            const float score = Sd[i] * ((float)kpar.x * kscale) + (float)kpar.y * qsum;
            const float vs = (float)vpar.x;
            const float vz = (float)vpar.y + 8.0f * vs;   // zero point of the centred codes
            if (full) {
                sc[i] = score;
                sv[i] = vs;
                zv[i] = vz;
            } else {
                const bool ok = t0 + 16 * (i >> 2) + 4 * kq + (i & 3) < t_end;
                sc[i] = ok ? score : -INFINITY;
                sv[i] = ok ? vs : 0.0f;
                zv[i] = ok ? vz : 0.0f;
            }
        }

        // ---- a9: online softmax (base 2); accumulators rescaled only when a max moved ------
        float tmax = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])),
                           fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
        tmax = fmaxf(tmax, wave_xor(tmax, 16));
        tmax = fmaxf(tmax, wave_xor(tmax, 32));
        // The reference max moves only when a score exceeds it by more than kLazyMax (base
        // 2), so the accumulators are rarely rescaled; weights stay below 2^kLazyMax.
        const bool moved = tmax > m + kLazyMax;
        const float m_new = moved ? tmax : m;
        const float alpha = moved ? __builtin_amdgcn_exp2f(m - m_new) : 1.0f;
        m = m_new;
        // Weight exponent: the f16 high and low parts of p * scale_V * 2^E keep ~22 bits only
        // while the low part stays a normal f16, so E puts the tile's largest possible weight
        // (p <= 2^kLazyMax) just below 2^14.  E only decreases; the accumulators follow
        // exactly.
        float smax = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                           fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
        smax = fmaxf(smax, wave_xor(smax, 16));
        smax = fmaxf(smax, wave_xor(smax, 32));
        float acc_f = alpha;
        bool e_moved = false;
        if (smax > 0.0f) {
            int ex;
            frexpf(smax, &ex);
            const int e_tile = 14 - (int)kLazyMax - ex;
            if (e_tile < E) {                      // uniform across the wave
                acc_f = ldexpf(alpha, e_tile - E);
                E = e_tile;
                e_moved = true;
            }
        }
        float psum = 0.0f, pz = 0.0f;
        f16x8 pb_hi, pb_lo;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float p = __builtin_amdgcn_exp2f(sc[i] - m_new);
            psum += p;
            pz += p * zv[i];
            const float w = p * ldexpf(sv[i], E);
            const _Float16 hi = (_Float16)w;
            pb_hi[i] = hi;
            pb_lo[i] = (_Float16)(w - (float)hi);
        }
        l = l * alpha + psum;
        z = z * alpha + pz;
        if (__builtin_amdgcn_ballot_w64(moved) || e_moved) {
#pragma unroll
            for (int b = 0; b < 8; ++b)
                acc[b] *= acc_f;
        }

        // ---- PV: A = V codes (rows: channel 8 n16 + b, k: the 8 tokens), B = p * scale -----
        uint32_t src[4][4];   // [lo bytes, lo >> 8, hi bytes, hi >> 8][token pair]
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            src[0][p] = __builtin_amdgcn_perm(T.vc[2 * p + 1], T.vc[2 * p], 0x05040100u);
            src[2][p] = __builtin_amdgcn_perm(T.vc[2 * p + 1], T.vc[2 * p], 0x07060302u);
            src[1][p] = src[0][p] >> 8;
            src[3][p] = src[2][p] >> 8;
        }
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const uint32_t *sp = src[b >> 1];
            const bool upper = b & 1;
            const uint32_t mask = upper ? kHiNib : kLoNib;
            const u32x4 r = {centred_codes(sp[0] & mask, upper), centred_codes(sp[1] & mask, upper),
                             centred_codes(sp[2] & mask, upper), centred_codes(sp[3] & mask, upper)};
            const f16x8 va = __builtin_bit_cast(f16x8, r);
            acc[b] = mfma16x16x32(va, pb_hi, acc[b]);
            acc[b] = mfma16x16x32(va, pb_lo, acc[b]);
        }
    }
};

template <int BK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3)))
void decode_split_kernel(DecodeArgs a)
{
    const int split = blockIdx.x;
    const int h = blockIdx.y;
    const int s = blockIdx.z;
    const int L = min(a.seq_lens[s], a.max_seq_len);
    const int wg_begin = split * a.split_tokens;
    if (wg_begin >= L)
        return;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // the wave index, and with it the token range, is uniform across the wave: keep it
    // scalar so the page-table lookups and the loop control stay on the scalar unit
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = a.group;
    const int wave_tokens = a.split_tokens / kDecodeWaves;
    const int t_begin = wg_begin + wave * wave_tokens;
    const int t_end = min(L, t_begin + wave_tokens);

    // rotated query rows in the prologue, the four waves' states in the epilogue
    __shared__ float lds_o[kDecodeWaves][kMaxGroup][kHeadDim + 4];
    __shared__ QOperand qop;
    __shared__ uint32_t lds_par[kDecodeWaves][64];
    __shared__ float lds_m[kDecodeWaves][kMaxGroup];
    __shared__ float lds_l[kDecodeWaves][kMaxGroup];
    __shared__ float lds_qsum[kMaxGroup];
    __shared__ float lds_kscale[kMaxGroup];
    float(*q_lds)[kHeadDim + 4] = lds_o[0];

    // ---- a6: wave 0 rotates the G queries of this KV head, folds sm_scale * log2(e) ---------
    if (wave == 0) {
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
        // power-of-two factor 2^f placing the largest |q' * 2^f| in [2^20, 2^21)
        int e = 0;
        if (amax > 0.0f)
            frexpf(amax, &e);
#pragma unroll
        for (int i = 0; i < 32; ++i)
            q_lds[g][32 * ql + i] = ldexpf(x[i], 21 - e);
        if (ql == 0) {
            lds_qsum[g] = sum;
            lds_kscale[g] = ldexpf(1.0f, e - 21);
        }
    }
    __syncthreads();

    // B operands of QK^T: int8 digits of the quantised query in lane order
    for (int i = tid; i < 2 * 64; i += 64 * kDecodeWaves) {
        const int ks = i >> 6, ln = i & 63;
        const int n = ln & 15, q4 = ln >> 4;
        uint32_t dig[3][4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            dig[0][j] = dig[1][j] = dig[2][j] = 0u;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int32_t q = (int32_t)rintf(q_lds[n][32 * q4 + 8 * (e >> 2) + 2 * (e & 3) + ks]);
            const int32_t lo = ((q + 128) & 255) - 128;
            const int32_t r1 = (q - lo) >> 8;
            const int32_t mid = ((r1 + 128) & 255) - 128;
            const int32_t hi = (r1 - mid) >> 8;
            const int sh = 8 * (e & 3);
            dig[0][e >> 2] |= uint32_t(hi & 255) << sh;
            dig[1][e >> 2] |= uint32_t(mid & 255) << sh;
            dig[2][e >> 2] |= uint32_t(lo & 255) << sh;
        }
#pragma unroll
        for (int j = 0; j < 3; ++j)
            qop.v[ks][j][ln] = i32x4{int32_t(dig[j][0]), int32_t(dig[j][1]), int32_t(dig[j][2]), int32_t(dig[j][3])};
    }
    const int n16 = lane & 15;
    const int kq = lane >> 4;
    WaveState st;
    st.qsum = lds_qsum[n16];
    st.kscale = lds_kscale[n16];
    st.m = -INFINITY;
    st.l = 0.0f;
    st.z = 0.0f;
    st.E = 64;
#pragma unroll
    for (int b = 0; b < 8; ++b)
        st.acc[b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    __syncthreads();   // q_lds is reused below, qop is complete

    // ---- a7: page walk, one tile ahead of the math --------------------------------------
    const int32_t *ptab = a.page_table + (int64_t)s * a.max_pages;
    if (t_begin < t_end) {
        const LaneOffsets off = {uint32_t(n16 * kRowCodeBytes + 16 * kq),
                                 uint32_t(4 * kq * kRowCodeBytes + 4 * n16), uint32_t(4 * (lane & 15))};
        uint32_t *par_lds = lds_par[wave];
        Tile A, B;
        load_tile(A, a, ptab, h, t_begin, t_end, off, lane);
        int t0 = t_begin;
        while (true) {
            bool more = t0 + kTile < t_end;
            if (more)
                load_tile(B, a, ptab, h, t0 + kTile, t_end, off, lane);
            st.consume(A, t0, t_end, lane, qop, par_lds);
            t0 += kTile;
            if (!more)
                break;
            more = t0 + kTile < t_end;
            if (more)
                load_tile(A, a, ptab, h, t0 + kTile, t_end, off, lane);
            st.consume(B, t0, t_end, lane, qop, par_lds);
            t0 += kTile;
            if (!more)
                break;
        }
    }

    // ---- combine the four waves' states of this split -------------------------------------
    st.l += wave_xor(st.l, 16);
    st.l += wave_xor(st.l, 32);
    st.z += wave_xor(st.z, 16);
    st.z += wave_xor(st.z, 32);
    if (n16 < G) {
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const float unit = ldexpf((b & 1) ? 0.0625f : 1.0f, -st.E);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                lds_o[wave][n16][32 * kq + 8 * r + b] = st.acc[b][r] * unit + st.z;
        }
        if (kq == 0) {
            lds_m[wave][n16] = st.m;
            lds_l[wave][n16] = st.l;
        }
    }
    __syncthreads();
    for (int i = tid; i < G * kHeadDim; i += 64 * kDecodeWaves) {
        const int g = i >> 7, d = i & (kHeadDim - 1);
        float M = lds_m[0][g];
#pragma unroll
        for (int w = 1; w < kDecodeWaves; ++w)
            M = fmaxf(M, lds_m[w][g]);
        float o = 0.0f, lsum = 0.0f;
#pragma unroll
        for (int w = 0; w < kDecodeWaves; ++w) {
            const float f = lds_m[w][g] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(lds_m[w][g] - M);
            o += f * lds_o[w][g][d];
            lsum += f * lds_l[w][g];
        }
        const int64_t row = ((int64_t)s * a.num_q_heads + h * G + g) * a.max_splits + split;
        a.part_o[row * kHeadDim + d] = o;
        if (d == 0) {
            a.part_ml[2 * row] = M;
            a.part_ml[2 * row + 1] = lsum;
        }
    }
}

// ---- a10: combine the splits of one (sequence, query head), undo the V rotation ---------
template <int BV>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a)
{
    const int g = blockIdx.x;
    const int s = blockIdx.y;
    const int tid = threadIdx.x;
    const int L = min(a.seq_lens[s], a.max_seq_len);
    float *out = a.out + ((int64_t)s * a.num_q_heads + g) * kHeadDim;
    if (L <= 0) {
        if (tid < kHeadDim)
            out[tid] = 0.0f;
        return;
    }
    const int n = (L + a.split_tokens - 1) / a.split_tokens;
    const int64_t row0 = ((int64_t)s * a.num_q_heads + g) * a.max_splits;
    const float *ml = a.part_ml + 2 * row0;

    __shared__ float red[8];
    __shared__ float part[8][kHeadDim];

    // global max and normaliser over the splits
    float M = -INFINITY;
    for (int i = tid; i < n; i += 256)
        M = fmaxf(M, ml[2 * i]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        M = fmaxf(M, wave_xor(M, o));
    if ((tid & 63) == 0)
        red[tid >> 6] = M;
    __syncthreads();
    M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    float l = 0.0f;
    for (int i = tid; i < n; i += 256)
        l += __builtin_amdgcn_exp2f(ml[2 * i] - M) * ml[2 * i + 1];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        l += wave_xor(l, o);
    __syncthreads();
    if ((tid & 63) == 0)
        red[4 + (tid >> 6)] = l;
    __syncthreads();
    l = red[4] + red[5] + red[6] + red[7];

    // weighted sum of the partial outputs: thread = (split residue sub, 4 channels)
    const int sub = tid >> 5, dq = tid & 31;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    const float *po = a.part_o + row0 * kHeadDim + 4 * dq;
    for (int i = sub; i < n; i += 8) {
        const float w = __builtin_amdgcn_exp2f(ml[2 * i] - M);
        acc += w * *reinterpret_cast<const f32x4 *>(po + (int64_t)i * kHeadDim);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
        part[sub][4 * dq + j] = acc[j];
    __syncthreads();
    if (tid >= 64)
        return;
    const float inv_l = 1.0f / l;
    float o0 = 0.0f, o1 = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        o0 += part[k][2 * tid];
        o1 += part[k][2 * tid + 1];
    }
    o0 *= inv_l;
    o1 *= inv_l;
    const int lane = tid;
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
    hipLaunchKernelGGL(decode_split_kernel<BK>, grid, dim3(64 * kDecodeWaves), 0, s, a);
    return hipGetLastError();
}

template <int BV>
hipError_t launch_combine(const DecodeArgs &a, hipStream_t s)
{
    const dim3 grid((unsigned)a.num_q_heads, (unsigned)a.num_seqs);
    hipLaunchKernelGGL(decode_combine_kernel<BV>, grid, dim3(256), 0, s, a);
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
