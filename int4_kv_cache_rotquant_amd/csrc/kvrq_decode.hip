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
// (split, KV head, sequence) (sequences vary fastest when the whole grid is resident, so
// a sequence's workgroups share one XCD) -- for the extend, per (row block, KV head,
// split).  The four waves first prepare the query operands together (16 lanes per row),
// then share the split's 32-token tiles evenly, the next tiles' loads in flight while
// one is consumed:
//   QK^T  S[t][c] = sum_d code_K[t][d] q[d][c] on int8 MFMA 16x16x64: A = the
//         INT4 codes as bytes, B = the rotated queries of the MFMA columns rounded to
//         a 21-bit integer grid and cut into three int8 digits, so the products are
//         exact integers; score = scale_t * 2^-f * S + zero_t * sum(q') (the
//         de-quantisation factored out of the dot product);
//   softmax online, in base 2 (log2 e is folded into q'), with a lazy maximum;
//   PV    O'[d][c] += sum_t code_V[t][d] (p_t scale_t) + sum_t p_t zero_t, on f16
//         MFMA 16x16x32 with the codes placed in f16 mantissas (1 + code / 16 or
//         / 64, the constant part taken out of the sums) and the weights split into
//         f16 high and low parts.
// Columns: G <= 8 query heads take two columns each, one per 16-token half of every
// tile (F = 2); otherwise 16 columns of single heads, or, for the extend, query rows x
// heads in two blocks of 16 per wave (F = 1).  The four waves' states are merged in LDS
// into one split partial (o, m, l) -- or, when one split covers the rows, normalised,
// rotated back and written as the output directly.
// 2-bit tiles (mixed-precision caches) are loaded at half size and widened to the
// byte-per-code layout as they are consumed.  In the fused decode step, the workgroup
// whose split holds a sequence's last position first encodes and stores the new
// token's K/V rows (the write kernel's encoding), then reads them back with the rest.
// The log-sum-exp combine of the splits, then the inverse V rotation: in the split launch
// when its grid is resident at once and a row has at most 16 splits (the last split of
// each (sequence, KV head) to finish, elected by a counter in the workspace, merges
// them); otherwise launch 2: decode_combine_wave_kernel (one wave per (row, query head))
// for up to 64 splits, decode_combine_kernel (a 16-wave workgroup per (row, query head))
// beyond.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "kvrq_encode.h"
#include "kvrq_internal.h"

namespace kvrq {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float dpp_row_ror8(float x)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, false));
}

// DPP moves inside a 16-lane row: partner lane seg ^ 1, ^ 2, ^ 4, ^ 8.
__device__ __forceinline__ float dpp_xor1(float x) { return quad_swap1(x); }
__device__ __forceinline__ float dpp_xor2(float x) { return quad_swap2(x); }
__device__ __forceinline__ float dpp_xor4(float x)
{
    // reverse the quad (lane ^ 3), then mirror the half row (lane ^ 7)
    const int r = __builtin_amdgcn_mov_dpp(__float_as_int(x), 0x1B, 0xF, 0xF, true);
    return __int_as_float(__builtin_amdgcn_mov_dpp(r, 0x141, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_xor8(float x) { return dpp_row_ror8(x); }

template <int M>
__device__ __forceinline__ float dpp_xor(float x)
{
    if constexpr (M == 1)
        return dpp_xor1(x);
    else if constexpr (M == 2)
        return dpp_xor2(x);
    else if constexpr (M == 4)
        return dpp_xor4(x);
    else
        return dpp_xor8(x);
}

__device__ __forceinline__ float row16_sum(float x)
{
    x += dpp_xor1(x);
    x += dpp_xor2(x);
    x += dpp_xor4(x);
    return x + dpp_xor8(x);
}

__device__ __forceinline__ float row16_max(float x)
{
    x = fmaxf(x, dpp_xor1(x));
    x = fmaxf(x, dpp_xor2(x));
    x = fmaxf(x, dpp_xor4(x));
    return fmaxf(x, dpp_xor8(x));
}

// One butterfly stage of width 8 M across lanes seg and seg ^ M: the lower lane keeps
// u + w, the upper one u - w.
template <int M>
__device__ __forceinline__ void butterfly_across(float (&x)[8], int seg)
{
    const float sgn = (seg & M) ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        x[i] = __builtin_fmaf(x[i], sgn, dpp_xor<M>(x[i]));
}

// Query rotation: 16 lanes hold one query row, lane seg the channels [8 seg, 8 seg + 8);
// widths 1, 2, 4 in-lane, 8 .. 64 across the row, in the order of increasing width.
template <int B>
__device__ __forceinline__ void rotate_query_row(float (&x)[8], int seg)
{
    if constexpr (B > 1) {
        constexpr int in_lane = B < 8 ? B : 8;
#pragma unroll
        for (int h = 1; h < in_lane; h <<= 1) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (i & h)
                    continue;
                const float u = x[i], w = x[i + h];
                x[i] = u + w;
                x[i + h] = u - w;
            }
        }
        if constexpr (B >= 16)
            butterfly_across<1>(x, seg);
        if constexpr (B >= 32)
            butterfly_across<2>(x, seg);
        if constexpr (B >= 64)
            butterfly_across<4>(x, seg);
        if constexpr (B >= 128)
            butterfly_across<8>(x, seg);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            x[i] *= InvSqrt<B>::value;
    }
}

__device__ __forceinline__ float wave_xor(float x, int m)
{
    return __shfl_xor(x, m, 64);
}

// Maximum and sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48, which hold the 16
// tokens of one MFMA column between them (gfx950 row permutes: swap the upper 32
// lanes, then the odd 16-lane rows, with the same register).
__device__ __forceinline__ float max_raw(float a, float b)
{
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

__device__ __forceinline__ float col_max(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = max_raw(__uint_as_float(r[0]), __uint_as_float(r[1]));
    r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return max_raw(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float col_sum(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// V codes become f16 MFMA operands without arithmetic: a nibble moved into mantissa bits
// 6..9 under the exponent of 1.0 is the exact f16 value 1 + code / 16 (a high nibble left
// in bits 4..7: 1 + code / 64).  The accumulators are re-centred every kRecentre tiles by
// the weight sum of those tiles (1 + c / 16 - 1.5 = (c - 8) / 16, 1 + c / 64 - 1.125 =
// (c - 8) / 64), so they hold small centred sums and keep their precision.  The zero
// point then becomes zero + 8 scale: sum_t p_t (c_t s_t + z_t) = sum_t p_t s_t (c_t - 8)
// + sum_t p_t z_t + 8 sum_t p_t s_t.
constexpr int kRecentre = 8;
constexpr uint32_t kOne2 = 0x3C003C00u;     // f16x2 {1, 1}
constexpr uint32_t kMant47 = 0x00F000F0u;   // mantissa bits 4..7 of both halves

// Word 3 of a raw buffer resource on gfx9-family chips (32-bit data format, no swizzle).
constexpr int kBufferWord3 = 0x00020000;

// Cache policy of the decode's code loads: non-temporal ("nt"): the cache is read once per
// decode, and a streaming read runs at 7.0 TB/s with nt loads on MI355X against 6.3 with the
// default policy.  With two tiles really in flight per wave (walk_tiles) the Qwen3-32B-like
// decode went 610 -> 569 us.  (The extend keeps default-policy loads: its row blocks re-read
// a sequence's tiles from the L2.)
constexpr int kTileLoadAux = 2;

// K codes become int8 MFMA operands: the even and the odd nibbles of a dword, masked in
// place, are four bytes each.  Scores are integer dot products of codes with the query
// rounded to a 21-bit grid (three int8 digits), exact in the int32 accumulators.
constexpr uint32_t kNibBytes = 0x0F0F0F0Fu;

// Lazy softmax maximum (base 2): weights exp2(score - m) may grow to 2^kLazyMax before
// the reference max m moves and the accumulators are rescaled.
constexpr float kLazyMax = 8.0f;

// Running maximum before any score has been seen (finite, far below any real score).
constexpr float kNoScore = -1.0e30f;

__device__ __forceinline__ i32x4 mfma_i8(const i32x4 &a, const i32x4 &b, const i32x4 &c)
{
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16x16x32(const f16x8 &a, const f16x8 &b, const f32x4 &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Tokens are handled in tiles of 32.  Two layouts of the QK^T product:
//   F = 1 (9..16 query heads per KV head): a 16x16x64 MFMA covers 16 tokens x 16 heads
//         x 64 k (32 channels, one nibble parity); lane (n16, kq) ends with the scores of
//         head n16 for tokens 16 hf + 4 kq + r (8 per lane);
//   F = 2 (up to 8 heads): the same MFMAs, one pair of nibble steps per 16-token half,
//         but B columns 8..15 are zero in the first half's steps and columns 0..7 in the
//         second's, so both halves accumulate into one result: 32 tokens x 8 heads;
//         lane (n16, kq) ends with the scores of head n16 % 8 for tokens 4 kq + r + 16
//         (n16 / 8) (4 per lane) and keeps its own softmax state for that half of the
//         tile (merged at the end).
// One 32-token tile as this lane loads it (every load instruction reads from one page, at
// a scalar base and a per-lane offset that does not change from tile to tile):
//   kc[j]   16 code bytes of token 16 j + n16, bytes [16 kq, 16 kq + 16)
//   vc[j]   code dword n16 (channels 8 n16 .. 8 n16 + 7) of token 16 (j / 4) + 4 kq + j % 4
//   par     lanes 0..31: (scale, zero) of K of token lane; lanes 32..63: V of token
//           lane - 32; converted and shared through LDS when the tile is consumed
// 2-bit pools (CB bit 0: K, bit 1: V) load half the bytes:
//   kc[j].xy  8 code bytes of token 16 j + n16, bytes [8 kq, 8 kq + 8) (channels
//             32 kq .. 32 kq + 31 as for 4 bits)
//   vc[j]     the 16-bit code word n16 (channels 8 n16 .. 8 n16 + 7)
// and widen them to the 4-bit layout when the tile is consumed (spread2), so the rest of
// the pipeline is the same: a 2-bit code is a 4-bit code below 4 with the same meaning.
template <int CB> struct CodeWidths {
    static constexpr bool k2 = (CB & 1) != 0;
    static constexpr bool v2 = (CB & 2) != 0;
    static constexpr int k_row = k2 ? kRowCodeBytes / 2 : kRowCodeBytes;
    static constexpr int v_row = v2 ? kRowCodeBytes / 2 : kRowCodeBytes;
};

template <int CB>
struct Tile {
    using KWords = std::conditional_t<CodeWidths<CB>::k2, u32x2, u32x4>;
    KWords kc[2];
    uint32_t vc[8];
    uint32_t par;
};

// Eight 2-bit codes (bits 2i of a 16-bit value) -> eight 4-bit codes (bits 4i).
__device__ __forceinline__ uint32_t spread2(uint32_t x)
{
    x = (x | (x << 8)) & 0x00FF00FFu;
    x = (x | (x << 4)) & 0x0F0F0F0Fu;
    return (x | (x << 2)) & 0x33333333u;
}

// The K code words of one half tile in the 4-bit layout (2-bit words widened).
__device__ __forceinline__ u32x4 k_nibbles(const u32x4 &k) { return k; }
__device__ __forceinline__ u32x4 k_nibbles(const u32x2 &k)
{
    return u32x4{spread2(k.x & 0xFFFFu), spread2(k.x >> 16), spread2(k.y & 0xFFFFu),
                 spread2(k.y >> 16)};
}

// Issues the loads of the tile starting at t0 (< t_end).  A half tile that starts past
// the end re-reads the first half's rows: every load is in bounds and unconditional, and
// tokens past the end are removed by their parameters (zero) and score bias (-inf).
// Page ids of a window of 128 consecutive pages of a sequence, two per lane, so a tile's
// pages come from readlane instead of a scalar load whose latency every tile would wait for.
// The window moves on by 64 pages when a tile reaches past it.  The ids of the 64 pages after
// the window are requested one move ahead, raw: a load whose value is used right away (the
// range checks) makes the wave wait for every load in flight, its tiles included, while these
// are only checked and moved into the window at the next move, 64 pages later, by which time
// the tile waits in between have retired them (measured on MI355X, same machine: the extend
// 1,255 -> 1,251 us; the decodes, whose tile in flight is mostly back by a move, unchanged
// within 0.1%).
struct PageIds {
    int first;   // page index held by lane 0 of `id` (uniform)
    int id;      // lane j: page id of page index first + j (out-of-range ids read as 0)
    int next;    // lane j: page id of page index first + 64 + j
    int ahead;   // lane j: table entry of page index first + 128 + j, unchecked

    __device__ __forceinline__ static int check(const DecodeArgs &a, int v, int k)
    {
        return k < a.max_pages && (unsigned)v < (unsigned)a.num_pages ? v : 0;
    }
    // the table entry of page index k (k >= 0), read in bounds whatever k is
    __device__ __forceinline__ static int raw(const DecodeArgs &a, const int32_t *ptab, int k)
    {
        return ptab[min(k, a.max_pages - 1)];
    }
    __device__ __forceinline__ void fill(const DecodeArgs &a, const int32_t *ptab, int first_page,
                                         int lane)
    {
        first = first_page;
        id = check(a, raw(a, ptab, first_page + lane), first_page + lane);
        next = check(a, raw(a, ptab, first_page + 64 + lane), first_page + 64 + lane);
        ahead = raw(a, ptab, first_page + 128 + lane);
    }
    // page indexes up to `last` become reachable (callers ask in increasing order, at most
    // a few pages past the window)
    __device__ __forceinline__ void reach(const DecodeArgs &a, const int32_t *ptab, int last,
                                          int lane)
    {
        if (last - first >= 128) {
            first += 64;
            id = next;
            next = check(a, ahead, first + 64 + lane);
            ahead = raw(a, ptab, first + 128 + lane);
        }
    }
    __device__ __forceinline__ int page(int page_index) const
    {
        const int j = page_index - first;
        const int lo = __builtin_amdgcn_readlane(id, j & 63);
        const int hi = __builtin_amdgcn_readlane(next, j & 63);
        return j < 64 ? lo : hi;
    }
};

// Per-lane parts of the tile addresses, the same for every tile.
struct LaneAddr {
    uint32_t k;   // K code bytes within a (page, head) row block
    uint32_t v;   // V code bytes within a (page, head) row block
    int lane;

    template <int CB>
    __device__ __forceinline__ void init(int lane_)
    {
        using CW = CodeWidths<CB>;
        lane = lane_;
        const uint32_t n16 = lane & 15, kq = lane >> 4;
        k = CW::k2 ? n16 * CW::k_row + 8 * kq : n16 * kRowCodeBytes + 16 * kq;
        v = CW::v2 ? 4 * kq * CW::v_row + 2 * n16 : 4 * kq * kRowCodeBytes + 4 * n16;
    }
};

// A buffer resource for one (page, head) row block: base in scalar registers, so each
// load is that base plus the lane's 32-bit offset, with no 64-bit vector arithmetic per
// tile (offsets stay far below the record limit).
// The base is wave-uniform by construction; reading it through readfirstlane says so, so
// the compiler never wraps the loads in a loop over distinct bases.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_block(const uint8_t *base)
{
    // (readfirstlane returns int: take both halves as unsigned 32-bit values, so the low
    // half is not sign-extended into the high one)
    const uint64_t u = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(((uint64_t)hi << 32) | lo),
                                             (short)0, 0x7FFFFFFF, kBufferWord3);
}

// Loads of one (page, head) row block at a lane offset: through a buffer resource (BUF:
// scalar base, the row step as the scalar offset) or as plain global loads.
template <bool BUF>
struct RowBlock {
    const uint8_t *p;
    __amdgpu_buffer_rsrc_t r;

    __device__ __forceinline__ RowBlock(const uint8_t *base) : p(base)
    {
        if constexpr (BUF)
            r = row_block(base);
    }
    template <typename T>
    __device__ __forceinline__ T load(uint32_t lane_off, int row_off) const
    {
        if constexpr (!BUF)
            return *reinterpret_cast<const T *>(p + lane_off + row_off);
        else if constexpr (sizeof(T) == 16)
            return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(r, (int)lane_off, row_off, kTileLoadAux));
        else if constexpr (sizeof(T) == 8)
            return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b64(r, (int)lane_off, row_off, kTileLoadAux));
        else if constexpr (sizeof(T) == 4)
            return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b32(r, (int)lane_off, row_off, kTileLoadAux));
        else
            return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b16(r, (int)lane_off, row_off, kTileLoadAux));
    }
};

// The decode takes buffer loads; the extend plain loads.  Buffer loads in the extend measured
// no faster with default caching (MI355X, chunked prefill: 1239 against 1238 us) and much
// slower with the decode's non-temporal hint (1316 us): each row block's workgroup re-reads
// its sequence's prefix, which the L2 then no longer holds.
template <int CB, bool BUF>
__device__ __forceinline__ void load_tile(Tile<CB> &T, const DecodeArgs &a, const PageIds &pid, int h,
                                          int t0, int t_end, const LaneAddr &la)
{
    using CW = CodeWidths<CB>;
    const int P = 1 << a.page_log2;
    // The tile's loads stay together, in this order, after the code before the call: loads
    // moved across the consumption of the tile before would leave the in-order load counter
    // unable to tell the two tiles in flight apart, and the wait before each tile would then
    // wait for both (measured: the page walk streamed ~10% slower).  The wave issues them at a
    // raised priority, so they are not held behind the other waves' arithmetic (measured on
    // MI355X, same machine: the Qwen3-32B-like decode 573.2 -> 571.5 us, the 1M-token decode
    // 196.8 -> 196.1 us, the Qwen3-4B-like decode 19.94 -> 19.83 us).
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(2);
    // (page, head) row blocks of the two 16-token halves; uniform, so on the scalar unit
    // (cells, page * Hkv * P + token, are below 2^32)
    uint32_t cell[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        const int tb = hf && t0 + 16 >= t_end ? t0 : t0 + 16 * hf;
        const uint32_t page = (uint32_t)pid.page(tb >> a.page_log2);
        cell[hf] = (page * (uint32_t)a.num_kv_heads + (uint32_t)h) * (uint32_t)P +
                   (uint32_t)(tb & (P - 1));
    }
    // the parameter word of the lane: K (lanes 0..31) or V, first or second half.  Requested
    // ahead of the V codes (loads complete in order), so the tile's consumer converts the
    // parameters while the V codes are still arriving (the Qwen3-32B-like decode 568.8 ->
    // 567.8 us, same machine)
    const bool ph = (la.lane & 16) != 0;
    const uint32_t *kp0 = a.k_params + cell[0], *kp1 = a.k_params + cell[1];
    const uint32_t *vp0 = a.v_params + cell[0], *vp1 = a.v_params + cell[1];
    T.par = *((la.lane < 32 ? (ph ? kp1 : kp0) : (ph ? vp1 : vp0)) + (la.lane & 15));
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        const RowBlock<BUF> kb(a.k_codes + (uint64_t)cell[hf] * CW::k_row);
        T.kc[hf] = kb.template load<typename Tile<CB>::KWords>(la.k, 0);
    }
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        const RowBlock<BUF> vb(a.v_codes + (uint64_t)cell[hf] * CW::v_row);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if constexpr (CW::v2)
                T.vc[4 * hf + r] = vb.template load<uint16_t>(la.v, r * CW::v_row);
            else
                T.vc[4 * hf + r] = vb.template load<uint32_t>(la.v, r * kRowCodeBytes);
        }
    }
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
}

// B operands of QK^T in lane order: the query rounded to integers q = round(q' 2^f)
// (|q| <= 2^20, one f per KV head) and cut into int8 digits q = 2^16 hi + 2^8 mid + lo.
//   F = 1: v[par][digit][lane], element byte e of lane (n16, kq): channel 32 kq + 2 e + par
//          of head n16;
//   F = 2: v[2 j + par][digit][lane]: the same channel, of head n16 % 8, in the steps of
//          half j for the columns of that half (n16 / 8 == j), zero for the others.
template <int F>
struct QOperand {
    i32x4 v[2 * F][3][64];
};

// Parameters of one tile in fp32, per wave: [0] scale (K: times 2^-f), [1] zero,
// [2] score bias (0, or -inf past the end); K of token j at j, V at 32 + j.
struct ParLds {
    float v[3][64];
};

// Online-softmax state of one lane: the MFMA column it belongs to (head n16, or head
// n16 % 8 over one half of each tile when F = 2).
struct WaveState {
    float qsum;                 // sum of the rotated, scaled query (for the zero points)
    float m, l, z;              // running max (base 2), sums of p and p * zero_V
    float wsum;                 // sum of the PV weights w, scaled like acc
    int E;                      // weights enter the PV product as w = p * scale_V * 2^E
    float slim;                 // 2^(6 - E): a V scale this large needs a smaller E
    float wpend;                // this lane's weights since the last re-centring
    int nt;                     // tiles since the last re-centring
    f32x4 acc[8];               // sum_t w_t (code - 8) / u_b, d = 8 (4 kq + r) + b,
                                // u_b = 16 (even b) or 64 (odd b), once re-centred

    // take the constant parts 1.5 w (even b) and 1.125 w (odd b) out of the accumulators
    __device__ __forceinline__ void recentre()
    {
        const float W = col_sum(wpend);
        const float we = -1.5f * W, wo = -1.125f * W;
#pragma unroll
        for (int b = 0; b < 8; ++b)
            acc[b] += (b & 1) ? wo : we;
        wpend = 0.0f;
        nt = 0;
    }

    __device__ __forceinline__ void tick()
    {
        if (++nt == kRecentre)
            recentre();
    }

    // ---- a9: online softmax (base 2) of one tile's scores, the PV weights as f16 high and
    // low B operands
    template <int F>
    // smax: the largest V scale among the lane's tokens (the same for every column block)
    __device__ __forceinline__ void softmax(float (&sc)[8 / F], const float (&sv)[8 / F],
                                            const float (&zv)[8 / F], float smax, int lane,
                                            f16x8 &bh, f16x8 &bl)
    {
        constexpr int NS = 8 / F;            // scores per lane
        const int sub = F == 2 ? ((lane & 15) >> 3) : 0;
        // Most tiles change nothing: the maximum moves only when a score exceeds it by more
        // than kLazyMax, the weight exponent only when a V scale reaches slim = 2^(6 - E).
        // Lanes test their own scores; the column reductions run only when some lane asks.
        float tmax = sc[0];
#pragma unroll
        for (int i = 1; i < NS; ++i)
            tmax = fmaxf(tmax, sc[i]);
        float alpha = 1.0f;
        if (__builtin_amdgcn_ballot_w64(tmax > m + kLazyMax || smax >= slim)) {
            tmax = col_max(tmax);
            smax = col_max(smax);
            const bool moved = tmax > m + kLazyMax;
            const float m_new = moved ? tmax : m;
            alpha = moved ? __builtin_amdgcn_exp2f(m - m_new) : 1.0f;
            m = m_new;
            // weight exponent: the f16 high and low parts of w keep ~22 bits while the low
            // part is a normal f16, so E puts the largest possible weight of the tile
            // (p <= 2^8) just below 2^14; E only decreases, and the accumulators follow
            float acc_f = alpha;
            if (smax >= slim) {
                int ex;
                frexpf(smax, &ex);
                const int e_tile = 14 - (int)kLazyMax - ex;
                acc_f = ldexpf(alpha, e_tile - E);
                E = e_tile;
                slim = ldexpf(1.0f, 14 - (int)kLazyMax - E);
            }
            l *= alpha;
            z *= alpha;
            wsum *= acc_f;
            wpend *= acc_f;
#pragma unroll
            for (int b = 0; b < 8; ++b)
                acc[b] *= acc_f;
        }
        const float m_new = m;
        // p 2^E = exp2(score - (m - E)): the weights come out scaled, the sums of p are
        // scaled back once per tile
        const float mE = m_new - (float)E;
        float psum = 0.0f, pz = 0.0f, ws = 0.0f;
        float w[NS];
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const float pe = __builtin_amdgcn_exp2f(sc[i] - mE);
            psum += pe;
            pz = fmaf(pe, zv[i], pz);
            w[i] = pe * sv[i];
            ws += w[i];
        }
        const float uE = ldexpf(1.0f, -E);
        l = fmaf(psum, uE, l);
        z = fmaf(pz, uE, z);
        wsum += ws;
        wpend += ws;
        // B operand of PV, f16 high and low parts: the high part is w cut to the 11
        // significant bits of an f16 (exact to convert for the weights here, all below
        // 2^14), the low part the exact fp32 remainder rounded to nearest (an unbiased
        // split: the removed constant part of the V operands then adds no drift).  The high
        // part comes from the bits of w, never from a rounding, so no rewrite of the
        // product p * scale by the compiler can make the two parts disagree by an ulp.
        // k slot e of lane (n16, kq) is token 16 (e / 4) + 4 kq + e % 4
        uint32_t hp[NS / 2], lp[NS / 2];
#pragma unroll
        for (int j = 0; j < NS / 2; ++j) {
            const float h0 = __uint_as_float(__float_as_uint(w[2 * j]) & 0xFFFFE000u);
            const float h1 = __uint_as_float(__float_as_uint(w[2 * j + 1]) & 0xFFFFE000u);
            const f16x2 h = {(_Float16)h0, (_Float16)h1};
            const f16x2 r = {(_Float16)(w[2 * j] - h0), (_Float16)(w[2 * j + 1] - h1)};
            hp[j] = __builtin_bit_cast(uint32_t, h);
            lp[j] = __builtin_bit_cast(uint32_t, r);
        }
        u32x4 bhu, blu;
        if constexpr (F == 1) {
            bhu = u32x4{hp[0], hp[1], hp[2], hp[3]};
            blu = u32x4{lp[0], lp[1], lp[2], lp[3]};
        } else {
            bhu = sub ? u32x4{0u, 0u, hp[0], hp[1]} : u32x4{hp[0], hp[1], 0u, 0u};
            blu = sub ? u32x4{0u, 0u, lp[0], lp[1]} : u32x4{lp[0], lp[1], 0u, 0u};
        }
        bh = __builtin_bit_cast(f16x8, bhu);
        bl = __builtin_bit_cast(f16x8, blu);
    }

};

// One tile for NB blocks of 16 MFMA columns (NB > 1: extend, several query rows per wave):
// the parameters, the K operands and the V operands are built once and serve every block.
template <int F, bool EXT, int CB, int NB>
__device__ __forceinline__ void consume_tile(WaveState (&st)[NB], const Tile<CB> &T, int t0, int t_end,
                                             int lane, float kscale, const QOperand<F> *qop,
                                             ParLds &pl, const int (&col_len)[NB], int mask_from)
{
    static_assert(NB == 1 || F == 1, "several column blocks use the 16-column layout");
    constexpr int NS = 8 / F;            // scores per lane
    const int n16 = lane & 15, kq = lane >> 4;
    const int sub = F == 2 ? (n16 >> 3) : 0;

    // parameters: each lane converts one (scale, zero) pair (zero past the end of the
    // range, where the bias also removes the token from the softmax)
    {
        const bool valid = t0 + (lane & 31) < t_end;
        const f16x2 pr = __builtin_bit_cast(f16x2, valid ? T.par : 0u);
        pl.v[0][lane] = (float)pr.x * kscale;
        pl.v[1][lane] = (float)pr.y;
        pl.v[2][lane] = valid ? 0.0f : -INFINITY;
    }
    __builtin_amdgcn_wave_barrier();
    float sk[NS], zk[NS], bk[NS], sv[NS], zv[NS];
#pragma unroll
    for (int j = 0; j < NS / 4; ++j) {
        const int base = 4 * kq + 16 * (F == 2 ? sub : j);
        const f32x4 a0 = *reinterpret_cast<const f32x4 *>(&pl.v[0][base]);
        const f32x4 a1 = *reinterpret_cast<const f32x4 *>(&pl.v[1][base]);
        const f32x4 a2 = *reinterpret_cast<const f32x4 *>(&pl.v[2][base]);
        const f32x4 a3 = *reinterpret_cast<const f32x4 *>(&pl.v[0][32 + base]);
        const f32x4 a4 = *reinterpret_cast<const f32x4 *>(&pl.v[1][32 + base]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            sk[4 * j + r] = a0[r];
            zk[4 * j + r] = a1[r];
            bk[4 * j + r] = a2[r];
            sv[4 * j + r] = a3[r];
            zv[4 * j + r] = a4[r];
        }
    }

    // ---- a8: integer scores -----------------------------------------------------------
    float sc[NB][NS];
    if constexpr (F == 1) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const u32x4 w = k_nibbles(T.kc[hf]);
            const i32x4 ev = __builtin_bit_cast(i32x4, w & kNibBytes);
            const i32x4 od = __builtin_bit_cast(i32x4, (w >> 4) & kNibBytes);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                // digits from the top: each partial sum moves up by 2^8 before the next
                // digit's products are added, ending in the exact int32 dot product
                i32x4 acc = i32x4{0, 0, 0, 0};
#pragma unroll
                for (int d = 0; d < 3; ++d) {
                    if (d)
                        acc <<= 8;
                    acc = mfma_i8(ev, qop[b].v[0][d][lane], acc);
                    acc = mfma_i8(od, qop[b].v[1][d][lane], acc);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sc[b][4 * hf + r] = (float)acc[r];
            }
        }
    } else {
        // the two halves' steps accumulate into one result (B zero outside each half)
        i32x4 dg[3] = {i32x4{0, 0, 0, 0}, i32x4{0, 0, 0, 0}, i32x4{0, 0, 0, 0}};
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const u32x4 w = k_nibbles(T.kc[j]);
            const i32x4 ev = __builtin_bit_cast(i32x4, w & kNibBytes);
            const i32x4 od = __builtin_bit_cast(i32x4, (w >> 4) & kNibBytes);
#pragma unroll
            for (int d = 0; d < 3; ++d) {
                dg[d] = mfma_i8(ev, qop[0].v[2 * j][d][lane], dg[d]);
                dg[d] = mfma_i8(od, qop[0].v[2 * j + 1][d][lane], dg[d]);
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            // two shift-adds; kept apart, the compiler reassociates them into three steps
            int32_t t = (dg[0][r] << 8) + dg[1][r];
            asm("" : "+v"(t));
            sc[0][r] = (float)((t << 8) + dg[2][r]);
        }
    }

    f16x8 bh[NB], bl[NB];
    float smax = sv[0];
#pragma unroll
    for (int i = 1; i < NS; ++i)
        smax = max_raw(smax, sv[i]);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
        for (int i = 0; i < NS; ++i)
            sc[b][i] = fmaf(sc[b][i], sk[i], fmaf(zk[i], st[b].qsum, bk[i]));
        if constexpr (EXT) {
            // causal: token t is visible to the lane's column only if t < col_len
            if (t0 + kTile > mask_from) {
                const int kq4 = 4 * (lane >> 4);
#pragma unroll
                for (int i = 0; i < NS; ++i)
                    sc[b][i] = t0 + 16 * (i >> 2) + kq4 + (i & 3) < col_len[b] ? sc[b][i] : -INFINITY;
            }
        }
        st[b].template softmax<F>(sc[b], sv, zv, smax, lane, bh[b], bl[b]);
    }

    // ---- PV: A = V codes (rows: channel 8 n16 + b, k: the 8 tokens), B = weights -------
    // the high-nibble mask in a scalar register, opaque to constant folding, so that
    // (x & mask) | one is a single v_and_or_b32 (both constants as literals would not
    // fit one instruction and would cost an and and an or)
    uint32_t mant47, one2;
    asm("" : "=s"(mant47) : "0"(kMant47));
    asm("" : "=v"(one2) : "0"(kOne2));
    uint32_t vcode[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        vcode[j] = CodeWidths<CB>::v2 ? spread2(T.vc[j]) : T.vc[j];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        uint32_t src[4];   // byte k of tokens (2p, 2p + 1) in bits 0..7 and 16..23
#pragma unroll
        for (int p = 0; p < 4; ++p)
            src[p] = __builtin_amdgcn_perm(vcode[2 * p + 1], vcode[2 * p],
                                           0x0C000C00u | ((4u + k) << 16) | (uint32_t)k);
        u32x4 lo, hi;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            // the low nibble lands in mantissa bits 6..9; the high nibble lands in
            // bits 10..13, which the exponent of 1.0 sets anyway, and bits 14..15
            // receive the zero byte above it
            lo[p] = (src[p] << 6) | one2;
            hi[p] = (src[p] & mant47) | one2;
        }
        const f16x8 al = __builtin_bit_cast(f16x8, lo);
        const f16x8 ah = __builtin_bit_cast(f16x8, hi);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            st[b].acc[2 * k] = mfma16x16x32(al, bh[b], st[b].acc[2 * k]);
            st[b].acc[2 * k] = mfma16x16x32(al, bl[b], st[b].acc[2 * k]);
            st[b].acc[2 * k + 1] = mfma16x16x32(ah, bh[b], st[b].acc[2 * k + 1]);
            st[b].acc[2 * k + 1] = mfma16x16x32(ah, bl[b], st[b].acc[2 * k + 1]);
        }
    }
}

// The first two tiles of a walk: A at t_begin, B one tile on (or the last tile again).
template <int CB, bool BUF>
__device__ __forceinline__ void walk_first_tiles(Tile<CB> &A, Tile<CB> &B, const DecodeArgs &a,
                                                 PageIds &pid, const int32_t *ptab, int h,
                                                 int t_begin, int t_end, int lane)
{
    const int n = (t_end - t_begin + kTile - 1) / kTile;
    LaneAddr la;
    la.init<CB>(lane);
    const int last = t_begin + (n - 1) * kTile;
    load_tile<CB, BUF>(A, a, pid, h, t_begin, t_end, la);
    const int tb = min(t_begin + kTile, last);
    pid.reach(a, ptab, (min(tb + kTile, t_end) - 1) >> a.page_log2, lane);
    load_tile<CB, BUF>(B, a, pid, h, tb, t_end, la);
}

// ---- a7..a9: one wave's page walk over the tokens [t_begin, t_end), two register tiles in
// flight: each is refilled with the tile two ahead right after it is consumed, so the same
// loads are outstanding at every tile and the wait before a tile covers that tile's loads
// only.  The loop has one exit and issues both prefetches in every pass (a prefetch past the
// last tile re-reads it, an L2 hit): a path into the loop head with one tile in flight would
// make the compiler wait for both tiles everywhere.  The page-id window moves along with the
// prefetches, so the pipeline runs through the whole range without draining.
// pre: the caller has issued the first two tiles into A and B (walk_first_tiles) already;
// otherwise the walk issues them itself.
template <int F, bool EXT, int CB, int NB, bool BUF>
__device__ __forceinline__ void walk_tiles(WaveState (&st)[NB], const DecodeArgs &a, PageIds &pid,
                                           const int32_t *ptab, int h, int t_begin, int t_end,
                                           int lane, float kscale, const QOperand<F> *qop,
                                           ParLds &pl, const int (&col_len)[NB], int mask_from,
                                           Tile<CB> &A, Tile<CB> &B, bool pre = false)
{
    const int n = (t_end - t_begin + kTile - 1) / kTile;
    if (n <= 0)
        return;
    LaneAddr la;
    la.init<CB>(lane);
    const int last = t_begin + (n - 1) * kTile;   // start of the last tile
    // the largest page index a tile starting at t reads
    auto top_page = [&](int t) { return (min(t + kTile, t_end) - 1) >> a.page_log2; };
    if (!pre)
        walk_first_tiles<CB, BUF>(A, B, a, pid, ptab, h, t_begin, t_end, lane);
    int i = 0;
    for (; i + 2 < n; i += 2) {
        const int ta = t_begin + i * kTile;
        consume_tile<F, EXT, CB, NB>(st, A, ta, t_end, lane, kscale, qop, pl, col_len, mask_from);
#pragma unroll
        for (int b = 0; b < NB; ++b)
            st[b].tick();
        pid.reach(a, ptab, top_page(ta + 2 * kTile), lane);
        load_tile<CB, BUF>(A, a, pid, h, ta + 2 * kTile, t_end, la);
        consume_tile<F, EXT, CB, NB>(st, B, ta + kTile, t_end, lane, kscale, qop, pl, col_len,
                                     mask_from);
#pragma unroll
        for (int b = 0; b < NB; ++b)
            st[b].tick();
        const int tb = min(ta + 3 * kTile, last);
        pid.reach(a, ptab, top_page(tb), lane);
        load_tile<CB, BUF>(B, a, pid, h, tb, t_end, la);
    }
    consume_tile<F, EXT, CB, NB>(st, A, t_begin + i * kTile, t_end, lane, kscale, qop, pl, col_len,
                                 mask_from);
#pragma unroll
    for (int b = 0; b < NB; ++b)
        st[b].tick();
    if (i + 1 < n) {
        consume_tile<F, EXT, CB, NB>(st, B, t_begin + (i + 1) * kTile, t_end, lane, kscale, qop, pl,
                                     col_len, mask_from);
#pragma unroll
        for (int b = 0; b < NB; ++b)
            st[b].tick();
    }
}

// Inverse V rotation of one output row held as channels (2 lane, 2 lane + 1) by the
// 64 lanes of a wave: width 1 in-lane, widths 2.. across lanes.
template <int BV>
__device__ __forceinline__ void inverse_rotate_pair(float &o0, float &o1, int lane)
{
    if constexpr (BV > 1) {
        const float u = o0 + o1, w = o0 - o1;
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
        o0 *= InvSqrt<BV>::value;
        o1 *= InvSqrt<BV>::value;
    }
}

// The inverse V rotation for a block size known only at run time (uniform branch).
__device__ __forceinline__ void inverse_rotate_pair_rt(float &o0, float &o1, int lane, int bv)
{
    switch (bv) {
    case 16: inverse_rotate_pair<16>(o0, o1, lane); break;
    case 32: inverse_rotate_pair<32>(o0, o1, lane); break;
    case 64: inverse_rotate_pair<64>(o0, o1, lane); break;
    case 128: inverse_rotate_pair<128>(o0, o1, lane); break;
    default: break;
    }
}

// ---- a10 by one wave for one output row of up to 64 splits, whose partials start at slot
// base (lane j holds split j's maximum and normaliser, lane l the channels 2 l, 2 l + 1)
constexpr int kCombineEarly = 4;

// A float pair of the partials.  COH: read at device scope, past this XCD's L2, for
// partials that other workgroups of the same launch wrote at device scope.
template <bool COH>
__device__ __forceinline__ float2 load_pair(const float *p)
{
    if constexpr (COH) {
        const uint64_t u = __hip_atomic_load(reinterpret_cast<const uint64_t *>(p), __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
        return make_float2(__uint_as_float((uint32_t)u), __uint_as_float((uint32_t)(u >> 32)));
    } else {
        return *reinterpret_cast<const float2 *>(p);
    }
}

// The first kCombineEarly splits' outputs and every split's (m, l) are requested together;
// each row holds max_splits slots, so these loads stay inside the workspace whatever the
// row's length.
template <bool COH>
__device__ __forceinline__ void combine_loads(const DecodeArgs &a, int64_t base, int lane,
                                              float2 (&v0)[kCombineEarly], float2 &ml)
{
    const float *po = a.part_o + base * kHeadDim + 2 * lane;
#pragma unroll
    for (int k = 0; k < kCombineEarly; ++k)
        v0[k] = k < a.max_splits ? load_pair<COH>(po + (int64_t)k * kHeadDim) : make_float2(0.0f, 0.0f);
    ml = make_float2(-INFINITY, 0.0f);
    if (lane < a.max_splits)
        ml = load_pair<COH>(a.part_ml + 2 * (base + lane));
}

// The log-sum-exp merge of the row's n (1..64) splits: the weights come from two wave
// reductions by row permutes, the outputs are summed with each split's weight broadcast
// from its lane.  o0, o1: the normalised output, still in the rotated basis.
template <bool COH>
__device__ __forceinline__ void combine_merge(const DecodeArgs &a, int64_t base, int n, int lane,
                                              const float2 (&v0)[kCombineEarly], float2 ml,
                                              float &o0, float &o1)
{
    const float *po = a.part_o + base * kHeadDim + 2 * lane;
    const float m = lane < n ? ml.x : -INFINITY, l = lane < n ? ml.y : 0.0f;
    const float M = col_max(row16_max(m));
    const float wj = lane < n ? __builtin_amdgcn_exp2f(m - M) : 0.0f;
    const float lsum = col_sum(row16_sum(wj * l));
    o0 = 0.0f;
    o1 = 0.0f;
#pragma unroll
    for (int k = 0; k < kCombineEarly; ++k) {
        if (k < n) {
            const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wj), k));
            o0 = fmaf(w, v0[k].x, o0);
            o1 = fmaf(w, v0[k].y, o1);
        }
    }
    int i = kCombineEarly;
    for (; i + 4 <= n; i += 4) {
        float2 v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            v[k] = load_pair<COH>(po + (int64_t)(i + k) * kHeadDim);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wj), i + k));
            o0 = fmaf(w, v[k].x, o0);
            o1 = fmaf(w, v[k].y, o1);
        }
    }
    for (; i < n; ++i) {
        const float2 v = load_pair<COH>(po + (int64_t)i * kHeadDim);
        const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wj), i));
        o0 = fmaf(w, v.x, o0);
        o1 = fmaf(w, v.y, o1);
    }
    const float inv_l = 1.0f / lsum;
    o0 *= inv_l;
    o1 *= inv_l;
}

// Fused decode step: lanes 0-3 encode the new K row of (sequence s, KV head h) and lanes
// 4-7 its V row, exactly as the write kernel does, into the slot given for it.
template <int BK, typename Args>
__device__ __forceinline__ void write_new_rows(Args &a, int s, int h, int lane)
{
    const int ql = lane & 3;
    const bool is_v = lane >= 4;
    const int32_t slot = a.new_slots[s];
    const uint16_t *src = (is_v ? a.v_new + s * a.v_new_stride : a.k_new + s * a.k_new_stride)
                          + h * kHeadDim + 32 * ql;
    float x[32];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        bf16x8_to_f32(reinterpret_cast<const u32x4 *>(src)[j], x + 8 * j);
    if (!is_v) {
        encode_row<BK, 0>(x, slot, a.k_codes_w, a.k_params_w, a.num_slots, a.num_kv_heads,
                             a.page_log2, h, ql, a.k_bits);
        return;
    }
    uint8_t *vc = a.v_codes_w;
    uint32_t *vp = a.v_params_w;
    switch (a.v_block) {
    case 16: encode_row<16, 0>(x, slot, vc, vp, a.num_slots, a.num_kv_heads, a.page_log2, h, ql, a.v_bits); break;
    case 32: encode_row<32, 0>(x, slot, vc, vp, a.num_slots, a.num_kv_heads, a.page_log2, h, ql, a.v_bits); break;
    case 64: encode_row<64, 0>(x, slot, vc, vp, a.num_slots, a.num_kv_heads, a.page_log2, h, ql, a.v_bits); break;
    case 128: encode_row<128, 0>(x, slot, vc, vp, a.num_slots, a.num_kv_heads, a.page_log2, h, ql, a.v_bits); break;
    default: encode_row<0, 0>(x, slot, vc, vp, a.num_slots, a.num_kv_heads, a.page_log2, h, ql, a.v_bits); break;
    }
}

template <int BK, int F, bool EXT, int CB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(F == 2 ? kSplitWavesF2 : 2)))
void decode_split_kernel(DecodeArgs a)
{
    static_assert(!EXT || F == 1, "extend columns use the 16-column layout");
    // column blocks of 16 per wave: extend takes kExtendBlocks (more query rows share each
    // tile's operands), the decode one
    constexpr int NB = EXT ? kExtendBlocks : 1;
    const int h = blockIdx.y;
    const int G = a.group;
    // The MFMA columns: decode: the G query heads of sequence s (grid: split, KV head,
    // sequence); extend: query rows row0 .. row0 + nrows - 1 of sequence s, G heads each
    // (grid: row block, KV head, split), row i of the chunk attending over tokens 0..pos.
    int s, L, ncols, split;
    int64_t row0 = 0;      // extend: first query row of this workgroup
    int pos0 = 0;          // extend: the position of that row in its sequence
    if constexpr (EXT) {
        split = blockIdx.z;
        s = blockIdx.x / a.blocks_per_seq;
        const int lb = blockIdx.x - s * a.blocks_per_seq;
        const int q0 = a.qo_start[s], n = a.qo_start[s + 1] - q0;
        // qo_start is device data the host cannot check: a block whose rows fall outside
        // [0, total_q) does nothing, and a block is cut at total_q, so q, out and the
        // partials are only ever addressed inside their rows
        if (q0 < 0 || lb * a.rows_per_block >= n || q0 + lb * a.rows_per_block >= a.num_rows)
            return;
        row0 = q0 + lb * a.rows_per_block;
        const int nrows = min(min(a.rows_per_block, n - lb * a.rows_per_block),
                              a.num_rows - (int)row0);
        pos0 = min(a.seq_lens[s], a.max_seq_len) - n + lb * a.rows_per_block;
        L = pos0 + nrows;
        ncols = nrows * G;
    } else {
        split = a.seq_major ? blockIdx.z : blockIdx.x;
        s = a.seq_major ? blockIdx.x : blockIdx.z;
        L = min(a.seq_lens[s], a.max_seq_len);
        ncols = G;
    }
    const int wg_begin = split * a.split_tokens;
    if (wg_begin >= L) {
        // without a combine launch the splits write the output themselves: split 0 of an
        // empty sequence gives it zero rows
        if (!EXT && split == 0 && (a.max_splits == 1 || a.counters != nullptr)) {
            float4 *o = reinterpret_cast<float4 *>(
                a.out + ((int64_t)s * a.num_q_heads + (int64_t)h * G) * kHeadDim);
            for (int i = threadIdx.x; i < G * kHeadDim / 4; i += blockDim.x)
                o[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
        return;
    }
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // the wave index, and with it the token range, is uniform across the wave: keep it
    // scalar so the page-table lookups and the loop control stay on the scalar unit
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // fused decode step: the workgroup holding position L - 1 writes that token's rows
    // first; the barrier after the query prologue orders those stores before every load of
    // that position (only the wave whose first two tiles hold it waits for them to load), and
    // no other workgroup reads that position
    if constexpr (!EXT) {
        if (a.new_slots != nullptr && wave == 1 && split == (L - 1) / a.split_tokens && lane < 8)
            write_new_rows<BK>(a, s, h, lane);
    }
    // the waves share the split's tiles up to the row's length evenly (a split that the
    // length cuts short still keeps all four waves busy)
    const int wg_end = min(L, wg_begin + a.split_tokens);
    const int n_tiles = (wg_end - wg_begin + kTile - 1) / kTile;
    const int t_begin = wg_begin + (wave * n_tiles / kDecodeWaves) * kTile;
    const int t_end = min(wg_end, wg_begin + ((wave + 1) * n_tiles / kDecodeWaves) * kTile);

    // the first chunk's page ids are requested before the query prologue, so their latency
    // overlaps it
    const int32_t *ptab = a.page_table + (int64_t)s * a.max_pages;
    // (page ids and tile addresses are clamped into the table and the pool, so the tile loads
    // are in bounds for any range, an empty one included)
    PageIds pid;
    pid.fill(a, ptab, t_begin >> a.page_log2, lane);

    // the waves' partial states in the epilogue (F = 2: the two halves of each column are
    // merged inside the wave first, so one slot per query head and wave)
    constexpr int kSlots = F == 2 ? 8 : 16;
    __shared__ float lds_o[kDecodeWaves][kSlots][kHeadDim + 4];
    __shared__ QOperand<F> qop[NB];
    __shared__ ParLds lds_par[kDecodeWaves];
    __shared__ float lds_m[kDecodeWaves][kSlots];
    __shared__ float lds_l[kDecodeWaves][kSlots];
    __shared__ float lds_qsum[kMaxGroup * NB];
    __shared__ float lds_amax[kDecodeWaves];

    // ---- a6: the query rows of this KV head (16 lanes per row, 8 channels per lane): rotate
    // them, fold sm_scale * log2(e), round them to one integer grid and cut them into the
    // int8 digits of the QK^T B operands
    const int seg = lane & 15;   // channels [8 seg, 8 seg + 8)
    float x[NB][8];
    float amax = 0.0f;
    // The query rows are requested (unconditionally: a lane past the columns reads the
    // first column's row, which every workgroup has, and zeroes it), then, for the decode,
    // the wave's first two tiles, so that the tile loads overlap the query prologue, the
    // query rows' latency included, and the walk starts on data already in registers (a
    // load round trip at kernel start, ~3 us on the Qwen3-4B-like decode, is paid once).
    // Loads return in order, so the prologue's wait for the query rows does not wait for the
    // tiles; a load issued under a branch would make the compiler wait for every load issued
    // before it where the paths join, so the tiles are always issued.  (Decode only: the
    // extend's long workgroups gain nothing from it.  In the workgroup of a fused step that
    // writes the new token's rows, the wave whose first two tiles hold that token does not use
    // them: its reads of it must follow those stores, which the prologue's barriers order, so
    // its walk issues them again.)
    u32x4 qw[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const int g = b * 16 + wave * 4 + (lane >> 4);
        const int gc = g < ncols ? g : 0;
        const int64_t qrow = EXT ? (row0 + gc / G) * a.num_q_heads + h * G + gc % G
                                 : (int64_t)s * a.num_q_heads + h * G + gc;
        qw[b] = *reinterpret_cast<const u32x4 *>(a.q + qrow * kHeadDim + 8 * seg);
    }
    Tile<CB> TA, TB;
    // only a wave whose first two tiles hold the new token (position L - 1) must wait for its
    // write; the other waves of the writing workgroup keep their early tiles
    const bool writer = a.new_slots != nullptr && split == (L - 1) / a.split_tokens &&
                        L - 1 >= t_begin && L - 1 < t_begin + 2 * kTile;
    const bool pre = !EXT && !writer && t_begin < t_end;
    if constexpr (!EXT)
        walk_first_tiles<CB, true>(TA, TB, a, pid, ptab, h, t_begin, t_end, lane);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const int g = b * 16 + wave * 4 + (lane >> 4);
        const uint32_t d[4] = {qw[b].x, qw[b].y, qw[b].z, qw[b].w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            x[b][2 * m] = g < ncols ? __uint_as_float(d[m] << 16) : 0.0f;
            x[b][2 * m + 1] = g < ncols ? __uint_as_float(d[m] & 0xFFFF0000u) : 0.0f;
        }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const int g = b * 16 + wave * 4 + (lane >> 4);
        rotate_query_row<BK>(x[b], seg);
        float sum = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            x[b][i] *= a.q_scale;
            amax = fmaxf(amax, fabsf(x[b][i]));
            sum += x[b][i];
        }
        sum = row16_sum(sum);
        if (seg == 0 && g < kMaxGroup * NB)
            lds_qsum[g] = sum;
    }
    amax = col_max(row16_max(amax));
    if (lane == 0)
        lds_amax[wave] = amax;
    // the B operands start as zeros: rows past the columns and, for F = 2, the other
    // half's steps stay so
    {
        constexpr int kWords = (int)(sizeof(QOperand<F>) * NB / 16);
        i32x4 *z = reinterpret_cast<i32x4 *>(&qop[0]);
        for (int i = tid; i < kWords; i += 64 * kDecodeWaves)
            z[i] = i32x4{0, 0, 0, 0};
    }
    __syncthreads();
    // one power-of-two factor 2^f for all columns: max |q' 2^f| in [2^19, 2^20)
    amax = fmaxf(fmaxf(lds_amax[0], lds_amax[1]), fmaxf(lds_amax[2], lds_amax[3]));
    int e = 0;
    if (amax > 0.0f)
        frexpf(amax, &e);
    const float grid = ldexpf(1.0f, 20 - e);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const int g = b * 16 + wave * 4 + (lane >> 4);
        if (g < ncols) {
            // q = round(q' 2^f) (|q| <= 2^20) from the bits of q' 2^f + 1.5 2^23, offset by
            // 128 (1 + 2^8 + 2^16) so that its three low bytes are the balanced int8 digits
            // + 128: q = 2^16 hi + 2^8 mid + lo, each digit in [-128, 127]
            uint32_t u[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                u[i] = __float_as_uint(__builtin_fmaf(x[b][i], grid, 0x1.8p23f)) +
                       (0x808080u - 0x4B400000u);
            // element e of a lane's B operand is channel 32 kq + 2 e + par: this lane's
            // channels of one parity are bytes 0..3 of its dword seg % 4 in lane
            // column + 16 (seg / 4)
            const int col = F == 2 ? g : g - b * 16;
            const int ln = col + 16 * (seg >> 2);
#pragma unroll
            for (int par = 0; par < 2; ++par) {
#pragma unroll
                for (int dg = 0; dg < 3; ++dg) {
                    const uint32_t k = 2 - dg;   // byte of the digit: hi 2, mid 1, lo 0
                    const uint32_t lo = __builtin_amdgcn_perm(u[par + 2], u[par], 0x0C0C0400u + k * 0x101u);
                    const uint32_t hi = __builtin_amdgcn_perm(u[par + 6], u[par + 4], 0x0C0C0400u + k * 0x101u);
                    const int32_t word = (int32_t)((lo | (hi << 16)) ^ 0x80808080u);
                    if constexpr (F == 2) {
                        // the same digits in both halves' steps: half j at column g + 8 j
                        reinterpret_cast<int32_t *>(&qop[0].v[par][dg][ln])[seg & 3] = word;
                        reinterpret_cast<int32_t *>(&qop[0].v[2 + par][dg][ln + 8])[seg & 3] = word;
                    } else {
                        reinterpret_cast<int32_t *>(&qop[b].v[par][dg][ln])[seg & 3] = word;
                    }
                }
            }
        }
    }
    const int n16 = lane & 15;
    const int kq = lane >> 4;
    const int gl = F == 2 ? (n16 & 7) : n16;   // this lane's column (query head)
    // extend: the lane's column sees tokens 0 .. col_len - 1; tiles that reach past the
    // first row's position mask per column
    int col_len[NB];
    const int mask_from = pos0 + 1;
    WaveState st[NB];
    // K lanes scale by 2^-f (the integer query's grid), V lanes by 1
    const float kscale = lane < 32 ? ldexpf(1.0f, e - 20) : 1.0f;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const int gb = b * 16 + gl;
        col_len[b] = EXT ? (gb < ncols ? pos0 + gb / G + 1 : 0) : 0;
        st[b].qsum = lds_qsum[gb];
        // a finite start: with F = 2 half a tile may hold no valid token while nothing has
        // been seen yet, and exp2(-inf - (-inf)) would poison the sums
        st[b].m = kNoScore;
        st[b].l = 0.0f;
        st[b].z = 0.0f;
        st[b].wsum = 0.0f;
        st[b].E = 64;
        st[b].slim = 0x1p-58f;   // 2^(6 - E)
        st[b].wpend = 0.0f;
        st[b].nt = 0;
#pragma unroll
        for (int c = 0; c < 8; ++c)
            st[b].acc[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    __syncthreads();   // qop is complete

    // ---- a7..a9: the page walk
    walk_tiles<F, EXT, CB, NB, !EXT>(st, a, pid, ptab, h, t_begin, t_end, lane, kscale, qop,
                                     lds_par[wave], col_len, mask_from, TA, TB, pre);

    // ---- the waves' (and, for F = 2, the two halves') partial states of this split, one
    // block of 16 columns at a time through the same LDS.  The output rows are written here
    // when this is the row's only split and no combine launch follows (one split in the
    // launch, or a short row under the in-kernel combine).
    const bool direct = a.max_splits == 1 || (!EXT && a.counters != nullptr && L <= a.split_tokens);
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
        const int cb0 = blk * 16;                 // first column of the block
        const int nc = min(ncols - cb0, 16);      // its columns (uniform)
        if (nc <= 0)
            break;
        if (blk > 0)
            __syncthreads();   // the previous block's reads of lds_o are done
        WaveState &sb = st[blk];
        sb.recentre();
        sb.l = col_sum(sb.l);
        sb.z = col_sum(sb.z);
        sb.wsum = col_sum(sb.wsum);
        float o[8][4];
        {
            const float u_even = ldexpf(16.0f, -sb.E), u_odd = ldexpf(64.0f, -sb.E);
            const float zero = fmaf(8.0f, ldexpf(sb.wsum, -sb.E), sb.z);
#pragma unroll
            for (int c = 0; c < 8; ++c)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    o[c][r] = fmaf(sb.acc[c][r], (c & 1) ? u_odd : u_even, zero);
        }
        float m_w = sb.m, l_w = sb.l;
        if constexpr (F == 2) {
            // lanes n16 and n16 ^ 8 (one 16-lane row) hold the two halves of head n16 % 8
            const float m_o = dpp_row_ror8(sb.m);
            const float M = fmaxf(sb.m, m_o);
            const float fa = __builtin_amdgcn_exp2f(sb.m - M), fb = __builtin_amdgcn_exp2f(m_o - M);
            l_w = sb.l * fa + dpp_row_ror8(sb.l) * fb;
            m_w = M;
#pragma unroll
            for (int c = 0; c < 8; ++c)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    o[c][r] = o[c][r] * fa + dpp_row_ror8(o[c][r]) * fb;
        }
        if (n16 < kSlots && gl < nc) {
#pragma unroll
            for (int c = 0; c < 8; ++c)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    lds_o[wave][n16][32 * kq + 8 * r + c] = o[c][r];
            if (kq == 0) {
                lds_m[wave][n16] = m_w;
                lds_l[wave][n16] = l_w;
            }
        }
        __syncthreads();
        if (direct) {
            // the row's only split: merge the waves, normalise, undo the V rotation and
            // write the output rows here; wave w takes columns w, w + 4, ..., lane l
            // channels 2 l and 2 l + 1
            for (int gc = wave; gc < nc; gc += kDecodeWaves) {
                float M = lds_m[0][gc];
#pragma unroll
                for (int w = 1; w < kDecodeWaves; ++w)
                    M = fmaxf(M, lds_m[w][gc]);
                float o0 = 0.0f, o1 = 0.0f, lsum = 0.0f;
#pragma unroll
                for (int w = 0; w < kDecodeWaves; ++w) {
                    const float f = __builtin_amdgcn_exp2f(lds_m[w][gc] - M);
                    o0 += f * lds_o[w][gc][2 * lane];
                    o1 += f * lds_o[w][gc][2 * lane + 1];
                    lsum += f * lds_l[w][gc];
                }
                const float inv_l = 1.0f / lsum;
                o0 *= inv_l;
                o1 *= inv_l;
                inverse_rotate_pair_rt(o0, o1, lane, a.v_block);
                const int g = cb0 + gc;
                const int64_t qrow = EXT ? (row0 + g / G) * a.num_q_heads + h * G + g % G
                                         : (int64_t)s * a.num_q_heads + h * G + g;
                *reinterpret_cast<float2 *>(a.out + qrow * kHeadDim + 2 * lane) =
                    make_float2(o0, o1);
            }
            continue;
        }
        for (int i = tid; i < nc * kHeadDim; i += 64 * kDecodeWaves) {
            const int gc = i >> 7, d = i & (kHeadDim - 1);
            float M = lds_m[0][gc];
#pragma unroll
            for (int w = 1; w < kDecodeWaves; ++w)
                M = fmaxf(M, lds_m[w][gc]);
            float acc = 0.0f, lsum = 0.0f;
#pragma unroll
            for (int w = 0; w < kDecodeWaves; ++w) {
                const float f = __builtin_amdgcn_exp2f(lds_m[w][gc] - M);
                acc += f * lds_o[w][gc][d];
                lsum += f * lds_l[w][gc];
            }
            const int g = cb0 + gc;
            const int64_t qrow = EXT ? (row0 + g / G) * a.num_q_heads + h * G + g % G
                                     : (int64_t)s * a.num_q_heads + h * G + g;
            const int64_t row = qrow * a.max_splits + split;
            if (!EXT && a.counters != nullptr) {
                // device-scope stores: they pass this XCD's L2, so the split that merges
                // in this launch reads them from any XCD
                __hip_atomic_store(a.part_o + row * kHeadDim + d, acc, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
                if (d == 0) {
                    __hip_atomic_store(a.part_ml + 2 * row, M, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                    __hip_atomic_store(a.part_ml + 2 * row + 1, lsum, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                }
            } else {
                a.part_o[row * kHeadDim + d] = acc;
                if (d == 0) {
                    a.part_ml[2 * row] = M;
                    a.part_ml[2 * row + 1] = lsum;
                }
            }
        }
    }
    if constexpr (!EXT) {
        if (a.counters != nullptr && !direct) {
            // a10 in this launch: each split's partials have completed before it counts
            // itself in; the split that counts last reads them all at device scope, merges
            // them and clears the counter for the next call.  The ordering rests on the
            // hardware, not on a fence: the partial stores above are agent-scope (sc1)
            // stores, which complete at the device's coherence point, past this XCD's L2;
            // s_waitcnt(0) waits until every one of this thread's stores has been
            // acknowledged; the barrier then makes every thread's stores complete before
            // thread 0 issues the counter update (an agent-scope atomic at the same point).
            // The split that sees the count reach n reads the partials with agent-scope
            // loads, which bypass its own XCD's L2 and fetch from that same point.  (A
            // device-scope release fence would also order them, but on this chip it writes
            // back and invalidates the whole L2 of the XCD, the other workgroups' tiles
            // included: the Qwen3-4B-like decode took 61 us with one instead of 18.)
            __shared__ int lds_last;
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            int32_t *cnt = a.counters + (int64_t)s * a.num_kv_heads + h;
            const int n = (L + a.split_tokens - 1) / a.split_tokens;
            if (tid == 0)
                lds_last = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                           n - 1;
            __syncthreads();
            if (!lds_last)
                return;
            if (tid == 0)
                __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            // the lane index afresh from the exec mask: keeping the kernel's own live up to
            // here costs a spill
            const int cl = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
            for (int g = wave; g < G; g += kDecodeWaves) {
                const int64_t qrow = (int64_t)s * a.num_q_heads + h * G + g;
                float2 v0[kCombineEarly], ml;
                combine_loads<true>(a, qrow * a.max_splits, cl, v0, ml);
                float o0, o1;
                combine_merge<true>(a, qrow * a.max_splits, n, cl, v0, ml, o0, o1);
                inverse_rotate_pair_rt(o0, o1, cl, a.v_block);
                *reinterpret_cast<float2 *>(a.out + qrow * kHeadDim + 2 * cl) =
                    make_float2(o0, o1);
            }
        }
    }
}

// ---- the balanced decode ------------------------------------------------------------------
// One resident round of workgroups in NG groups of Hkv, one workgroup per KV head of a group.
// Group j takes the tile columns [T j / NG, T (j + 1) / NG) of the (sequence, 32-token tile)
// space in that order (T tile columns in all), and its workgroup h walks them for KV head h.
// Every workgroup streams the same number of bytes, so none waits for a long sequence at the
// end (a grid of per-split workgroups in several rounds leaves the chip part idle while its
// last round drains: ~8% of the Qwen3-32B-like decode), and the Hkv workgroups of a group read
// the Hkv row blocks of the same pages at the same time, from one XCD (their launch indices
// differ by NG, a multiple of the 8 XCDs): the pages stay a contiguous read for the memory,
// and the parameter lines that neighbouring heads share are fetched once.
// A workgroup walks its share as segments, one sequence each: a segment that holds all tiles
// of its (sequence, KV head) pair writes the output itself; otherwise it leaves a partial at
// slot (j + s) Hkv + h (a pair's partials sit Hkv slots apart, and the slots of different
// pairs never overlap), merged either by the last of the pair's workgroups to finish (elected
// by a counter) or, when pairs span many groups, by a combine launch.

// Largest share index whose share starts at or before tile x (shares start at floor(w T / N)).
__device__ __forceinline__ int share_of(int64_t x, int64_t T, int N)
{
    int w = (int)(x * N / T);
    while (w + 1 < N && (int64_t)(w + 1) * T / N <= x)
        ++w;
    return w;
}

// Merge of one pair's n partials (slots slot0 + k stride, k < n) for query head g of its
// group: one wave, lane l with channels 2 l, 2 l + 1; device-scope loads (other workgroups of
// the launch wrote the partials).  o0, o1: the normalised output, still in the rotated basis.
__device__ __forceinline__ void merge_slots(const float *part_o, const float *part_ml, int64_t G,
                                            int64_t slot0, int64_t stride, int n, int g, int lane,
                                            float &o0, float &o1)
{
    auto row = [&](int k) { return (slot0 + k * stride) * G + g; };
    float M = -INFINITY;
    for (int k = lane; k < n; k += 64)
        M = fmaxf(M, load_pair<true>(part_ml + 2 * row(k)).x);
    M = col_max(row16_max(M));
    float lsum = 0.0f;
    for (int k = lane; k < n; k += 64) {
        const float2 ml = load_pair<true>(part_ml + 2 * row(k));
        lsum += __builtin_amdgcn_exp2f(ml.x - M) * ml.y;
    }
    lsum = col_sum(row16_sum(lsum));
    o0 = 0.0f;
    o1 = 0.0f;
    int k = 0;
    for (; k + 4 <= n; k += 4) {
        float2 ml[4], v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            ml[j] = load_pair<true>(part_ml + 2 * row(k + j));
            v[j] = load_pair<true>(part_o + row(k + j) * kHeadDim + 2 * lane);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float wj = __builtin_amdgcn_exp2f(ml[j].x - M);
            o0 = fmaf(wj, v[j].x, o0);
            o1 = fmaf(wj, v[j].y, o1);
        }
    }
    for (; k < n; ++k) {
        const float2 ml = load_pair<true>(part_ml + 2 * row(k));
        const float2 v = load_pair<true>(part_o + row(k) * kHeadDim + 2 * lane);
        const float wj = __builtin_amdgcn_exp2f(ml.x - M);
        o0 = fmaf(wj, v.x, o0);
        o1 = fmaf(wj, v.y, o1);
    }
    const float inv_l = 1.0f / lsum;
    o0 *= inv_l;
    o1 *= inv_l;
}

// The kernel arguments seen through the kernarg segment, re-read where they are used: the
// balanced decode loops over segments, and arguments kept in registers from one segment's
// prologue to the next would stay live through the tile loop and spill.
typedef __attribute__((address_space(4))) const DecodeArgs KArgs;

__device__ __forceinline__ KArgs &kargs()
{
    KArgs *p = (KArgs *)(__builtin_amdgcn_kernarg_segment_ptr());
    asm volatile("" : "+s"(p));
    return *p;
}

// Tiles per sequence, prefix-summed into tiles[0..kBalancedMaxSeqs] (tiles[s] = tiles of the
// sequences before s; entries from num_seqs on hold the total).  Called by all NT threads of
// a workgroup (each a run of kBalancedMaxSeqs / NT sequences); wsum holds NT / 64 ints; ends
// with a barrier.
template <int NT>
__device__ __forceinline__ void tile_prefix(int *tiles, int *wsum, int tid, int lane, int wave)
{
    KArgs &k = kargs();
    const int S = k.num_seqs;
    constexpr int kPer = kBalancedMaxSeqs / NT;
    int loc[kPer];
    int sum = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int s = tid * kPer + j;
        int n = 0;
        if (s < S) {
            const int L = min(k.seq_lens[s], k.max_seq_len);
            n = L > 0 ? (L + kTile - 1) / kTile : 0;
        }
        loc[j] = n;
        sum += n;
    }
    int incl = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off, 64);
        if (lane >= off)
            incl += y;
    }
    if (lane == 63)
        wsum[wave] = incl;
    __syncthreads();
    int run = incl - sum;
    for (int i = 0; i < wave; ++i)
        run += wsum[i];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        tiles[tid * kPer + j] = run;
        run += loc[j];
    }
    if (tid == NT - 1)
        tiles[kBalancedMaxSeqs] = run;
    __syncthreads();
}

template <int BK, int F, int CB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(F == 2 ? kBalancedWavesF2 : 2)))
void decode_balanced_kernel(DecodeArgs a)
{
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    constexpr int kSlots = F == 2 ? 8 : 16;
    __shared__ float lds_o[kDecodeWaves][kSlots][kHeadDim + 4];
    __shared__ QOperand<F> qop[1];
    __shared__ ParLds lds_par[kDecodeWaves];
    __shared__ float lds_m[kDecodeWaves][kSlots];
    __shared__ float lds_l[kDecodeWaves][kSlots];
    __shared__ float lds_qsum[kMaxGroup];
    __shared__ float lds_amax[kDecodeWaves];
    __shared__ int lds_tiles[kBalancedMaxSeqs + 1];   // tiles of the sequences before s
    __shared__ int lds_wsum[kDecodeWaves];
    __shared__ int lds_last;
    // the current segment (sequence, first tile, end tile), reloaded after the tile loop so
    // that none of it stays in registers while the tiles stream
    __shared__ int lds_seg[3];
    __shared__ int lds_next;   // first tile column of the next segment

    tile_prefix<64 * kDecodeWaves>(lds_tiles, lds_wsum, tid, lane, wave);
    // empty sequences get zero rows (they hold no tiles)
    for (int s = blockIdx.x; s < kargs().num_seqs; s += gridDim.x) {
        KArgs &k = kargs();
        if (min(k.seq_lens[s], k.max_seq_len) <= 0) {
            float4 *o = reinterpret_cast<float4 *>(k.out + (int64_t)s * k.num_q_heads * kHeadDim);
            for (int i = tid; i < k.num_q_heads * kHeadDim / 4; i += blockDim.x)
                o[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
    }
    // this workgroup: KV head h of group j; fewer tile columns than groups: one each
    const int NG = gridDim.x / kargs().num_kv_heads;
    const int h = blockIdx.x / NG;
    const int j = blockIdx.x - h * NG;
    {
        const int T = lds_tiles[kargs().num_seqs];
        const int N = min(NG, T);
        if (j >= N)
            return;
        if (tid == 0)
            lds_next = (int)((int64_t)j * T / N);
    }
    const int n16 = lane & 15;
    const int kq = lane >> 4;
    const int gl = F == 2 ? (n16 & 7) : n16;   // this lane's column (query head)
    const int seg = lane & 15;                 // prologue: channels [8 seg, 8 seg + 8)
    ParLds &pl = lds_par[wave];
    while (true) {
        // ---- the next segment: from tile column g to the end of its sequence or the share
        __syncthreads();   // lds_next and lds_seg are written, the last segment is done
        {
            const int S = kargs().num_seqs;
            const int T = lds_tiles[S];
            const int N = min(NG, T);
            const int g1 = (int)((int64_t)(j + 1) * T / N);
            const int g = lds_next;
            if (g >= g1)
                break;
            // the sequence holding column g: P[s] <= g < P[s + 1]
            int s = 0, hi = S;
            while (hi - s > 1) {
                const int mid = (s + hi) >> 1;
                if (lds_tiles[mid] <= g)
                    s = mid;
                else
                    hi = mid;
            }
            const int seg_end = min(g1, lds_tiles[s + 1]);
            __syncthreads();   // every thread has read lds_next
            if (tid == 0) {
                lds_seg[0] = s;
                lds_seg[1] = g - lds_tiles[s];
                lds_seg[2] = seg_end - lds_tiles[s];
                lds_next = seg_end;
            }
            __syncthreads();
        }
        const int s = __builtin_amdgcn_readfirstlane(lds_seg[0]);
        const int t0 = __builtin_amdgcn_readfirstlane(lds_seg[1]);
        const int t1 = __builtin_amdgcn_readfirstlane(lds_seg[2]);
        KArgs &k = kargs();
        const int G = k.group;
        const int L = min(k.seq_lens[s], k.max_seq_len);
        // fused decode step: the segment holding position L - 1 writes that token's rows
        // first; the prologue's barriers order those stores before every load of that
        // position (only the wave whose first two tiles hold it waits for them to load), and
        // no other workgroup reads that position
        if (k.new_slots != nullptr && wave == 1 && lane < 8 && (L - 1) / kTile >= t0 &&
            (L - 1) / kTile < t1)
            write_new_rows<BK>(k, s, h, lane);
        // the waves share the segment's tiles evenly
        const int n_tiles = t1 - t0;
        const int seg_tok0 = t0 * kTile, seg_tok1 = min(L, t1 * kTile);
        const int t_begin = seg_tok0 + (wave * n_tiles / kDecodeWaves) * kTile;
        const int t_end = min(seg_tok1, seg_tok0 + ((wave + 1) * n_tiles / kDecodeWaves) * kTile);
        const int32_t *ptab = a.page_table + (int64_t)s * a.max_pages;
        // (page ids and tile addresses are clamped into the table and the pool, so the loads
        // below are in bounds for any range, an empty one included)
        PageIds pid;
        pid.fill(a, ptab, t_begin >> a.page_log2, lane);

        // ---- a6: the query rows of (s, h): rotate, scale, round to one grid, cut into digits
        float x[8];
        float amax = 0.0f;
        // The query row is requested, then the wave's first two tiles of the segment, so that
        // the tile loads overlap the query prologue, the query row's latency included: both
        // are unconditional (a lane past the G heads reads head 0's row and zeroes it), as a
        // load issued under a branch would make the compiler wait for every load issued
        // before it where the paths join.  In the segment of a fused step that writes the new
        // token's rows, the wave whose first two tiles hold that token does not use these
        // tiles: its reads of it must follow those stores, which the prologue's barriers
        // order, so its walk issues them again.
        Tile<CB> TA, TB;
        // only a wave whose first two tiles hold the new token (position L - 1) must wait for
        // its write; the other waves of the segment keep their early tiles
        const bool writer = k.new_slots != nullptr && (L - 1) / kTile >= t0 && (L - 1) / kTile < t1 &&
                            L - 1 >= t_begin && L - 1 < t_begin + 2 * kTile;
        const bool pre = !writer && t_begin < t_end;
        {
            const int gq = wave * 4 + (lane >> 4);
            const int64_t qrow = (int64_t)s * k.num_q_heads + h * G + (gq < G ? gq : 0);
            const u32x4 wq = *reinterpret_cast<const u32x4 *>(k.q + qrow * kHeadDim + 8 * seg);
            walk_first_tiles<CB, true>(TA, TB, a, pid, ptab, h, t_begin, t_end, lane);
            const uint32_t d[4] = {wq.x, wq.y, wq.z, wq.w};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                x[2 * m] = gq < G ? __uint_as_float(d[m] << 16) : 0.0f;
                x[2 * m + 1] = gq < G ? __uint_as_float(d[m] & 0xFFFF0000u) : 0.0f;
            }
            rotate_query_row<BK>(x, seg);
            float sum = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                x[i] *= k.q_scale;
                amax = fmaxf(amax, fabsf(x[i]));
                sum += x[i];
            }
            sum = row16_sum(sum);
            if (seg == 0 && gq < kMaxGroup)
                lds_qsum[gq] = sum;
        }
        amax = col_max(row16_max(amax));
        if (lane == 0)
            lds_amax[wave] = amax;
        {
            constexpr int kWords = (int)(sizeof(QOperand<F>) / 16);
            i32x4 *z = reinterpret_cast<i32x4 *>(&qop[0]);
            for (int i = tid; i < kWords; i += 64 * kDecodeWaves)
                z[i] = i32x4{0, 0, 0, 0};
        }
        __syncthreads();
        amax = fmaxf(fmaxf(lds_amax[0], lds_amax[1]), fmaxf(lds_amax[2], lds_amax[3]));
        int e = 0;
        if (amax > 0.0f)
            frexpf(amax, &e);
        const float grid = ldexpf(1.0f, 20 - e);
        {
            const int gq = wave * 4 + (lane >> 4);
            if (gq < G) {
                uint32_t u[8];
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    u[i] = __float_as_uint(__builtin_fmaf(x[i], grid, 0x1.8p23f)) +
                           (0x808080u - 0x4B400000u);
                const int ln = gq + 16 * (seg >> 2);
#pragma unroll
                for (int par = 0; par < 2; ++par) {
#pragma unroll
                    for (int dg = 0; dg < 3; ++dg) {
                        const uint32_t k = 2 - dg;
                        const uint32_t lo = __builtin_amdgcn_perm(u[par + 2], u[par], 0x0C0C0400u + k * 0x101u);
                        const uint32_t hi = __builtin_amdgcn_perm(u[par + 6], u[par + 4], 0x0C0C0400u + k * 0x101u);
                        const int32_t word = (int32_t)((lo | (hi << 16)) ^ 0x80808080u);
                        if constexpr (F == 2) {
                            reinterpret_cast<int32_t *>(&qop[0].v[par][dg][ln])[seg & 3] = word;
                            reinterpret_cast<int32_t *>(&qop[0].v[2 + par][dg][ln + 8])[seg & 3] = word;
                        } else {
                            reinterpret_cast<int32_t *>(&qop[0].v[par][dg][ln])[seg & 3] = word;
                        }
                    }
                }
            }
        }
        WaveState st[1];
        const int col_len[1] = {0};
        const float kscale = lane < 32 ? ldexpf(1.0f, e - 20) : 1.0f;
        st[0].m = kNoScore;
        st[0].l = 0.0f;
        st[0].z = 0.0f;
        st[0].wsum = 0.0f;
        st[0].E = 64;
        st[0].slim = 0x1p-58f;
        st[0].wpend = 0.0f;
        st[0].nt = 0;
#pragma unroll
        for (int c = 0; c < 8; ++c)
            st[0].acc[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        __syncthreads();   // qop and lds_qsum are complete
        st[0].qsum = lds_qsum[gl];

        // ---- a7..a9: the page walk
        walk_tiles<F, false, CB, 1, true>(st, a, pid, ptab, h, t_begin, t_end, lane, kscale, qop, pl,
                                          col_len, 0, TA, TB, pre);

        // ---- the waves' (and for F = 2 the two halves') states of this segment
        WaveState &sb = st[0];
        KArgs &ke = kargs();
        const int eG = ke.group;
        const int Hkv = ke.num_kv_heads;
        const int es = __builtin_amdgcn_readfirstlane(lds_seg[0]);
        const int e_t0 = __builtin_amdgcn_readfirstlane(lds_seg[1]);
        const int e_t1 = __builtin_amdgcn_readfirstlane(lds_seg[2]);
        const int ent = lds_tiles[es + 1] - lds_tiles[es];
        sb.recentre();
        sb.l = col_sum(sb.l);
        sb.z = col_sum(sb.z);
        sb.wsum = col_sum(sb.wsum);
        float o[8][4];
        {
            const float u_even = ldexpf(16.0f, -sb.E), u_odd = ldexpf(64.0f, -sb.E);
            const float zero = fmaf(8.0f, ldexpf(sb.wsum, -sb.E), sb.z);
#pragma unroll
            for (int c = 0; c < 8; ++c)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    o[c][r] = fmaf(sb.acc[c][r], (c & 1) ? u_odd : u_even, zero);
        }
        float m_w = sb.m, l_w = sb.l;
        if constexpr (F == 2) {
            const float m_o = dpp_row_ror8(sb.m);
            const float M = fmaxf(sb.m, m_o);
            const float fa = __builtin_amdgcn_exp2f(sb.m - M), fb = __builtin_amdgcn_exp2f(m_o - M);
            l_w = sb.l * fa + dpp_row_ror8(sb.l) * fb;
            m_w = M;
#pragma unroll
            for (int c = 0; c < 8; ++c)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    o[c][r] = o[c][r] * fa + dpp_row_ror8(o[c][r]) * fb;
        }
        if (n16 < kSlots && gl < eG) {
#pragma unroll
            for (int c = 0; c < 8; ++c)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    lds_o[wave][n16][32 * kq + 8 * r + c] = o[c][r];
            if (kq == 0) {
                lds_m[wave][n16] = m_w;
                lds_l[wave][n16] = l_w;
            }
        }
        __syncthreads();
        if (e_t0 == 0 && e_t1 == ent) {
            // the pair's only segment: merge the waves, normalise, undo the V rotation, write
            for (int gc = wave; gc < eG; gc += kDecodeWaves) {
                float M = lds_m[0][gc];
#pragma unroll
                for (int wv = 1; wv < kDecodeWaves; ++wv)
                    M = fmaxf(M, lds_m[wv][gc]);
                float o0 = 0.0f, o1 = 0.0f, lsum = 0.0f;
#pragma unroll
                for (int wv = 0; wv < kDecodeWaves; ++wv) {
                    const float f = __builtin_amdgcn_exp2f(lds_m[wv][gc] - M);
                    o0 += f * lds_o[wv][gc][2 * lane];
                    o1 += f * lds_o[wv][gc][2 * lane + 1];
                    lsum += f * lds_l[wv][gc];
                }
                const float inv_l = 1.0f / lsum;
                o0 *= inv_l;
                o1 *= inv_l;
                inverse_rotate_pair_rt(o0, o1, lane, ke.v_block);
                const int64_t qrow = (int64_t)es * ke.num_q_heads + h * eG + gc;
                *reinterpret_cast<float2 *>(ke.out + qrow * kHeadDim + 2 * lane) = make_float2(o0, o1);
            }
            continue;
        }
        // a partial of the pair: device-scope stores (past this XCD's L2), so the workgroup
        // or the launch that merges reads them from any XCD
        const int64_t slot = (int64_t)(j + es) * Hkv + h;
        for (int i = tid; i < eG * kHeadDim; i += 64 * kDecodeWaves) {
            const int gc = i >> 7, d = i & (kHeadDim - 1);
            float M = lds_m[0][gc];
#pragma unroll
            for (int wv = 1; wv < kDecodeWaves; ++wv)
                M = fmaxf(M, lds_m[wv][gc]);
            float acc = 0.0f, lsum = 0.0f;
#pragma unroll
            for (int wv = 0; wv < kDecodeWaves; ++wv) {
                const float f = __builtin_amdgcn_exp2f(lds_m[wv][gc] - M);
                acc += f * lds_o[wv][gc][d];
                lsum += f * lds_l[wv][gc];
            }
            const int64_t row = slot * eG + gc;
            __hip_atomic_store(ke.part_o + row * kHeadDim + d, acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (d == 0) {
                __hip_atomic_store(ke.part_ml + 2 * row, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(ke.part_ml + 2 * row + 1, lsum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        if (ke.balanced_combine)
            continue;   // a combine launch merges the partials
        // Count this workgroup in once its partial stores have completed.  The ordering rests
        // on the hardware: the stores above are agent-scope (sc1) stores, which complete at
        // the device's coherence point, and s_waitcnt(0) waits until every one of this
        // thread's stores has been acknowledged; the barrier then makes every thread's stores
        // complete before thread 0 issues the counter update.  The workgroup that sees the
        // count reach n reads the partials with agent-scope loads, which bypass its own
        // XCD's L2 and fetch from that same point.  (A device-scope release fence would also
        // order them, but on this chip it writes back and invalidates the whole L2 of the
        // XCD, the other workgroups' tiles included.)
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        const int64_t pair = (int64_t)es * Hkv + h;
        const int T = lds_tiles[ke.num_seqs];
        const int N = min(NG, T);
        const int j_lo = share_of(lds_tiles[es], T, N);
        const int j_hi = share_of(lds_tiles[es + 1] - 1, T, N);
        if (tid == 0)
            lds_last = __hip_atomic_fetch_add(ke.counters + pair, 1, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT) == j_hi - j_lo;
        __syncthreads();
        if (lds_last) {
            if (tid == 0)
                __hip_atomic_store(ke.counters + pair, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            for (int gc = wave; gc < eG; gc += kDecodeWaves) {
                float o0, o1;
                merge_slots(ke.part_o, ke.part_ml, eG, (int64_t)(j_lo + es) * Hkv + h, Hkv,
                            j_hi - j_lo + 1, gc, lane, o0, o1);
                inverse_rotate_pair_rt(o0, o1, lane, ke.v_block);
                const int64_t qrow = (int64_t)es * ke.num_q_heads + h * eG + gc;
                *reinterpret_cast<float2 *>(ke.out + qrow * kHeadDim + 2 * lane) = make_float2(o0, o1);
            }
        }
    }
}

// ---- a10 for the balanced decode when pairs span many groups: one 1024-thread workgroup per
// (sequence, query head) merges the pair's partials, 32 of them at a time (thread = partial
// residue of 32, four channels), and undoes the V rotation.  Pairs of one segment were
// written by the split launch and are skipped.
template <int BV>
__global__ __launch_bounds__(1024) void decode_balanced_combine_kernel(DecodeArgs a)
{
    const int s = blockIdx.x;
    const int gq = blockIdx.y;            // query head
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int G = a.group;
    const int Hkv = a.num_kv_heads;
    const int h = gq / G, g = gq - h * G;
    __shared__ int lds_tiles[kBalancedMaxSeqs + 1];
    __shared__ int lds_wsum[16];
    __shared__ float red[32];
    __shared__ float part[32][kHeadDim];
    tile_prefix<1024>(lds_tiles, lds_wsum, tid, tid & 63, wave);
    const int T = lds_tiles[a.num_seqs];
    const int nt = lds_tiles[s + 1] - lds_tiles[s];
    if (nt == 0)
        return;
    const int NG = a.balanced_wgs / Hkv;
    const int N = min(NG, T);
    const int j_lo = share_of(lds_tiles[s], T, N);
    const int j_hi = share_of(lds_tiles[s + 1] - 1, T, N);
    const int n = j_hi - j_lo + 1;
    if (n == 1)
        return;
    auto row = [&](int k) { return ((int64_t)(j_lo + k + s) * Hkv + h) * G + g; };
    float M = -INFINITY;
    for (int k = tid; k < n; k += 1024)
        M = fmaxf(M, a.part_ml[2 * row(k)]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        M = fmaxf(M, wave_xor(M, o));
    if ((tid & 63) == 0)
        red[wave] = M;
    __syncthreads();
    M = red[0];
#pragma unroll
    for (int w = 1; w < 16; ++w)
        M = fmaxf(M, red[w]);
    float l = 0.0f;
    for (int k = tid; k < n; k += 1024)
        l += __builtin_amdgcn_exp2f(a.part_ml[2 * row(k)] - M) * a.part_ml[2 * row(k) + 1];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        l += wave_xor(l, o);
    if ((tid & 63) == 0)
        red[16 + wave] = l;
    const int sub = tid >> 5, dq = tid & 31;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 4
    for (int k = sub; k < n; k += 32) {
        const float wk = __builtin_amdgcn_exp2f(a.part_ml[2 * row(k)] - M);
        acc += wk * *reinterpret_cast<const f32x4 *>(a.part_o + row(k) * kHeadDim + 4 * dq);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
        part[sub][4 * dq + c] = acc[c];
    __syncthreads();
    if (tid >= 64)
        return;
    l = 0.0f;
#pragma unroll
    for (int w = 0; w < 16; ++w)
        l += red[16 + w];
    const float inv_l = 1.0f / l;
    float o0 = 0.0f, o1 = 0.0f;
#pragma unroll 8
    for (int k = 0; k < 32; ++k) {
        o0 += part[k][2 * tid];
        o1 += part[k][2 * tid + 1];
    }
    o0 *= inv_l;
    o1 *= inv_l;
    inverse_rotate_pair<BV>(o0, o1, tid);
    *reinterpret_cast<float2 *>(a.out + ((int64_t)s * a.num_q_heads + gq) * kHeadDim + 2 * tid) =
        make_float2(o0, o1);
}

// Tokens attended by output row r of the combine: the sequence length (decode) or the
// causal length of query row r (extend: the sequence holding r by binary search over
// qo_start, then its position + 1).
__device__ __forceinline__ int row_length(const DecodeArgs &a, int r)
{
    if (a.qo_start == nullptr)
        return min(a.seq_lens[r], a.max_seq_len);
    int lo = 0, hi = a.num_seqs;   // qo_start[lo] <= r < qo_start[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (a.qo_start[mid] <= r)
            lo = mid;
        else
            hi = mid;
    }
    const int n = a.qo_start[lo + 1] - a.qo_start[lo];
    // at most max_seq_len even for a qo_start that breaks its preconditions, so a row never
    // counts more splits than the workspace holds
    return min(min(a.seq_lens[lo], a.max_seq_len) - n + (r - a.qo_start[lo]) + 1, a.max_seq_len);
}

// ---- a10: combine the splits of one (sequence, query head), undo the V rotation ---------
template <int BV>
__global__ __launch_bounds__(1024) void decode_combine_kernel(DecodeArgs a)
{
    // one workgroup of 16 waves per (output row, query head), for many splits
    const int s = blockIdx.x;
    const int g = blockIdx.y;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int L = row_length(a, s);
    float *out = a.out + ((int64_t)s * a.num_q_heads + g) * kHeadDim;
    if (L <= 0) {
        if (tid < kHeadDim)
            out[tid] = 0.0f;
        return;
    }
    const int n = (L + a.split_tokens - 1) / a.split_tokens;
    const int64_t row0 = ((int64_t)s * a.num_q_heads + g) * a.max_splits;
    const float *ml = a.part_ml + 2 * row0;

    __shared__ float red[32];
    __shared__ float part[32][kHeadDim];

    // global max and normaliser over the splits
    float M = -INFINITY;
    for (int i = tid; i < n; i += 1024)
        M = fmaxf(M, ml[2 * i]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        M = fmaxf(M, wave_xor(M, o));
    if ((tid & 63) == 0)
        red[wave] = M;
    __syncthreads();
    M = red[0];
#pragma unroll
    for (int w = 1; w < 16; ++w)
        M = fmaxf(M, red[w]);
    float l = 0.0f;
    for (int i = tid; i < n; i += 1024)
        l += __builtin_amdgcn_exp2f(ml[2 * i] - M) * ml[2 * i + 1];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        l += wave_xor(l, o);
    if ((tid & 63) == 0)
        red[16 + wave] = l;

    // weighted sum of the partial outputs: thread = (split residue sub of 32, 4 channels)
    const int sub = tid >> 5, dq = tid & 31;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    const float *po = a.part_o + row0 * kHeadDim + 4 * dq;
#pragma unroll 4
    for (int i = sub; i < n; i += 32) {
        const float w = __builtin_amdgcn_exp2f(ml[2 * i] - M);
        acc += w * *reinterpret_cast<const f32x4 *>(po + (int64_t)i * kHeadDim);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
        part[sub][4 * dq + j] = acc[j];
    __syncthreads();
    if (tid >= 64)
        return;
    l = 0.0f;
#pragma unroll
    for (int w = 0; w < 16; ++w)
        l += red[16 + w];
    const float inv_l = 1.0f / l;
    float o0 = 0.0f, o1 = 0.0f;
#pragma unroll 8
    for (int k = 0; k < 32; ++k) {
        o0 += part[k][2 * tid];
        o1 += part[k][2 * tid + 1];
    }
    o0 *= inv_l;
    o1 *= inv_l;
    const int lane = tid;
    inverse_rotate_pair<BV>(o0, o1, lane);
    *reinterpret_cast<float2 *>(out + 2 * lane) = make_float2(o0, o1);
}

// ---- a10 for up to 64 splits: one wave per (sequence, query head) ---------------------
// Four query heads per workgroup, no barrier.
template <int BV>
__global__ __launch_bounds__(256) void decode_combine_wave_kernel(DecodeArgs a)
{
    const int lane = threadIdx.x & 63;
    const int s = blockIdx.x;
    const int g = blockIdx.y * 4 + (threadIdx.x >> 6);
    if (g >= a.num_q_heads)
        return;
    // the partials are requested before the row's length is known, so one memory round
    // trip serves rows of up to four splits
    const int64_t base = ((int64_t)s * a.num_q_heads + g) * a.max_splits;
    float2 v0[kCombineEarly], ml;
    combine_loads<false>(a, base, lane, v0, ml);
    const int L = row_length(a, s);
    float *out = a.out + ((int64_t)s * a.num_q_heads + g) * kHeadDim;
    if (L <= 0) {
        *reinterpret_cast<float2 *>(out + 2 * lane) = make_float2(0.0f, 0.0f);
        return;
    }
    const int n = (L + a.split_tokens - 1) / a.split_tokens;   // 1..64
    float o0, o1;
    combine_merge<false>(a, base, n, lane, v0, ml, o0, o1);
    inverse_rotate_pair<BV>(o0, o1, lane);
    *reinterpret_cast<float2 *>(out + 2 * lane) = make_float2(o0, o1);
}

template <int BK, bool EXT, int CB>
void launch_f1(const DecodeArgs &a, const dim3 &grid, hipStream_t s)
{
    hipLaunchKernelGGL((decode_split_kernel<BK, 1, EXT, CB>), grid, dim3(64 * kDecodeWaves), 0, s, a);
}

template <int BK, bool EXT>
void launch_f1_widths(const DecodeArgs &a, const dim3 &grid, hipStream_t s)
{
    const int cb = (a.k_bits == 2 ? 1 : 0) | (a.v_bits == 2 ? 2 : 0);
    switch (cb) {
    case 1: launch_f1<BK, EXT, 1>(a, grid, s); break;
    case 2: launch_f1<BK, EXT, 2>(a, grid, s); break;
    case 3: launch_f1<BK, EXT, 3>(a, grid, s); break;
    default: launch_f1<BK, EXT, 0>(a, grid, s); break;
    }
}

// The decode's split grid fits on the device at once (kSplitWavesF2 workgroups per CU; two
// for the 16-column kernel).
bool one_round(const DecodeArgs &a)
{
    const int64_t wgs = (int64_t)a.max_splits * a.num_kv_heads * a.num_seqs;
    return wgs <= (int64_t)device_cus() * (a.group > 8 ? 2 : kSplitWavesF2);
}

template <int BK>
hipError_t launch_split(const DecodeArgs &a, hipStream_t s)
{
    if (a.qo_start != nullptr) {
        const dim3 grid((unsigned)(a.num_seqs * a.blocks_per_seq), (unsigned)a.num_kv_heads,
                        (unsigned)a.max_splits);
        launch_f1_widths<BK, true>(a, grid, s);
        return hipGetLastError();
    }
    // Workgroups go to the 8 XCDs round-robin in launch order.  When the whole grid is
    // resident at once, sequences vary fastest: each sequence's workgroups then share one
    // XCD (its L2) and the empty splits of short sequences spread over all XCDs (the
    // Qwen3-4B-like decode: 21.1 -> 19.7 us).  A grid of several rounds keeps splits
    // fastest, so that the long sequences' splits do not all come last (Qwen3-32B-like:
    // 639 us, against 728 with sequences fastest).
    DecodeArgs b = a;
    b.seq_major = one_round(a) && a.max_splits <= 65535 ? 1 : 0;
    const dim3 grid = b.seq_major
        ? dim3((unsigned)a.num_seqs, (unsigned)a.num_kv_heads, (unsigned)a.max_splits)
        : dim3((unsigned)a.max_splits, (unsigned)a.num_kv_heads, (unsigned)a.num_seqs);
    const int cb = (a.k_bits == 2 ? 1 : 0) | (a.v_bits == 2 ? 2 : 0);
    const dim3 block(64 * kDecodeWaves);
    if (a.group > 8)
        launch_f1_widths<BK, false>(b, grid, s);
    else if (cb == 1)
        hipLaunchKernelGGL((decode_split_kernel<BK, 2, false, 1>), grid, block, 0, s, b);
    else if (cb == 2)
        hipLaunchKernelGGL((decode_split_kernel<BK, 2, false, 2>), grid, block, 0, s, b);
    else if (cb == 3)
        hipLaunchKernelGGL((decode_split_kernel<BK, 2, false, 3>), grid, block, 0, s, b);
    else
        hipLaunchKernelGGL((decode_split_kernel<BK, 2, false, 0>), grid, block, 0, s, b);
    return hipGetLastError();
}

template <int BK, int F>
void launch_balanced_widths(const DecodeArgs &a, hipStream_t s)
{
    const dim3 grid((unsigned)a.balanced_wgs), block(64 * kDecodeWaves);
    const int cb = (a.k_bits == 2 ? 1 : 0) | (a.v_bits == 2 ? 2 : 0);
    switch (cb) {
    case 1: hipLaunchKernelGGL((decode_balanced_kernel<BK, F, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((decode_balanced_kernel<BK, F, 2>), grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL((decode_balanced_kernel<BK, F, 3>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((decode_balanced_kernel<BK, F, 0>), grid, block, 0, s, a); break;
    }
}

template <int BK>
hipError_t launch_balanced(const DecodeArgs &a, hipStream_t s)
{
    if (a.group > 8)
        launch_balanced_widths<BK, 1>(a, s);
    else
        launch_balanced_widths<BK, 2>(a, s);
    return hipGetLastError();
}

template <int BV>
hipError_t launch_combine(const DecodeArgs &a, hipStream_t s)
{
    if (a.max_splits <= 64) {
        const dim3 grid((unsigned)a.num_rows, (unsigned)((a.num_q_heads + 3) / 4));
        hipLaunchKernelGGL(decode_combine_wave_kernel<BV>, grid, dim3(256), 0, s, a);
    } else {
        const dim3 grid((unsigned)a.num_rows, (unsigned)a.num_q_heads);
        hipLaunchKernelGGL(decode_combine_kernel<BV>, grid, dim3(1024), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace

int decode_resident_wgs(int group)
{
    return device_cus() * (group > 8 ? 2 : kBalancedWavesF2);
}

int launch_decode(int k_block, int v_block, const DecodeArgs &args, void *stream)
{
    if (args.num_seqs == 0 || args.num_rows == 0)
        return 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (args.balanced_wgs > 0) {
        hipError_t e;
        switch (k_block) {
        case 0: e = launch_balanced<0>(args, s); break;
        case 16: e = launch_balanced<16>(args, s); break;
        case 32: e = launch_balanced<32>(args, s); break;
        case 64: e = launch_balanced<64>(args, s); break;
        case 128: e = launch_balanced<128>(args, s); break;
        default: return hipErrorInvalidValue;
        }
        if (e != hipSuccess || !args.balanced_combine)
            return e;
        const dim3 grid((unsigned)args.num_seqs, (unsigned)args.num_q_heads);
        switch (v_block) {
        case 0: hipLaunchKernelGGL(decode_balanced_combine_kernel<0>, grid, dim3(1024), 0, s, args); break;
        case 16: hipLaunchKernelGGL(decode_balanced_combine_kernel<16>, grid, dim3(1024), 0, s, args); break;
        case 32: hipLaunchKernelGGL(decode_balanced_combine_kernel<32>, grid, dim3(1024), 0, s, args); break;
        case 64: hipLaunchKernelGGL(decode_balanced_combine_kernel<64>, grid, dim3(1024), 0, s, args); break;
        case 128: hipLaunchKernelGGL(decode_balanced_combine_kernel<128>, grid, dim3(1024), 0, s, args); break;
        default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    // The in-kernel combine pays where launch latency dominates: a grid resident in one
    // round, of at most kInKernelCombineSplits splits per row (the Qwen3-4B-like decode
    // 19.4 -> 18.4 us, the small-batch fused step 21.3 -> 17.6 us).  Otherwise the combine
    // launch: in a grid of several rounds each workgroup would hold its slot until its
    // stores and its count complete (Qwen3-32B-like: 663 us against 640), and one workgroup
    // merging 64 splits per head is slower than the combine's one wave per head (1M
    // tokens: 227 us against 222).
    DecodeArgs a = args;
    if (a.counters != nullptr && !(a.max_splits <= kInKernelCombineSplits && one_round(a)))
        a.counters = nullptr;
    hipError_t e;
    switch (k_block) {
    case 0: e = launch_split<0>(a, s); break;
    case 16: e = launch_split<16>(a, s); break;
    case 32: e = launch_split<32>(a, s); break;
    case 64: e = launch_split<64>(a, s); break;
    case 128: e = launch_split<128>(a, s); break;
    default: return hipErrorInvalidValue;
    }
    // one split, or the in-kernel combine: the splits write the output themselves
    if (e != hipSuccess || a.max_splits == 1 || a.counters != nullptr)
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
