// Fused block-Hadamard rotation + token-wise INT4 quantisation + paged store
// for gfx950 (SAW-INT4: K~ = quant(K H_blk), V~ = quant(V H_blk); wispaper.ai
// blog, section 3 core formula, fused into the KV-cache write so that no
// separate rotation launch exists and the arithmetic hides under the memory
// time, same section, consequences 1 and 2).
//
// Work split: four lanes (a quad) per (token, head, tensor) row of 128 channels;
// lane ql of the quad owns the 32 contiguous channels [32 ql, 32 ql + 32):
//   * its bf16 input is 64 contiguous bytes (four 16-byte loads);
//   * its INT4 output is 16 contiguous bytes (one 16-byte store);
//   * butterfly widths 1..16 stay inside the lane (blocks of 16 and 32 need no
//     cross-lane traffic); widths 32 and 64 pair lanes ql^1 and ql^2 of the
//     quad through DPP quad permutes.
// A wave encodes tiles of 16 consecutive tokens of one head, the K tile and then
// the V tile, so its 64-byte row stores and 4-byte parameter stores land in
// consecutive slots of a page.  Waves are persistent: each walks the tile pairs
// with a stride of the grid's wave count and keeps the next tile's loads in
// flight while it encodes the current one.  The small per-lane footprint keeps
// two waves per SIMD resident; each keeps a tile pair in flight while it encodes the last.
//
// Bit-exactness: every step runs in IEEE binary32 in a fixed order --
// butterfly widths 1, 2, 4, ... with (u+w, u-w), then * fp32(1/sqrt b); exact
// min/max; correctly rounded (mx-mn)/15 and 1/scale; round-to-nearest-even
// binary16 parameters; codes from the stored parameters.  Contraction is
// disabled for this file (-ffp-contract=off) so no multiply-add is fused.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "kvrq_encode.h"
#include "kvrq_internal.h"

namespace kvrq {
namespace {

// The raw input of one tile as this lane holds it.
struct RowLoad {
    u32x4 raw[4];     // 32 bf16 channels
    int32_t slot;     // slot of the row's token
    bool valid;       // false past the last token: nothing is stored
};

// Issues the loads of one row.  Rows past the last token re-read the last token and are
// marked invalid: every load is unconditional, so the loads of the next tile stay in
// flight while the current one is encoded (a conditional load would make the compiler
// wait for all outstanding loads where the paths join).
__device__ __forceinline__ void load_row(RowLoad &R, const uint16_t *src_base, int64_t stride,
                                         const int32_t *slots, int64_t t, int64_t num_tokens, int ql)
{
    R.valid = t < num_tokens;
    const int64_t tc = R.valid ? t : num_tokens - 1;
    R.slot = slots[tc];
    const u32x4 *s4 = reinterpret_cast<const u32x4 *>(src_base + tc * stride + 32 * ql);
#pragma unroll
    for (int j = 0; j < 4; ++j)
        R.raw[j] = s4[j];
}

// Each wave walks tile pairs: the K tile and the V tile of the same 16 tokens of one
// head.  Pairs go in groups of 2 Hkv: pair i of group g is tile 2 g + (i & 1) of head i / 2,
// so the four waves of a workgroup take 2 heads x 2 consecutive tiles (512 contiguous bytes
// of each of 32 token rows; 2 KiB runs of two (page, head) blocks), and waves that run side
// by side read all heads of the same tokens (measured on MI355X against one tile of four
// heads per workgroup: the 32k chunk 34.1 -> 33.8 us, the Qwen3-4B-like write 44.3 -> 44.0
// us; four tiles of one head: 35.9 and 46.7 us).  The loop is
// unrolled over the two tensors, so each half is compiled for its own block size, and
// K and V work is spread evenly over the waves.
//
// STAGED: the encoded tiles of up to kWriteStage pairs per wave wait in LDS (73.7 KB per
// workgroup, two workgroups per CU: the chip's LDS holds a 32k-token chunk's whole output)
// and are stored in one burst when the stage is full and at the end.  HBM does not overlap
// reads and writes, and the stores interleaved with the loads cost more than the same
// stores in a burst after them (measured on MI355X, same machine: the 32k chunk 33.8 -> 32.9
// us, the Qwen3-4B-like write 44.1 -> 41.8 us).  A wave with fewer pairs than a full stage stores
// as it goes: a short write has too little reading left to hide the burst behind (the 16k
// long-context chunk, four pairs per wave: 19.4 -> 21.3 us staged).
template <int BK, int BV, int KBITS, int VBITS, bool STAGED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kWriteWavesPerSimd)))
void rotquant_write_kernel(WriteArgs a)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ql = lane & 3;
    const int row = lane >> 2;
    const int64_t tiles_per_head = (a.num_tokens + kWriteTile - 1) / kWriteTile;
    const int64_t num_pairs = (tiles_per_head + 1) / 2 * 2 * a.num_kv_heads;
    const int64_t stride_w = (int64_t)gridDim.x * (blockDim.x >> 6);
    int64_t pair = (int64_t)blockIdx.x * (blockDim.x >> 6) + wave;
    if (pair >= num_pairs)
        return;

    auto issue = [&](RowLoad &R, const uint16_t *src, int64_t stride, int64_t pr) {
        const int64_t g2 = pr / (2 * a.num_kv_heads);
        const int64_t r2 = pr - g2 * 2 * a.num_kv_heads;
        const int64_t tt = 2 * g2 + (r2 & 1);
        const int64_t h = r2 >> 1;
        // the staged write issues its loads at a raised priority, so they are not held
        // behind the other waves' encoding (measured on MI355X, same machine: the 32k chunk 31.9
        // -> 31.4 us, the Qwen3-4B-like write 41.7 -> 41.4 us; the unstaged 16k-token chunk,
        // whose stores go out between the loads, 19.07 -> 19.63 us, so it keeps one priority)
        if constexpr (STAGED)
            __builtin_amdgcn_s_setprio(2);
        load_row(R, src + h * kHeadDim, stride, a.slots, tt * kWriteTile + row, a.num_tokens, ql);
        if constexpr (STAGED)
            __builtin_amdgcn_s_setprio(0);
    };

    // the stage: [wave][K, V][pair]; nothing when not STAGED
    constexpr int NST = STAGED ? kWriteStage : 1;
    __shared__ StageSlot stage[STAGED ? 4 : 1][2][NST];
    int nst = 0;
    auto flush_one = [&](const StageSlot &S, uint8_t *codes, uint32_t *params, int bits) {
        const uint32_t cell = S.cell[row];
        if (cell != 0xFFFFFFFFu) {
            const u32x4 p = S.piece[lane];
            if (bits == 4)
                store_row<true>(reinterpret_cast<u32x4 *>(codes + (uint64_t)cell * kRowCodeBytes) + ql, p);
            else
                store_row<true>(reinterpret_cast<u32x2 *>(codes + (uint64_t)cell * (kRowCodeBytes / 2)) + ql,
                                u32x2{p.x, p.y});
            if (ql == 0)
                params[cell] = S.par[row];
        }
    };
    auto flush = [&]() {
        for (int k = 0; k < nst; ++k) {
            flush_one(stage[wave][0][k], a.k_codes, a.k_params, KBITS);
            flush_one(stage[wave][1][k], a.v_codes, a.v_params, VBITS);
        }
        nst = 0;
    };
    // Two register sets, K and V: each is refilled with the next pair's tile as soon as
    // its bf16 input is widened to fp32, so up to two tiles are in flight while one is
    // encoded.
    RowLoad RK, RV;
    issue(RK, a.k, a.k_stride, pair);
    issue(RV, a.v, a.v_stride, pair);
    while (true) {
        const int h = (int)((pair % (2 * a.num_kv_heads)) >> 1);
        const int64_t next = pair + stride_w;
        const bool more = next < num_pairs;
        const int64_t pf = more ? next : pair;   // past the end: re-read this pair (no store)
        float x[32];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            bf16x8_to_f32(RK.raw[j], x + 8 * j);
        int32_t slot = RK.valid ? RK.slot : -1;
        issue(RK, a.k, a.k_stride, pf);
        encode_row<BK, KBITS, true>(x, slot, a.k_codes, a.k_params, a.num_slots, a.num_kv_heads,
                                    a.page_log2, h, ql, 4, STAGED ? &stage[wave][0][nst] : nullptr);

#pragma unroll
        for (int j = 0; j < 4; ++j)
            bf16x8_to_f32(RV.raw[j], x + 8 * j);
        slot = RV.valid ? RV.slot : -1;
        issue(RV, a.v, a.v_stride, pf);
        encode_row<BV, VBITS, true>(x, slot, a.v_codes, a.v_params, a.num_slots, a.num_kv_heads,
                                    a.page_log2, h, ql, 4, STAGED ? &stage[wave][1][nst] : nullptr);
        if (STAGED && ++nst == NST)
            flush();
        if (!more)
            break;
        pair = next;
    }
    if constexpr (STAGED)
        flush();
}

// bf16 paged copy: the same slot scatter with no quantisation.
__global__ __launch_bounds__(256) void bf16_paged_write_kernel(CopyArgs a)
{
    const int64_t t = (int64_t)blockIdx.x * 64 + (threadIdx.x >> 2);
    if (t >= a.num_tokens)
        return;
    const int32_t slot = a.slots[t];
    if (slot < 0 || slot >= a.num_slots)
        return;
    const int h = blockIdx.y;
    const int ql = threadIdx.x & 3;
    const int64_t page = slot >> a.page_log2;
    const int64_t off = slot & ((1 << a.page_log2) - 1);
    const int64_t cell = ((page * a.num_kv_heads + h) << a.page_log2) + off;
    const uint16_t *src = blockIdx.z == 0 ? a.k + t * a.k_stride : a.v + t * a.v_stride;
    uint16_t *dst = blockIdx.z == 0 ? a.k_cache : a.v_cache;
    const u32x4 *s4 = reinterpret_cast<const u32x4 *>(src + h * kHeadDim + 32 * ql);
    u32x4 *d4 = reinterpret_cast<u32x4 *>(dst + cell * kHeadDim + 32 * ql);
    u32x4 w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        w[j] = s4[j];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        d4[j] = w[j];
}

__global__ __launch_bounds__(256) void device_copy_kernel(u32x4 *__restrict__ dst,
                                                          const u32x4 *__restrict__ src, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        dst[i] = src[i];
}

// Streaming read of n 16-byte elements: grid-stride, four non-temporal loads in flight per
// lane, every load instruction of the grid covering one contiguous span; the words are
// folded into one value per lane that is stored only if it equals `magic` (never, for the
// data it is given), so the loads cannot be dropped and nothing is written.
__global__ __launch_bounds__(256) void device_read_kernel(const u32x4 *__restrict__ src, int64_t n,
                                                          uint32_t *sink, uint32_t magic)
{
    constexpr int U = 4;
    const int64_t nth = (int64_t)gridDim.x * blockDim.x;
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    int64_t i = 0;
    for (; (i + U) * nth <= n; i += U) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = __builtin_nontemporal_load(src + (i + u) * nth + tid);
#pragma unroll
        for (int u = 0; u < U; ++u)
            acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (int64_t e = i * nth + tid; e < n; e += nth) {
        const u32x4 v = __builtin_nontemporal_load(src + e);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == magic)
        *sink = acc;
}

// Page-gather read: the cache pages of a list, whole (K and V codes and parameters of every
// KV head), in list order, with non-temporal loads; the words are folded as in the streaming
// read and nothing is written.  These are the decode's bytes in the decode's page order with
// no arithmetic: the ceiling of a read over a page-scattered cache, next to the streaming
// read's ceiling over contiguous memory.  Each wave takes a contiguous share of the list's
// units (17 lines of 1 KiB: 8 of K codes, 8 of V codes, one of parameters, 512 bytes of each
// tensor) and keeps two units in flight: the next unit is issued before the current one is
// folded, so the wait before each fold covers that unit only.
struct ReadUnit {
    u32x4 v[17];
};

// Issues the loads of unit q of page index pi (scheduling barriers keep the 17 loads
// together: without them the compiler interleaves loads and folds and keeps only a few
// loads in flight).
__device__ __forceinline__ void issue_unit(ReadUnit &U, const PagedReadArgs &a, int64_t pi, int q,
                                           int lane)
{
    __builtin_amdgcn_sched_barrier(0);
    int p = a.pages[pi];
    p = (unsigned)p < (unsigned)a.num_pages ? p : 0;
    const uint64_t unit = (uint64_t)p * (uint64_t)a.units_per_page + (uint64_t)q;
    const u32x4 *kc = reinterpret_cast<const u32x4 *>(a.k_codes + unit * 8192u) + lane;
    const u32x4 *vc = reinterpret_cast<const u32x4 *>(a.v_codes + unit * 8192u) + lane;
    const u32x4 *pr = reinterpret_cast<const u32x4 *>((lane < 32 ? a.k_params : a.v_params) +
                                                      unit * 512u) + (lane & 31);
#pragma unroll
    for (int j = 0; j < 8; ++j)
        U.v[j] = __builtin_nontemporal_load(kc + 64 * j);
#pragma unroll
    for (int j = 0; j < 8; ++j)
        U.v[8 + j] = __builtin_nontemporal_load(vc + 64 * j);
    U.v[16] = __builtin_nontemporal_load(pr);
    __builtin_amdgcn_sched_barrier(0);
}

// Folds a unit into acc where it stands: the empty asm takes acc as an operand, so the
// compiler cannot sink the folds past the next unit's loads (which would make it copy the
// unit's registers, and wait for all of its loads, before reusing them).
__device__ __forceinline__ void fold_unit(uint32_t &acc, const ReadUnit &U)
{
#pragma unroll
    for (int j = 0; j < 17; ++j)
        acc ^= U.v[j].x ^ U.v[j].y ^ U.v[j].z ^ U.v[j].w;
    asm("" : "+v"(acc));
}

__global__ __launch_bounds__(256) void paged_read_kernel(PagedReadArgs a)
{
    const int lane = threadIdx.x & 63;
    const int64_t W = (int64_t)gridDim.x * (blockDim.x >> 6);
    const int64_t w = (int64_t)blockIdx.x * (blockDim.x >> 6) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t n_units = a.num_list * a.units_per_page;
    const int64_t u0 = n_units * w / W, u1 = n_units * (w + 1) / W;
    if (u0 >= u1)
        return;
    // unit u is unit q = u % units_per_page of page index pi = u / units_per_page; (pi, q)
    // advance one unit per issue, on the scalar unit
    const int upp = a.units_per_page;
    int64_t pi = u0 / upp;
    int q = (int)(u0 - pi * upp);
    auto next = [&]() {
        if (++q == upp) {
            q = 0;
            ++pi;
        }
    };
    uint32_t acc = 0;
    ReadUnit A, B;
    issue_unit(A, a, pi, q, lane);
    next();
    int64_t u = u0;
    for (; u + 2 < u1; u += 2) {
        issue_unit(B, a, pi, q, lane);
        next();
        fold_unit(acc, A);
        issue_unit(A, a, pi, q, lane);
        next();
        fold_unit(acc, B);
    }
    if (u + 1 < u1) {
        issue_unit(B, a, pi, q, lane);
        fold_unit(acc, A);
        fold_unit(acc, B);
    } else {
        fold_unit(acc, A);
    }
    if (acc == a.magic)
        *a.sink = acc;
}

// Page-gather read per (page, KV head) block, the decode's way: workgroup (h, j) of NG
// groups reads KV head h of share j of the list, its four waves a quarter each, in blocks of
// 16 tokens (a (page, head) block at page size 16, a quarter of one at 64), NU blocks (NU / 2
// of the decode's 32-token tiles) issued before the previous NU are folded.  VW = 0: the
// decode's load shapes (16 bytes of K per lane, four 4-byte V loads per lane at the PV
// operand's offsets, one 4-byte parameter word per lane); VW = 1: V as one 16-byte load per
// lane (whole lines).  The same bytes as the whole-page read, in units of 2,176 bytes.
template <int VW>
struct BlockUnit {
    u32x4 k;
    u32x4 v;
    uint32_t par;
};

template <int VW>
__device__ __forceinline__ void issue_block(BlockUnit<VW> &U, const PagedReadArgs &a, int64_t u,
                                            int qpp, int h, int lane)
{
    __builtin_amdgcn_sched_barrier(0);
    const int64_t pi = u / qpp;
    int p = a.pages[pi];
    p = (unsigned)p < (unsigned)a.num_pages ? p : 0;
    const uint64_t cell = ((uint64_t)p * a.num_kv_heads + h) * a.page_size + 16 * (uint64_t)(u - pi * qpp);
    const uint8_t *kb = a.k_codes + cell * kRowCodeBytes, *vb = a.v_codes + cell * kRowCodeBytes;
    U.k = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(kb) + lane);
    if constexpr (VW == 1) {
        U.v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(vb) + lane);
    } else {
        const uint32_t *v32 = reinterpret_cast<const uint32_t *>(vb + 256 * (lane >> 4) + 4 * (lane & 15));
        U.v.x = __builtin_nontemporal_load(v32);
        U.v.y = __builtin_nontemporal_load(v32 + 16);
        U.v.z = __builtin_nontemporal_load(v32 + 32);
        U.v.w = __builtin_nontemporal_load(v32 + 48);
    }
    const uint8_t *pb = lane < 32 ? a.k_params : a.v_params;
    U.par = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(pb) + cell + (lane & 15));
    __builtin_amdgcn_sched_barrier(0);
}

template <int VW>
__device__ __forceinline__ void fold_block(uint32_t &acc, const BlockUnit<VW> &U)
{
    acc ^= U.k.x ^ U.k.y ^ U.k.z ^ U.k.w ^ U.v.x ^ U.v.y ^ U.v.z ^ U.v.w ^ U.par;
    asm("" : "+v"(acc));
}

template <int VW, int NU>
__global__ __launch_bounds__(256) void paged_read_blocks_kernel(PagedReadArgs a)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int NG = gridDim.x / a.num_kv_heads;
    const int h = blockIdx.x / NG, j = blockIdx.x - h * NG;
    if (h >= a.num_kv_heads)
        return;
    const int qpp = a.page_size / 16;
    const int64_t n = a.num_list * qpp;
    const int64_t g0 = n * j / NG, g1 = n * (j + 1) / NG;
    const int64_t w0 = g0 + (g1 - g0) * wave / 4, w1 = g0 + (g1 - g0) * (wave + 1) / 4;
    if (w0 >= w1)
        return;
    // past the share's end the last block is read again (in flight, not counted)
    auto cl = [&](int64_t u) { return u < w1 ? u : w1 - 1; };
    uint32_t acc = 0;
    BlockUnit<VW> X[NU], Y[NU];
#pragma unroll
    for (int k = 0; k < NU; ++k)
        issue_block(X[k], a, cl(w0 + k), qpp, h, lane);
    int64_t u = w0;
    for (; u + NU < w1; u += 2 * NU) {
#pragma unroll
        for (int k = 0; k < NU; ++k)
            issue_block(Y[k], a, cl(u + NU + k), qpp, h, lane);
#pragma unroll
        for (int k = 0; k < NU; ++k)
            fold_block(acc, X[k]);
#pragma unroll
        for (int k = 0; k < NU; ++k)
            issue_block(X[k], a, cl(u + 2 * NU + k), qpp, h, lane);
#pragma unroll
        for (int k = 0; k < NU; ++k)
            fold_block(acc, Y[k]);
    }
#pragma unroll
    for (int k = 0; k < NU; ++k)
        fold_block(acc, X[k]);
    if (acc == a.magic)
        *a.sink = acc;
}

// Persistent grid: enough workgroups for a few resident waves per SIMD, each wave
// then walks several tiles so its next loads overlap its current arithmetic.
unsigned write_grid(const WriteArgs &a, int wgs_per_cu)
{
    const int cus = device_cus();
    // one wave per (K, V) tile pair at most, four waves per workgroup
    const int64_t pairs = (a.num_tokens + kWriteTile - 1) / kWriteTile * a.num_kv_heads;
    const int64_t wgs = (pairs + 3) / 4;
    const int64_t cap = (int64_t)cus * wgs_per_cu;
    return (unsigned)(wgs < cap ? wgs : cap);
}

template <int BK, int BV>
hipError_t launch_bk_bv(const WriteArgs &a, hipStream_t s)
{
    // the code widths are template arguments, so each kernel carries one encoder per tensor
    // staged when every wave of the two-workgroups-per-CU grid has a full stage of pairs to
    // encode (4-bit pools); otherwise the grid takes three workgroups per CU
    const int64_t pairs = (a.num_tokens + kWriteTile - 1) / kWriteTile * a.num_kv_heads;
    const unsigned grid2 = write_grid(a, kWriteWgsPerCu);
    const bool staged = a.k_bits != 2 && a.v_bits != 2 && pairs >= (int64_t)kWriteStage * 4 * grid2;
    const dim3 grid(staged ? grid2 : write_grid(a, kWriteWgsPerCuUnstaged));
    if (a.k_bits == 2 && a.v_bits == 2)
        hipLaunchKernelGGL((rotquant_write_kernel<BK, BV, 2, 2, false>), grid, dim3(256), 0, s, a);
    else if (a.k_bits == 2)
        hipLaunchKernelGGL((rotquant_write_kernel<BK, BV, 2, 4, false>), grid, dim3(256), 0, s, a);
    else if (a.v_bits == 2)
        hipLaunchKernelGGL((rotquant_write_kernel<BK, BV, 4, 2, false>), grid, dim3(256), 0, s, a);
    else if (staged)
        hipLaunchKernelGGL((rotquant_write_kernel<BK, BV, 4, 4, true>), grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((rotquant_write_kernel<BK, BV, 4, 4, false>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int BK>
hipError_t launch_bv(int v_block, const WriteArgs &a, hipStream_t s)
{
    switch (v_block) {
    case 0: return launch_bk_bv<BK, 0>(a, s);
    case 16: return launch_bk_bv<BK, 16>(a, s);
    case 32: return launch_bk_bv<BK, 32>(a, s);
    case 64: return launch_bk_bv<BK, 64>(a, s);
    case 128: return launch_bk_bv<BK, 128>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

int device_cus()
{
    static int cus = 0;
    if (cus == 0) {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cus = n;
    }
    return cus;
}

int launch_rotquant_write(int k_block, int v_block, const WriteArgs &a, void *stream)
{
    if (a.num_tokens == 0)
        return 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (k_block) {
    case 0: return launch_bv<0>(v_block, a, s);
    case 16: return launch_bv<16>(v_block, a, s);
    case 32: return launch_bv<32>(v_block, a, s);
    case 64: return launch_bv<64>(v_block, a, s);
    case 128: return launch_bv<128>(v_block, a, s);
    default: return hipErrorInvalidValue;
    }
}

int launch_bf16_paged_write(const CopyArgs &a, void *stream)
{
    if (a.num_tokens == 0)
        return 0;
    const dim3 grid((unsigned)((a.num_tokens + 63) / 64), (unsigned)a.num_kv_heads, 2);
    hipLaunchKernelGGL(bf16_paged_write_kernel, grid, dim3(256), 0, static_cast<hipStream_t>(stream), a);
    return hipGetLastError();
}

int launch_device_copy(void *dst, const void *src, size_t bytes, void *stream)
{
    const int64_t n = (int64_t)(bytes / 16);
    if (n == 0)
        return 0;
    // one 16-byte element per lane, one-shot: the fastest plain copy measured (6.2 TB/s on
    // 1 GiB, against 4.6-4.8 for grid-stride loops of 2k-16k workgroups)
    int64_t blocks = (n + 255) / 256;
    if (blocks > 0x7FFFFFFF)
        blocks = 0x7FFFFFFF;
    hipLaunchKernelGGL(device_copy_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<u32x4 *>(dst),
                       static_cast<const u32x4 *>(src), n);
    return hipGetLastError();
}

int launch_device_read(const void *src, size_t bytes, uint32_t *sink, void *stream)
{
    const int64_t n = (int64_t)(bytes / 16);
    if (n == 0)
        return 0;
    // two 256-lane workgroups per CU (eight waves): the fastest streaming read measured
    // (7.0 TB/s on 3 GiB, against 6.3 with four and 5.7 with sixteen waves per CU)
    const int64_t blocks = std::min<int64_t>((int64_t)device_cus() * 2, (n + 255) / 256);
    hipLaunchKernelGGL(device_read_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4 *>(src), n, sink,
                       0x9E3779B9u);
    return hipGetLastError();
}

int launch_paged_read(const PagedReadArgs &a, int wgs_per_cu, void *stream)
{
    if (a.num_list == 0)
        return 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (a.pattern == 0) {
        hipLaunchKernelGGL(paged_read_kernel, dim3((unsigned)(device_cus() * wgs_per_cu)), dim3(256), 0, s, a);
    } else {
        // whole groups of Hkv workgroups, as the balanced decode
        const int groups = std::max(1, device_cus() * wgs_per_cu / a.num_kv_heads);
        const dim3 grid((unsigned)(groups * a.num_kv_heads));
        if (a.pattern == 1)
            hipLaunchKernelGGL((paged_read_blocks_kernel<0, 4>), grid, dim3(256), 0, s, a);
        else if (a.pattern == 2)
            hipLaunchKernelGGL((paged_read_blocks_kernel<1, 4>), grid, dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((paged_read_blocks_kernel<0, 8>), grid, dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

const char *hip_error_string(int err)
{
    return hipGetErrorString(static_cast<hipError_t>(err));
}

}  // namespace kvrq
