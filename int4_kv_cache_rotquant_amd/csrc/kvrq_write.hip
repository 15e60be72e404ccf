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
// five waves per SIMD resident, enough to cover memory latency with arithmetic.
//
// Bit-exactness: every step runs in IEEE binary32 in a fixed order --
// butterfly widths 1, 2, 4, ... with (u+w, u-w), then * fp32(1/sqrt b); exact
// min/max; correctly rounded (mx-mn)/15 and 1/scale; round-to-nearest-even
// binary16 parameters; codes from the stored parameters.  Contraction is
// disabled for this file (-ffp-contract=off) so no multiply-add is fused.
#include <hip/hip_runtime.h>

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
// head, pair i covering head i % num_kv_heads, so waves that run side by side read all
// heads of the same tokens (whole 2 KB-per-token input rows at once).  The loop is
// unrolled over the two tensors, so each half is compiled for its own block size, and
// K and V work is spread evenly over the waves.
template <int BK, int BV, int KBITS, int VBITS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kWriteWavesPerSimd)))
void rotquant_write_kernel(WriteArgs a)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ql = lane & 3;
    const int row = lane >> 2;
    const int64_t tiles_per_head = (a.num_tokens + kWriteTile - 1) / kWriteTile;
    const int64_t num_pairs = tiles_per_head * a.num_kv_heads;
    const int64_t stride_w = (int64_t)gridDim.x * (blockDim.x >> 6);
    int64_t pair = (int64_t)blockIdx.x * (blockDim.x >> 6) + wave;
    if (pair >= num_pairs)
        return;

    auto issue = [&](RowLoad &R, const uint16_t *src, int64_t stride, int64_t pr) {
        const int64_t tt = pr / a.num_kv_heads;
        const int64_t h = pr - tt * a.num_kv_heads;
        load_row(R, src + h * kHeadDim, stride, a.slots, tt * kWriteTile + row, a.num_tokens, ql);
    };

    // Two register sets, K and V: each is refilled with the next pair's tile as soon as
    // its bf16 input is widened to fp32, so up to two tiles are in flight while one is
    // encoded.
    RowLoad RK, RV;
    issue(RK, a.k, a.k_stride, pair);
    issue(RV, a.v, a.v_stride, pair);
    while (true) {
        const int h = (int)(pair % a.num_kv_heads);
        const int64_t next = pair + stride_w;
        const bool more = next < num_pairs;
        const int64_t pf = more ? next : pair;   // past the end: re-read this pair (no store)
        float x[32];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            bf16x8_to_f32(RK.raw[j], x + 8 * j);
        int32_t slot = RK.valid ? RK.slot : -1;
        issue(RK, a.k, a.k_stride, pf);
        encode_row<BK, KBITS>(x, slot, a.k_codes, a.k_params, a.num_slots, a.num_kv_heads,
                              a.page_log2, h, ql);

#pragma unroll
        for (int j = 0; j < 4; ++j)
            bf16x8_to_f32(RV.raw[j], x + 8 * j);
        slot = RV.valid ? RV.slot : -1;
        issue(RV, a.v, a.v_stride, pf);
        encode_row<BV, VBITS>(x, slot, a.v_codes, a.v_params, a.num_slots, a.num_kv_heads,
                              a.page_log2, h, ql);
        if (!more)
            break;
        pair = next;
    }
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

// Persistent grid: enough workgroups for a few resident waves per SIMD, each wave
// then walks several tiles so its next loads overlap its current arithmetic.
unsigned write_grid(const WriteArgs &a)
{
    const int cus = device_cus();
    // one wave per (K, V) tile pair at most, four waves per workgroup
    const int64_t pairs = (a.num_tokens + kWriteTile - 1) / kWriteTile * a.num_kv_heads;
    const int64_t wgs = (pairs + 3) / 4;
    const int64_t cap = (int64_t)cus * kWriteWgsPerCu;
    return (unsigned)(wgs < cap ? wgs : cap);
}

template <int BK, int BV>
hipError_t launch_bk_bv(const WriteArgs &a, hipStream_t s)
{
    // the code widths are template arguments, so each kernel carries one encoder per tensor
    const dim3 grid(write_grid(a));
    if (a.k_bits == 2 && a.v_bits == 2)
        hipLaunchKernelGGL((rotquant_write_kernel<BK, BV, 2, 2>), grid, dim3(256), 0, s, a);
    else if (a.k_bits == 2)
        hipLaunchKernelGGL((rotquant_write_kernel<BK, BV, 2, 4>), grid, dim3(256), 0, s, a);
    else if (a.v_bits == 2)
        hipLaunchKernelGGL((rotquant_write_kernel<BK, BV, 4, 2>), grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((rotquant_write_kernel<BK, BV, 4, 4>), grid, dim3(256), 0, s, a);
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

const char *hip_error_string(int err)
{
    return hipGetErrorString(static_cast<hipError_t>(err));
}

}  // namespace kvrq
