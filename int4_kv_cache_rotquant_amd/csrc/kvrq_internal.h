// Internal interface between the C-ABI layer (kvrq_abi.cpp) and the HIP
// launchers (kvrq_write.hip, kvrq_decode.hip).  Plain types only; every
// shape has been validated by the ABI layer before a launcher is called.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace kvrq {

constexpr int kHeadDim = 128;       // channels per head
constexpr int kRowCodeBytes = 64;   // packed INT4 bytes per (token, head) row (2-bit: 32)
constexpr int kTile = 32;           // decode tokens per inner step
constexpr int kWriteTile = 16;      // write tokens per wave step (four lanes per row)
// write waves per SIMD: two, each walking twice as many tiles as at five (measured on
// MI355X: the 32k-token chunk 35.9 -> 34.7 us, the Qwen3-4B-like write 45.3 -> 42.7 us with
// the temporal parameter stores; one wave per SIMD leaves the rotation exposed)
constexpr int kWriteWavesPerSimd = 2;
// persistent write grid: 256-lane workgroups per CU, one wave per SIMD each, so all of them
// are resident at once (one more, waiting for a slot, measured 8% slower on 16k-token chunks)
constexpr int kWriteWgsPerCu = kWriteWavesPerSimd;
// a write that stores as it goes (too few tile pairs per wave to stage them) runs three
// workgroups per CU (its 104 VGPRs allow four): the 16k-token long-context chunk 19.67 ->
// 19.34 us against two, four no faster (measured on MI355X, same machine)
constexpr int kWriteWgsPerCuUnstaged = 3;
constexpr int kWriteStage = 8;      // tile pairs per wave staged in LDS by the staged write
constexpr int kMaxGroup = 16;       // query heads per KV head handled by one decode wave
constexpr int kDecodeWaves = 4;     // waves per decode workgroup, each on its own token range
constexpr int kExtendBlocks = 2;    // extend: 16-column blocks per wave (query rows x heads)
// split workspaces start with this many int32 split counters (used by the split decode when
// sequences x KV heads fits them, its grid is resident at once and a row has at most
// kInKernelCombineSplits splits, and by the balanced decode); the partials follow
constexpr int kSplitCounters = 16384;
constexpr size_t kCounterBytes = size_t(kSplitCounters) * 4;
constexpr int kInKernelCombineSplits = 16;   // most splits per row merged inside the split launch
// the balanced decode keeps the tiles per sequence (prefix sums) in LDS: at most this many
// sequences
constexpr int kBalancedMaxSeqs = 1024;
// most workgroups of the balanced decode (its workspace is sized for this many)
constexpr int kBalancedMaxWgs = 2048;
// waves per SIMD (workgroups per CU) of the balanced decode with up to eight query heads per
// KV head: two, so that its segment loop fits the register file without spilling (~180
// VGPRs; the split kernel measured the same at two, three and four)
constexpr int kBalancedWavesF2 = 2;
// waves per SIMD of the split decode with up to eight query heads per KV head (its tile walk,
// the page-id window and the epilogue take ~140 VGPRs)
constexpr int kSplitWavesF2 = 3;

struct WriteArgs {
    const uint16_t *k;          // bf16 bits
    const uint16_t *v;
    int64_t num_tokens;
    int64_t k_stride;           // elements between tokens
    int64_t v_stride;
    const int32_t *slots;
    uint8_t *k_codes;
    uint8_t *v_codes;
    uint32_t *k_params;         // (scale | zero << 16) binary16 pairs
    uint32_t *v_params;
    int64_t num_slots;          // num_pages * page_size; slots at or above are skipped
    int32_t num_kv_heads;
    int32_t page_log2;
    int32_t k_bits = 4;         // code widths of the pools: 4, or 2 (32-byte rows)
    int32_t v_bits = 4;
};

struct CopyArgs {
    const uint16_t *k;
    const uint16_t *v;
    int64_t num_tokens;
    int64_t k_stride;
    int64_t v_stride;
    const int32_t *slots;
    uint16_t *k_cache;          // bf16 [pages][Hkv][P][128]
    uint16_t *v_cache;
    int64_t num_slots;
    int32_t num_kv_heads;
    int32_t page_log2;
};

// Page-gather read (a measurement kernel): the cache pages of a list, in list order.
// Pattern 0 reads whole pages per wave, as units of 17 lines of 1 KiB (8 lines of K codes,
// 8 of V codes, one of parameters: 512 bytes of K, 512 of V), units_per_page per page.
// Patterns 1 to 3 read per (page, KV head) block of 16 tokens as the decode does (one
// workgroup per KV head and share of the list); 1 with the decode's load shapes and depth
// (two 32-token tiles in flight per wave), 2 with 16-byte V loads, 3 with the decode's
// shapes and four tiles in flight.
struct PagedReadArgs {
    const uint8_t *k_codes;
    const uint8_t *v_codes;
    const uint8_t *k_params;
    const uint8_t *v_params;
    const int32_t *pages;       // [num_list]; ids outside [0, num_pages) read page 0
    int64_t num_list;
    int32_t units_per_page;     // pattern 0: num_kv_heads * page_size / 128
    int32_t num_pages;
    int32_t num_kv_heads;
    int32_t page_size;
    int32_t pattern;            // 0 .. 3
    uint32_t *sink;
    uint32_t magic;
};

struct DecodePlan {
    int32_t split_tokens;       // tokens per workgroup, multiple of kTile * kDecodeWaves
    int32_t max_splits;         // ceil(max_seq_len / split_tokens), >= 1
    int32_t balanced_wgs = 0;   // > 0: the balanced decode with this many workgroups (at
                                // most kBalancedMaxWgs; the split plan is then unused)
};

struct DecodeArgs {
    const uint8_t *k_codes;
    const uint8_t *v_codes;
    const uint32_t *k_params;
    const uint32_t *v_params;
    const uint16_t *q;          // bf16 [S][Hq][128]
    const int32_t *page_table;  // [S][max_pages]
    const int32_t *seq_lens;    // [S]
    float *out;                 // [S][Hq][128]
    // decode with 2..kInKernelCombineSplits splits in a grid resident at once: one counter
    // per (sequence, KV head), zero on entry and on exit; the split workgroup that counts
    // last merges the partials (no combine launch)
    int32_t *counters = nullptr;
    float *part_o = nullptr;    // [S][Hq][max_splits][128]
    float *part_ml = nullptr;   // [S][Hq][max_splits][2]
    int32_t num_seqs;
    int32_t num_pages;          // page ids outside [0, num_pages) read page 0 instead
    int32_t max_seq_len;        // longer seq_lens entries are clamped to it
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t group;              // Hq / Hkv
    int32_t page_log2;
    int32_t max_pages;
    int32_t split_tokens;
    int32_t max_splits;
    // decode grid order: 0 = (split, KV head, sequence), 1 = (sequence, KV head, split)
    int32_t seq_major = 0;
    // > 0: the balanced decode, one resident round of this many workgroups (NG groups of
    // Hkv, group j's share of the (sequence, tile) columns read by one workgroup per KV
    // head); its partials are indexed by slot = (j + sequence) * Hkv + KV head,
    // [slot][G][128] and [slot][G][2]
    int32_t balanced_wgs = 0;
    // balanced decode: 1 = a combine launch merges the pairs of several shares (pairs span
    // many groups), 0 = the last workgroup of each pair merges it
    int32_t balanced_combine = 0;
    float q_scale;              // sm_scale * log2(e)
    // extend (chunked prefill) only; qo_start == nullptr for the decode.  The output
    // rows are then query rows: q, out [total_q][Hq][128], part_* [total_q][Hq][splits]
    const int32_t *qo_start = nullptr;  // [S + 1] first query row of each sequence
    int32_t num_rows;           // rows of the combine: S (decode) or total_q (extend)
    int32_t rows_per_block;     // query rows per workgroup (32 / group, at least 1)
    int32_t blocks_per_seq;     // ceil(max_q_len / rows_per_block)
    // fused decode step only (new_slots == nullptr otherwise): each sequence's new token,
    // written by the workgroup whose split holds position seq_len - 1, before it reads
    const int32_t *new_slots = nullptr;  // [S] slot of the new token (negative: not written)
    const uint16_t *k_new = nullptr;     // bf16 rows [S][Hkv][128], token strides below
    const uint16_t *v_new = nullptr;
    int64_t k_new_stride = 0;            // elements
    int64_t v_new_stride = 0;
    uint8_t *k_codes_w = nullptr;        // the same cache as k_codes ..., writable
    uint8_t *v_codes_w = nullptr;
    uint32_t *k_params_w = nullptr;
    uint32_t *v_params_w = nullptr;
    int64_t num_slots = 0;               // num_pages * page_size
    int32_t v_block = 0;
    // code widths of the two pools: 4, or 2 (32-byte rows, widened to the 4-bit layout
    // in registers)
    int32_t k_bits = 4;
    int32_t v_bits = 4;
};

// bytes of the static decode scratch behind kv_int4_paged_decode_noalloc (per device)
constexpr size_t kNoallocScratchBytes = size_t(32) << 20;

// Returns a hipError_t value (0 = success).
int launch_rotquant_write(int k_block, int v_block, const WriteArgs &a, void *stream);
int launch_bf16_paged_write(const CopyArgs &a, void *stream);
int launch_device_copy(void *dst, const void *src, size_t bytes, void *stream);
int launch_device_read(const void *src, size_t bytes, uint32_t *sink, void *stream);
int launch_paged_read(const PagedReadArgs &a, int wgs_per_cu, void *stream);
// decode, or extend when a.qo_start is set
int launch_decode(int k_block, int v_block, const DecodeArgs &a, void *stream);
// workgroups of one resident round of the balanced decode (kBalancedWavesF2 per CU; two for
// more than eight query heads per KV head)
int decode_resident_wgs(int group);
const char *hip_error_string(int err);
// device address of the static decode scratch on the current device (looked up, and its
// counters cleared on `stream`, on the first call for that device)
int noalloc_scratch(void **ptr, void *stream);
// compute units of the current device (read once per process; 256 if the query fails)
int device_cus();

}  // namespace kvrq
