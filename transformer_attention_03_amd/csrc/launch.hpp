// Kernel parameter blocks and launchers shared between the host API and the kernels.
// The fields mirror the attention parameter block of doppler (gpu/kernels/attention.js,
// createAttentionUniformBuffer), passed by value as kernel arguments instead of a uniform
// buffer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ta03 {

struct DecodeParams {
    const float* q;            // [B][H][D] f32
    const void* k;             // f16 [Hkv][kv_len][D]  or  int8 pages [P][16][Hkv][D]
    const void* v;
    const float* k_scales;     // paged: [P][16][Hkv]
    const float* v_scales;
    const int32_t* page_table; // paged: [B][max_pages]
    const int32_t* kv_lens;    // paged: [B] (device)
    float* o;                  // [B][H][D] f32
    float* part_o;             // [B][H][n_split_max][D]
    float* part_m;             // [B][H][n_split_max]
    float* part_l;             // [B][H][n_split_max]
    uint32_t* tickets;         // [B][Hkv * head_chunks], zero between calls
    int H, Hkv;
    int group, nch;            // query heads per KV head; head chunks (workgroups) per KV head
    unsigned long long nch_inv; // ceil(2^32 / nch): y / nch = (y * nch_inv) >> 32 for y < 2^16
    int kv_len;                // contiguous cache length (unused when paged); ring: tokens so far
    int ring;                  // ring cache capacity in tokens (token t at row t mod ring); 0 = none
    int num_pages, max_pages;
    int window;
    float scale, scale_log2;   // scale and scale * log2(e)
    float softcap, inv_softcap;
    int split_tokens;          // contiguous: logical tokens per workgroup
    int n_split_max;           // split partials per (sequence, head): workspace row stride
    int batch;                 // paged: sequences
    int n_wg;                  // paged: workgroups per head chunk (grid.x)
    // tiered (one sequence): k, v, k_scales, v_scales, page_table hold the int8 paged cold
    // tier with positions [0, tier_cold_len); hot_k, hot_v the f16 ring [Hkv][ring][D] with
    // position t at row (t + ring_off) mod ring; kv_len = all positions
    const void* hot_k;
    const void* hot_v;
    int ring_off;
    int tier_cold_len;
    int tier_cold_splits;      // workgroups [0, tier_cold_splits) take cold splits
    int tier_k_lo;             // first visible position
    int tier_cold_tokens;      // tokens per cold split (split_tokens: per hot split)
    int tier_cold_stride;      // contiguous cold tier: rows per KV head
};

struct FwdParams {
    const void* q;             // element strides below
    const void* k;
    const void* v;
    void* o;
    long q_row, q_head;        // strides (elements) between query rows / query heads
    long k_row, k_head;        // same for K and V
    long o_row, o_head;
    int seq_len, kv_len;
    int H, Hkv;
    int causal, window;
    float scale, scale_log2;
    float softcap, inv_softcap;
    int n_qblocks;             // query blocks per head
    const int32_t* kv_len_dev; // optional: the kv length, read on the device (kv_len is then its maximum)
};

struct BlockLocalParams {
    const float* q;            // [padded_len][H * 128]
    const float* k;            // [kv_rows][H * 128], row r = position r - pad_left
    const float* v;
    const float* pos;          // [max_past + max_future + 1][H * 128]
    float* o;                  // [padded_len][H * 128]
    int seq, padded_len, H;
    int max_past, max_future, pad_left;
    float cap, inv_cap;        // logit cap (0 = off) and its inverse
};

hipError_t launch_block_local(const BlockLocalParams& p, hipStream_t st);
int block_local_max_span();
int block_local_head_dim();

hipError_t launch_decode(const DecodeParams& p, int head_dim, int gc, bool paged, int batch,
                         hipStream_t st);
int decode_tokens_per_block();
int decode_waves(int head_dim, bool paged);
int decode_max_heads_per_workgroup();
int decode_workgroups_per_cu(int head_dim, bool paged);
int decode_max_splits();
int decode_max_split_tokens_paged();
// tiered decode: grid (n_splits, Hkv * head chunks); the cold tier is int8 (with per-row
// scales) or f16, paged or contiguous
hipError_t launch_decode_tiered(const DecodeParams& p, int head_dim, int gc, int n_splits, bool cold_int8,
                                bool cold_paged, hipStream_t st);

// Library-owned decode scratch of this GPU (the device of `st`, or the current device for
// the null stream): its device address, looked up once per device.
hipError_t decode_scratch(void** ptr, hipStream_t st);
size_t decode_scratch_bytes();
// n uint32 words set to zero by a kernel on `st`
hipError_t zero_words(uint32_t* p, int n, hipStream_t st);

// dtype: 0 f32, 1 f16
hipError_t launch_fwd(const FwdParams& p, int head_dim, int dtype, hipStream_t st);
// query rows per workgroup for this call shape (the launcher picks the same configuration)
int fwd_block_rows(int head_dim, int dtype, int seq_len, int H);

}  // namespace ta03
