// Launch interface between the C ABI layer (pa_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

enum : int { kF16 = 0, kBF16 = 1 };   // 16-bit element types

struct ReshapeArgs {
    const void* key;
    const void* value;
    void* k_cache;
    void* v_cache;
    const int64_t* slot_mapping;
    int64_t num_tokens;
    int64_t num_slots;       // num_blocks * block_size
    int32_t row_vecs;        // 16-byte vectors per token row (kv_heads * head_dim / 8)
    // slots from the block table instead (slot_mapping nullptr): token t is the
    // newest of sequence t, at position seq_lens[t] - 1 (clamped to the row)
    const int32_t* block_tables;
    const int32_t* seq_lens;
    int32_t table_stride;
    int32_t block_size;
};
hipError_t launch_reshape_and_cache(const ReshapeArgs& a, hipStream_t stream);

// Cache write into an FP8 (E4M3) cache: per (token, kv head) row, scale =
// amax / 448 and codes = e4m3(x / scale).
struct ReshapeFp8Args {
    const void* key;
    const void* value;
    uint8_t* k_cache;        // [NB][16][Hkv][D] codes
    uint8_t* v_cache;
    float* k_scales;         // [NB][Hkv][16]
    float* v_scales;
    const int64_t* slot_mapping;
    int64_t num_tokens;
    int64_t num_slots;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t dtype;           // type of key / value
};
hipError_t launch_reshape_and_cache_fp8(const ReshapeFp8Args& a, hipStream_t stream);

struct CopyBlocksArgs {
    void* k_cache;
    void* v_cache;
    const int64_t* block_pairs;   // [num_pairs][2] = (src, dst)
    int64_t num_pairs;
    int64_t num_blocks;
    int64_t block_vecs;           // 16-byte vectors per block (block_size * kv_heads * head_dim / 8)
    int64_t wgs_per_pair;         // workgroups per pair (1024 vectors each)
};
hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream);

struct DecodeArgs {
    void* out;
    const void* q;
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_tables;   // [num_seqs][table_stride]
    const int32_t* seq_lens;
    float* ws_acc;           // [B][Hq][num_parts][D]
    float2* ws_ml;           // [B][Hq][num_parts] = (max, sum), log2 domain
    int32_t num_seqs;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t group;           // q heads per kv head
    int32_t gqa_mfma;        // 1: QK^T on matrix cores (head_dim 128, group 3..16)
    int32_t heads_per_wave;  // q heads one wave carries (1, 2, 4, 8; 16 with gqa_mfma)
    int32_t head_chunks;     // ceil(group / heads_per_wave)
    int32_t head_dim;
    int32_t max_blocks_per_seq;   // 16-token blocks per sequence (table_stride << block_shift)
    int64_t num_blocks;           // 16-token blocks in the pool
    int32_t table_stride;         // entries per block-table row
    int32_t block_shift;          // log2(cache block size / 16): 0 or 1 (sub_block)
    int32_t part_blocks;     // partition length in blocks
    int32_t num_parts;       // partitions per sequence the grid covers
    float scale_log2;        // softmax scale times log2(e)
    int32_t dtype;
    int32_t stream_kv;       // 1: no block is read twice in this call; stream K/V
    // FP8 cache only: per (block, kv head, token) float32 scales
    const float* k_scales;   // [NB][Hkv][16]
    const float* v_scales;
    // several queries per sequence (draft verification): column c of a kv head
    // is query c / group, q head c % group; 1 and group for plain decode
    int32_t q_per_seq;
    int32_t cols;
    // balanced split (single query): the waves share the blocks of all units
    // evenly instead of taking fixed partitions; num_items = waves launched
    int32_t balanced;
    int32_t num_items;
    int32_t state_heads;     // balanced: head slots per partial-state slot, min(heads_per_wave, cols)
    // sequence groups (shared prefixes; balanced split on matrix cores):
    // seqs_per_wave > 1 consecutive sequences share one wave, 16 / group
    // columns' worth (column c: member c / group, head c % group).  The
    // balanced stream then runs over owners, group after group: the group's
    // shared blocks, then each member's blocks past them; owner_blocks[o]
    // holds the counts (the plan kernel writes them).  A shared segment leaves
    // the states of its 16 columns at slots
    // shared_base + ((group + stretch) * num_kv_heads + g) * 16 + column.
    int32_t seqs_per_wave;
    int64_t shared_base;
    int32_t* owner_blocks;
    // the decode step's cache write, done by the decode itself (pa_decode_step):
    // new_k / new_v [num_seqs][Hkv][D] hold each sequence's newest token, at
    // position seq_len - 1; the wave that reads that token's block takes the
    // row from here and stores it to its slot (nullptr: no write)
    const void* new_k;
    const void* new_v;
};
hipError_t launch_decode_partitions(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_group_plan(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_grouped(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_grouped_fp8(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_partitions_fp8(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_merge(const DecodeArgs& a, hipStream_t stream);

struct PrefillArgs {
    void* out;
    const void* q;
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_tables;
    const int32_t* ctx_lens;
    const int32_t* query_start_loc;
    int32_t num_seqs;
    int64_t num_tokens;
    int32_t max_q_len;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t group;
    int32_t max_blocks_per_seq;   // 16-token blocks per sequence (table_stride << block_shift)
    int64_t num_blocks;           // 16-token blocks in the pool
    int32_t table_stride;         // entries per block-table row
    int32_t block_shift;          // log2(cache block size / 16): 0 or 1 (sub_block)
    float scale_log2;
    int32_t dtype;
    int32_t head_dim;        // 64 or 128
    // FP8 cache only: per (block, kv head, token) float32 scales
    const float* k_scales;   // [NB][Hkv][16]
    const float* v_scales;
};
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_prefill_fp8(const PrefillArgs& a, hipStream_t stream);

// Debug builds (PA_DEBUG_BOUNDS): before a call's own kernels, one small kernel
// checks the device-resident indices the call is about to use and sets bits
// of a device word for what it finds out of range (the bit values of pa.h).
enum : uint32_t { kBoundsBlockId = 1u, kBoundsSeqLen = 2u, kBoundsSlot = 4u, kBoundsQueryRange = 8u };
enum : int32_t { kBoundsDecode = 0, kBoundsPrefill = 1, kBoundsSlots = 2, kBoundsPairs = 3 };
struct BoundsArgs {
    uint32_t* word;
    int32_t kind;
    const int32_t* block_tables;      // decode, prefill
    const int32_t* seq_lens;          // decode: tokens of each sequence
    const int32_t* ctx_lens;          // prefill
    const int32_t* query_start_loc;   // prefill
    const int64_t* indices;           // slots (cache write) or (src, dst) pairs (block copy)
    int64_t count;                    // sequences, tokens or pairs
    int64_t num_tokens;               // prefill: packed query rows
    int64_t limit;                    // 16-token blocks in the pool, or slots for a cache write
    int32_t table_stride;
    int32_t block_shift;
    int32_t max_blocks16;             // 16-token blocks a table row can name
    int32_t max_q_len;
};
hipError_t launch_bounds_check(const BoundsArgs& a, hipStream_t stream);

}  // namespace pa
