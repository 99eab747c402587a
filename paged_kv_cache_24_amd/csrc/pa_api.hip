// C ABI of libpa: host-side validation, kernel selection and launch.
//
// Every check runs before anything is enqueued ("fail early": unsupported
// configurations are refused at the boundary, not deep inside a kernel --
// "Hardware abstraction and portability", §九 on early capability checks).
// No call reads device memory, synchronises or allocates, so each call is
// capturable in a HIP graph; the decode workspace is owned by the caller.
#include <algorithm>
#include <atomic>
#include <math.h>
#include <mutex>
#include <stdint.h>

#include "kernels.h"
#include "pa.h"

// Static scratch of pa_decode_noalloc: the split-KV partial states of callers
// that cannot allocate.  Every GPU the library runs on holds its own copy
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not device memory: its device address is looked up once per device with
// hipGetSymbolAddress, and only that address is ever handed to a kernel.
static __device__ __align__(256) float scratch[PA_NOALLOC_SCRATCH_BYTES / sizeof(float)];

#ifdef PA_DEBUG_BOUNDS
// Debug builds: the word the index checks set bits in (one per device, like
// `scratch`; read and cleared by pa_debug_bounds).
static __device__ uint32_t debug_word;
static_assert(pa::kBoundsBlockId == PA_DEBUG_BLOCK_ID && pa::kBoundsSeqLen == PA_DEBUG_SEQ_LEN &&
                  pa::kBoundsSlot == PA_DEBUG_SLOT && pa::kBoundsQueryRange == PA_DEBUG_QUERY_RANGE,
              "the kernels' bits are the header's");
#endif

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mutex;

// Device address of the current device's copy of a __device__ variable, looked
// up once per device and kept in `cache`; nullptr when the device cannot be
// queried or the symbol cannot be resolved.
template <class Symbol>
void* symbol_address(std::atomic<void*> (&cache)[kMaxDevices], const Symbol& symbol) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void* ptr = cache[dev].load(std::memory_order_acquire);
    if (ptr) return ptr;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    ptr = cache[dev].load(std::memory_order_relaxed);
    if (!ptr) {
        if (hipGetSymbolAddress(&ptr, symbol) != hipSuccess) return nullptr;
        cache[dev].store(ptr, std::memory_order_release);
    }
    return ptr;
}

void* scratch_address() { return symbol_address(g_scratch_addr, HIP_SYMBOL(scratch)); }

#ifdef PA_DEBUG_BOUNDS
std::atomic<void*> g_debug_addr[kMaxDevices];
uint32_t* debug_word_address() {
    return static_cast<uint32_t*>(symbol_address(g_debug_addr, HIP_SYMBOL(debug_word)));
}

// enqueue the index checks of a call; false if they could not be launched
bool check_bounds(pa::BoundsArgs a, hipStream_t stream) {
    a.word = debug_word_address();
    return a.word && pa::launch_bounds_check(a, stream) == hipSuccess;
}

pa::BoundsArgs bounds_args(int32_t kind, int64_t count, int64_t limit) {
    pa::BoundsArgs a{};
    a.kind = kind;
    a.count = count;
    a.limit = limit;
    return a;
}
#endif

// the index checks of a decode call (debug builds; true elsewhere)
bool check_decode_bounds(const pa::DecodeArgs& d, hipStream_t stream) {
#ifdef PA_DEBUG_BOUNDS
    pa::BoundsArgs ba = bounds_args(pa::kBoundsDecode, d.num_seqs, d.num_blocks);
    ba.block_tables = d.block_tables;
    ba.seq_lens = d.seq_lens;
    ba.table_stride = d.table_stride;
    ba.block_shift = d.block_shift;
    ba.max_blocks16 = d.max_blocks_per_seq;
    return check_bounds(ba, stream);
#else
    (void)d;
    (void)stream;
    return true;
#endif
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr uint32_t kDecodeFlags = PA_DECODE_STREAM_KV | PA_DECODE_SHARED_PREFIX;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool supported_dtype(pa_dtype d) { return d == PA_F16 || d == PA_BF16; }

// log2(block_size / 16) for the block sizes the 16-bit calls take (16, 32), or
// -1.  The kernels walk every cache in 16-token blocks; a 32-token block is two
// of them (sub_block in common.h).  The FP8 calls take 16 only: their scales
// are laid out per 16-token block.
int32_t block_shift(int32_t block_size) {
    return block_size == 16 ? 0 : block_size == 32 ? 1 : -1;
}

int32_t ceil_div(int64_t a, int64_t b) { return (int32_t)((a + b - 1) / b); }

// heads one decode wave carries: the smallest of 1, 2, 4, 8 covering the group
int32_t heads_per_wave(int32_t group) {
    if (group <= 1) return 1;
    if (group <= 2) return 2;
    if (group <= 4) return 4;
    return 8;
}

// most q heads per kv head: decode splits them into chunks of 8 or 16 heads
// per wave, prefill's workgroups hold at least one position of all of them
constexpr int32_t kMaxGroup = 128;

// decode runs on matrix cores when 3+ q heads share a kv head at head_dim 128
bool uses_gqa_kernel(int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim) {
    return head_dim == 128 && num_kv_heads > 0 && num_q_heads / num_kv_heads >= 3;
}

// max_blocks16: 16-token blocks per sequence
int32_t default_partition(int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t max_blocks16) {
    // About eight partitions for the longest sequence the tables allow, within
    // [256, cap] tokens.  Measured on MI355X: the vector-ALU kernel (group <= 2)
    // is fastest at 512-token partitions (more items even out the length mix),
    // the matrix-core kernel at 1024-2048 (it keeps fewer waves resident, so
    // longer items hide its start-up latency better).
    const int32_t cap = uses_gqa_kernel(num_q_heads, num_kv_heads, head_dim) ? 2048 : 512;
    const int64_t want = (int64_t)max_blocks16 * 16 / 8;
    int32_t p = 256;
    while (p < cap && p < want) p <<= 1;
    return p;
}

// Balanced split of single-query decode (see balanced_walk in common.h): the
// waves launched, one round of the 16-bit decode kernels at 3 resident waves
// per SIMD (160 and 131 VGPRs) on 256 CUs x 4 SIMDs, so every wave has the same
// share of the work and no second round runs behind a few long sequences.
constexpr int32_t kBalancedWaves = 3072;
constexpr int32_t kBalancedWavesMfma = 3072;
// each wave scans seq_lens, 64 sequences per pass: at most 8 passes
constexpr int32_t kBalancedMaxSeqs = 512;

struct DecodeShape {
    bool valid;          // false: partition_tokens asks for a split this call cannot make
    int32_t part_tokens;
    int32_t num_parts;
    bool balanced;
    int32_t num_items;   // balanced: waves launched
    size_t ws_bytes;
};

// q heads one wave of the decode kernels carries, for `cols` columns
// (query, q head pairs) per kv head.  The balanced split numbers its units by
// head chunks, and its merge runs after the 16-bit and the FP8 kernels alike,
// so it takes chunks both carry: 16 on matrix cores, else at most 4.
int32_t decode_wave_heads(int32_t cols, int32_t head_dim, bool balanced) {
    if (head_dim == 128 && cols >= 3) return 16;
    return balanced ? std::min(heads_per_wave(cols), 4) : heads_per_wave(cols);
}

// max_blocks16: 16-token blocks per sequence.  may_balance: a single-query
// call (multi-query calls take multi_balanced_shape instead).
//   partition_tokens > 0: fixed partitions of that length.
//   partition_tokens == 0: the balanced split when fixed partitions of the
//     default length would need more items than one round of resident waves
//     (kBalancedWaves) -- then a few long sequences would run alone in the last
//     round -- otherwise the default partitions, already a single round.
//   PA_PARTITION_BALANCED: the balanced split (not valid for multi-query calls
//     or more than kBalancedMaxSeqs sequences).
DecodeShape decode_shape(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t max_blocks16, int32_t partition_tokens,
                         bool may_balance) {
    DecodeShape s;
    s.valid = true;
    s.part_tokens = 0;
    s.num_parts = 0;
    s.balanced = false;
    s.num_items = 0;
    s.ws_bytes = 0;
    const int32_t group = num_q_heads / num_kv_heads;
    if (partition_tokens >= 0) {
        s.part_tokens = partition_tokens > 0
                            ? partition_tokens
                            : default_partition(num_q_heads, num_kv_heads, head_dim, max_blocks16);
        const int32_t part_blocks = s.part_tokens / 16;
        s.num_parts = max_blocks16 <= part_blocks ? 1 : ceil_div(max_blocks16, part_blocks);
        if (s.num_parts <= 1) {
            s.ws_bytes = 0;
        } else {
            const size_t states = (size_t)num_seqs * num_q_heads * s.num_parts;
            s.ws_bytes = states * ((size_t)head_dim * sizeof(float) + 2 * sizeof(float));
        }
        if (partition_tokens > 0) return s;
    }
    const int64_t part_items = partition_tokens == 0
        ? (int64_t)num_seqs * num_kv_heads * ceil_div(group, decode_wave_heads(group, head_dim, false)) * s.num_parts
        : 0;
    const bool want = partition_tokens == PA_PARTITION_BALANCED || part_items > kBalancedWaves;
    const int32_t hpw = decode_wave_heads(group, head_dim, true);
    const int64_t upb = (int64_t)num_kv_heads * ceil_div(group, hpw);   // waves per stretch
    const int64_t stretches = (hpw == 16 ? kBalancedWavesMfma : kBalancedWaves) / upb;
    const bool can = may_balance && num_seqs <= kBalancedMaxSeqs && stretches >= 1 &&
                     (int64_t)num_seqs * max_blocks16 <= INT32_MAX;
    if (want && can) {
        s.balanced = true;
        s.num_items = (int32_t)(stretches * upb);
        s.part_tokens = 0;
        s.num_parts = 0;
        const size_t states = (size_t)(num_seqs + stretches) * upb * std::min(hpw, group);
        s.ws_bytes = states * ((size_t)head_dim * sizeof(float) + 2 * sizeof(float));
    } else if (partition_tokens == PA_PARTITION_BALANCED) {
        s.valid = false;
    }
    return s;
}

// The balanced split of a multi-query decode (q_per_seq > 1): the stream runs
// over the sequences' blocks and each unit (kv head, chunk of 16 of its
// q_per_seq * group (query, head) columns) reads a block once for every query
// of its sequence; matrix-core path only (head_dim 128, 3+ columns per kv head).
// valid = false where it does not apply.
DecodeShape multi_balanced_shape(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t max_blocks16, int32_t q_per_seq) {
    DecodeShape s{};
    const int32_t cols = q_per_seq * (num_q_heads / num_kv_heads);
    if (head_dim != 128 || cols < 3 || num_seqs > kBalancedMaxSeqs || (int64_t)num_seqs * max_blocks16 > INT32_MAX)
        return s;
    const int64_t upb = (int64_t)num_kv_heads * ceil_div(cols, 16);
    const int64_t stretches = kBalancedWavesMfma / upb;
    if (stretches < 1) return s;
    s.valid = true;
    s.balanced = true;
    s.num_items = (int32_t)(stretches * upb);
    const size_t states = (size_t)(num_seqs + stretches) * upb * std::min(cols, 16);
    s.ws_bytes = states * ((size_t)head_dim * sizeof(float) + 2 * sizeof(float));
    return s;
}

pa_status check_decode(const void* out, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                       int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                       float scale, pa_dtype dtype, int32_t partition_tokens) {
    const int32_t sh = block_shift(block_size);
    if (!supported_dtype(dtype) || sh < 0 || (head_dim != 64 && head_dim != 128))
        return PA_ERR_UNSUPPORTED;
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0 ||
        num_blocks <= 0 || num_q_heads % num_kv_heads != 0 || num_q_heads / num_kv_heads > kMaxGroup ||
        (partition_tokens != PA_PARTITION_BALANCED && (partition_tokens < 0 || partition_tokens % 16 != 0)) ||
        !(scale > 0.f) || !isfinite(scale) ||
        (int64_t)max_blocks_per_seq * block_size > INT32_MAX || num_blocks > (INT64_C(1) << (31 - sh)))
        return PA_ERR_SHAPE;
    if (num_seqs == 0) return PA_OK;
    if (!out || !q || !k_cache || !v_cache || !block_tables || !seq_lens) return PA_ERR_NULL_PTR;
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
        return PA_ERR_ALIGNMENT;
    return PA_OK;
}

pa::DecodeArgs decode_args(void* out, const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                           int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                           float scale, pa_dtype dtype, const DecodeShape& shape, void* workspace,
                           uint32_t flags, int32_t q_per_seq = 1, int32_t seqs_per_wave = 1) {
    const int32_t sh = block_shift(block_size);
    pa::DecodeArgs a;
    a.out = out;
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.seq_lens = seq_lens;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.group = num_q_heads / num_kv_heads;
    a.q_per_seq = q_per_seq;
    a.cols = q_per_seq * a.group;   // (query, q head) columns per kv head
    // 3 or more columns per kv head make QK^T and PV real contractions: matrix cores
    a.gqa_mfma = head_dim == 128 && a.cols >= 3;
    a.heads_per_wave = decode_wave_heads(a.cols, head_dim, shape.balanced);
    a.k_scales = nullptr;
    a.v_scales = nullptr;
    a.head_chunks = ceil_div(a.cols, a.heads_per_wave);
    a.head_dim = head_dim;
    a.max_blocks_per_seq = max_blocks_per_seq << sh;
    a.num_blocks = num_blocks << sh;
    a.table_stride = max_blocks_per_seq;
    a.block_shift = sh;
    a.part_blocks = shape.part_tokens / 16;
    a.num_parts = shape.num_parts;
    a.scale_log2 = scale * kLog2e;
    a.dtype = dtype == PA_F16 ? pa::kF16 : pa::kBF16;
    a.stream_kv = (flags & PA_DECODE_STREAM_KV) != 0;
    a.balanced = shape.balanced;
    a.num_items = shape.num_items;
    a.state_heads = std::min(a.heads_per_wave, a.cols);
    float* ws = static_cast<float*>(workspace);
    const size_t upb = (size_t)num_kv_heads * a.head_chunks;
    size_t states = shape.balanced ? ((size_t)num_seqs + shape.num_items / upb) * upb * a.state_heads
                                   : (size_t)num_seqs * q_per_seq * num_q_heads * shape.num_parts;
    a.new_k = nullptr;
    a.new_v = nullptr;
    a.seqs_per_wave = seqs_per_wave;
    a.shared_base = (int64_t)states;
    size_t owners = 0;
    if (seqs_per_wave > 1) {   // the shared runs' states, 16 columns per (group + stretch, kv head)
        const size_t groups = ceil_div(num_seqs, seqs_per_wave);
        states += (groups + shape.num_items / upb) * num_kv_heads * 16;
        owners = groups * (seqs_per_wave + 1);
    }
    a.ws_acc = shape.ws_bytes ? ws : nullptr;
    a.ws_ml = shape.ws_bytes ? reinterpret_cast<float2*>(ws + states * head_dim) : nullptr;
    a.owner_blocks = shape.ws_bytes && owners ? reinterpret_cast<int32_t*>(a.ws_ml + states) : nullptr;
    return a;
}

// Sequence groups (PA_DECODE_SHARED_PREFIX on pa_decode): where the
// matrix-core kernel's 16 columns hold two or more sequences' heads (3 to 8 q
// heads per kv head) and the balanced split fits, one wave carries 16 / group
// consecutive sequences through the leading blocks they share and the balanced
// split runs over those shared runs and the members' own blocks.  Returns the
// sequences per wave, 1 where the groups do not apply.
int32_t group_seqs(uint32_t flags, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                   int32_t partition_tokens) {
    if (!(flags & PA_DECODE_SHARED_PREFIX) || (partition_tokens != 0 && partition_tokens != PA_PARTITION_BALANCED) ||
        !uses_gqa_kernel(num_q_heads, num_kv_heads, head_dim))
        return 1;
    const int32_t group = num_q_heads / num_kv_heads;
    return group <= 8 ? 16 / group : 1;
}

// The balanced shape with the groups' workspace: after the one-sequence
// states, (groups + stretches) * num_kv_heads * 16 states of the shared runs,
// then groups * (S + 1) int32 owner counts.  valid = false where the balanced
// split does not fit the call.
DecodeShape grouped_shape(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t max_blocks16, int32_t seqs_per_wave) {
    DecodeShape s = decode_shape(num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks16,
                                 PA_PARTITION_BALANCED, true);
    if (s.valid) {
        const size_t groups = ceil_div(num_seqs, seqs_per_wave);
        const size_t stretches = (size_t)s.num_items / num_kv_heads;
        s.ws_bytes += (groups + stretches) * num_kv_heads * 16 * ((size_t)head_dim * sizeof(float) + 2 * sizeof(float)) +
                      groups * (seqs_per_wave + 1) * sizeof(int32_t);
    }
    return s;
}

// Both decode phases launch one 4-wave workgroup per 4 items; their grids are
// checked here, before either is enqueued, so that a call that fails its
// checks has launched nothing.
bool decode_grids_fit(const pa::DecodeArgs& a) {
    const int64_t items = a.balanced ? a.num_items
                                     : (int64_t)a.num_seqs * a.num_kv_heads * a.head_chunks * a.num_parts;
    const int64_t rows = (int64_t)a.num_seqs * a.q_per_seq * a.num_q_heads;
    return (items + 3) / 4 <= INT32_MAX && (rows + 3) / 4 <= INT32_MAX;
}

pa_status check_workspace(const DecodeShape& shape, const void* workspace, size_t workspace_bytes) {
    if (shape.ws_bytes == 0) return PA_OK;
    if (!workspace || workspace_bytes < shape.ws_bytes) return PA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return PA_ERR_ALIGNMENT;
    return PA_OK;
}

// The first decode phase; with new_k / new_v also the step's cache write of each
// sequence's newest token, done by the decode kernels themselves.
pa_status decode_partitions(void* out, const void* q, const void* new_k, const void* new_v, const void* k_cache,
                            const void* v_cache, const int32_t* block_tables, const int32_t* seq_lens,
                            int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks, float scale,
                            pa_dtype dtype, int32_t partition_tokens, uint32_t flags, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
    if (flags & ~kDecodeFlags) return PA_ERR_UNSUPPORTED;
    pa_status st = check_decode(out, q, k_cache, v_cache, block_tables, seq_lens, num_seqs,
                                num_q_heads, num_kv_heads, head_dim, block_size,
                                max_blocks_per_seq, num_blocks, scale, dtype, partition_tokens);
    if (st != PA_OK || num_seqs == 0) return st;
    if (new_k && (!aligned16(new_k) || !aligned16(new_v))) return PA_ERR_ALIGNMENT;
    const DecodeShape shape = decode_shape(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                           max_blocks_per_seq << block_shift(block_size),
                                           partition_tokens, true);
    if (!shape.valid) return PA_ERR_SHAPE;
    st = check_workspace(shape, workspace, workspace_bytes);
    if (st != PA_OK) return st;
    pa::DecodeArgs a = decode_args(out, q, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_q_heads,
                                   num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, scale,
                                   dtype, shape, workspace, flags);
    a.new_k = new_k;
    a.new_v = new_v;
    if (!decode_grids_fit(a)) return PA_ERR_SHAPE;
    if (!check_decode_bounds(a, stream)) return PA_ERR_HIP;
    return pa::launch_decode_partitions(a, stream) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

// pa_decode / pa_decode_fp8 with PA_DECODE_SHARED_PREFIX: the sequence groups'
// plan, grouped split and merge, or kNotGrouped where the call does not take
// them (the caller then decodes without them).  fp8: k_scales / v_scales given.
constexpr pa_status kNotGrouped = static_cast<pa_status>(1);

pa_status decode_grouped(void* out, const void* q, const void* k_cache, const void* v_cache,
                         const float* k_scales, const float* v_scales, const int32_t* block_tables,
                         const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                         float scale, pa_dtype dtype, int32_t partition_tokens, uint32_t flags, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
    const bool fp8 = k_scales || v_scales;
    pa_status st = check_decode(out, q, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_q_heads,
                                num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, scale, dtype,
                                partition_tokens);
    if (st != PA_OK || num_seqs == 0) return st;
    if (fp8 && block_size != PA_BLOCK_SIZE) return kNotGrouped;   // the FP8 call refuses it itself
    const int32_t spw = group_seqs(flags, num_q_heads, num_kv_heads, head_dim, partition_tokens);
    if (spw <= 1) return kNotGrouped;
    const DecodeShape shape = grouped_shape(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                            max_blocks_per_seq << block_shift(block_size), spw);
    if (!shape.valid) return kNotGrouped;
    if (fp8) {
        if (!k_scales || !v_scales) return PA_ERR_NULL_PTR;
        if (!aligned16(k_scales) || !aligned16(v_scales)) return PA_ERR_ALIGNMENT;
    }
    st = check_workspace(shape, workspace, workspace_bytes);
    if (st != PA_OK) return st;
    pa::DecodeArgs a = decode_args(out, q, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_q_heads,
                                   num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, scale,
                                   dtype, shape, workspace, flags, 1, spw);
    a.k_scales = k_scales;
    a.v_scales = v_scales;
    if (!decode_grids_fit(a)) return PA_ERR_SHAPE;
    if (!check_decode_bounds(a, stream)) return PA_ERR_HIP;
    if ((fp8 ? pa::launch_decode_grouped_fp8(a, stream) : pa::launch_decode_grouped(a, stream)) != hipSuccess)
        return PA_ERR_HIP;
    return pa::launch_decode_merge(a, stream) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace

extern "C" {

uint64_t pa_kv_bytes_per_token(int32_t layers, int32_t kv_heads, int32_t head_dim,
                               int32_t dtype_bytes) {
    if (layers <= 0 || kv_heads <= 0 || head_dim <= 0 || dtype_bytes <= 0) return 0;
    return 2ull * (uint64_t)layers * (uint64_t)kv_heads * (uint64_t)head_dim * (uint64_t)dtype_bytes;
}

const char* pa_status_string(pa_status status) {
    switch (status) {
        case PA_OK: return "ok";
        case PA_ERR_NULL_PTR: return "a required pointer is NULL";
        case PA_ERR_UNSUPPORTED: return "unsupported head_dim, block_size or dtype";
        case PA_ERR_SHAPE: return "inconsistent or out-of-range sizes";
        case PA_ERR_WORKSPACE: return "decode workspace missing or too small";
        case PA_ERR_HIP: return "the HIP runtime refused a kernel launch";
        case PA_ERR_ALIGNMENT: return "a tensor or the workspace is not 16-byte aligned";
        case PA_ERR_SCRATCH:
            return "split-KV partial results exceed the static scratch of pa_decode_noalloc "
                   "(PA_NOALLOC_SCRATCH_BYTES); use pa_decode with a caller workspace";
        default: return "unknown status";
    }
}

pa_status pa_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                               const int64_t* slot_mapping, int64_t num_tokens,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int64_t num_blocks, pa_dtype dtype, hipStream_t stream) {
    if (!supported_dtype(dtype) || block_shift(block_size) < 0 || (head_dim != 64 && head_dim != 128))
        return PA_ERR_UNSUPPORTED;
    if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0 || num_blocks > INT64_MAX / block_size)
        return PA_ERR_SHAPE;
    if (num_tokens == 0) return PA_OK;
    if (!key || !value || !k_cache || !v_cache || !slot_mapping) return PA_ERR_NULL_PTR;
    if (!aligned16(key) || !aligned16(value) || !aligned16(k_cache) || !aligned16(v_cache))
        return PA_ERR_ALIGNMENT;
    pa::ReshapeArgs a;
    a.key = key;
    a.value = value;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.slot_mapping = slot_mapping;
    a.num_tokens = num_tokens;
    a.num_slots = num_blocks * block_size;   // a slot's row sits at the same place for any block_size
    a.row_vecs = num_kv_heads * head_dim / 8;
    a.block_tables = nullptr;
    a.seq_lens = nullptr;
    a.table_stride = 0;
    a.block_size = block_size;
#ifdef PA_DEBUG_BOUNDS
    pa::BoundsArgs ba = bounds_args(pa::kBoundsSlots, num_tokens, a.num_slots);
    ba.indices = slot_mapping;
    if (!check_bounds(ba, stream)) return PA_ERR_HIP;
#endif
    return pa::launch_reshape_and_cache(a, stream) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_pairs, int64_t num_pairs,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         int64_t num_blocks, pa_dtype dtype, hipStream_t stream) {
    if (!supported_dtype(dtype) || block_shift(block_size) < 0 || (head_dim != 64 && head_dim != 128))
        return PA_ERR_UNSUPPORTED;
    if (num_pairs < 0 || num_kv_heads <= 0 || num_blocks <= 0) return PA_ERR_SHAPE;
    if (num_pairs == 0) return PA_OK;
    if (!k_cache || !v_cache || !block_pairs) return PA_ERR_NULL_PTR;
    if (!aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_ALIGNMENT;
    pa::CopyBlocksArgs a;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_pairs = block_pairs;
    a.num_pairs = num_pairs;
    a.num_blocks = num_blocks;
    a.block_vecs = (int64_t)block_size * num_kv_heads * head_dim / 8;
    a.wgs_per_pair = (a.block_vecs + 1023) / 1024;
#ifdef PA_DEBUG_BOUNDS
    pa::BoundsArgs ba = bounds_args(pa::kBoundsPairs, num_pairs, num_blocks);
    ba.indices = block_pairs;
    if (!check_bounds(ba, stream)) return PA_ERR_HIP;
#endif
    return pa::launch_copy_blocks(a, stream) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_reshape_and_cache_fp8(const void* key, const void* value, void* k_cache,
                                   void* v_cache, float* k_scales, float* v_scales,
                                   const int64_t* slot_mapping, int64_t num_tokens,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                   int64_t num_blocks, pa_dtype dtype, hipStream_t stream) {
    if (!supported_dtype(dtype) || block_size != PA_BLOCK_SIZE || (head_dim != 64 && head_dim != 128))
        return PA_ERR_UNSUPPORTED;
    if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0 ||
        num_tokens > INT32_MAX / num_kv_heads)   // (token, head) pairs are counted in 32 bits
        return PA_ERR_SHAPE;
    if (num_tokens == 0) return PA_OK;
    if (!key || !value || !k_cache || !v_cache || !k_scales || !v_scales || !slot_mapping)
        return PA_ERR_NULL_PTR;
    if (!aligned16(key) || !aligned16(value) || !aligned16(k_cache) || !aligned16(v_cache) ||
        !aligned16(k_scales) || !aligned16(v_scales))
        return PA_ERR_ALIGNMENT;
    pa::ReshapeFp8Args a;
    a.key = key;
    a.value = value;
    a.k_cache = static_cast<uint8_t*>(k_cache);
    a.v_cache = static_cast<uint8_t*>(v_cache);
    a.k_scales = k_scales;
    a.v_scales = v_scales;
    a.slot_mapping = slot_mapping;
    a.num_tokens = num_tokens;
    a.num_slots = num_blocks * PA_BLOCK_SIZE;
    a.num_kv_heads = num_kv_heads;
    a.head_dim = head_dim;
    a.dtype = dtype == PA_F16 ? pa::kF16 : pa::kBF16;
#ifdef PA_DEBUG_BOUNDS
    pa::BoundsArgs ba = bounds_args(pa::kBoundsSlots, num_tokens, a.num_slots);
    ba.indices = slot_mapping;
    if (!check_bounds(ba, stream)) return PA_ERR_HIP;
#endif
    return pa::launch_reshape_and_cache_fp8(a, stream) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_copy_blocks_fp8(void* k_cache, void* v_cache, float* k_scales, float* v_scales,
                             const int64_t* block_pairs, int64_t num_pairs, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size, int64_t num_blocks,
                             hipStream_t stream) {
    if (block_size != PA_BLOCK_SIZE || (head_dim != 64 && head_dim != 128)) return PA_ERR_UNSUPPORTED;
    if (num_pairs < 0 || num_kv_heads <= 0 || num_blocks <= 0) return PA_ERR_SHAPE;
    if (num_pairs == 0) return PA_OK;
    if (!k_cache || !v_cache || !k_scales || !v_scales || !block_pairs) return PA_ERR_NULL_PTR;
    if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_scales) || !aligned16(v_scales))
        return PA_ERR_ALIGNMENT;
    // the copy kernel moves 16-byte vectors: a code block is 16 * Hkv * D bytes,
    // a scale block 16 * Hkv floats
    pa::CopyBlocksArgs a;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_pairs = block_pairs;
    a.num_pairs = num_pairs;
    a.num_blocks = num_blocks;
    a.block_vecs = (int64_t)num_kv_heads * head_dim;
    a.wgs_per_pair = (a.block_vecs + 1023) / 1024;
    if (num_pairs > INT32_MAX / a.wgs_per_pair) return PA_ERR_SHAPE;   // checked before either launch
#ifdef PA_DEBUG_BOUNDS
    pa::BoundsArgs ba = bounds_args(pa::kBoundsPairs, num_pairs, num_blocks);
    ba.indices = block_pairs;
    if (!check_bounds(ba, stream)) return PA_ERR_HIP;
#endif
    if (pa::launch_copy_blocks(a, stream) != hipSuccess) return PA_ERR_HIP;
    a.k_cache = k_scales;
    a.v_cache = v_scales;
    a.block_vecs = (int64_t)num_kv_heads * 4;
    a.wgs_per_pair = (a.block_vecs + 1023) / 1024;
    return pa::launch_copy_blocks(a, stream) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int32_t pa_decode_default_partition(int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t block_size, int32_t max_blocks_per_seq) {
    const int32_t sh = block_shift(block_size);
    if (num_q_heads <= 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0 || sh < 0 ||
        max_blocks_per_seq > (INT32_MAX >> sh))
        return 256;
    return default_partition(num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq << sh);
}

int32_t pa_decode_split(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                        int32_t block_size, int32_t max_blocks_per_seq, int32_t partition_tokens) {
    const int32_t sh = block_shift(block_size);
    if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 ||
        (head_dim != 64 && head_dim != 128) || sh < 0 || max_blocks_per_seq <= 0 ||
        max_blocks_per_seq > (INT32_MAX >> sh) ||
        (partition_tokens != PA_PARTITION_BALANCED && (partition_tokens < 0 || partition_tokens % 16)))
        return 0;
    const DecodeShape shape = decode_shape(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                           max_blocks_per_seq << sh, partition_tokens, true);
    if (!shape.valid) return 0;
    return shape.balanced ? PA_PARTITION_BALANCED : shape.part_tokens;
}

size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                                int32_t partition_tokens) {
    const int32_t sh = block_shift(block_size);
    if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || sh < 0 ||
        max_blocks_per_seq <= 0 || max_blocks_per_seq > (INT32_MAX >> sh) ||
        (partition_tokens != PA_PARTITION_BALANCED && (partition_tokens < 0 || partition_tokens % 16)))
        return 0;
    // enough for either split of this shape, and for sequence groups where they apply
    const int32_t mb16 = max_blocks_per_seq << sh;
    size_t need = std::max(decode_shape(num_seqs, num_q_heads, num_kv_heads, head_dim, mb16, partition_tokens,
                                        true).ws_bytes,
                           decode_shape(num_seqs, num_q_heads, num_kv_heads, head_dim, mb16, partition_tokens,
                                        false).ws_bytes);
    if (num_q_heads % num_kv_heads == 0 &&
        group_seqs(PA_DECODE_SHARED_PREFIX, num_q_heads, num_kv_heads, head_dim, partition_tokens) > 1) {
        const DecodeShape g = grouped_shape(num_seqs, num_q_heads, num_kv_heads, head_dim, mb16,
                                            group_seqs(PA_DECODE_SHARED_PREFIX, num_q_heads, num_kv_heads,
                                                       head_dim, partition_tokens));
        if (g.valid) need = std::max(need, g.ws_bytes);
    }
    return need;
}

pa_status pa_decode_partitions(void* out, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, const int32_t* seq_lens,
                               int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                               int64_t num_blocks, float scale, pa_dtype dtype,
                               int32_t partition_tokens, uint32_t flags, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
    return decode_partitions(out, q, nullptr, nullptr, k_cache, v_cache, block_tables, seq_lens, num_seqs,
                             num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                             scale, dtype, partition_tokens, flags, workspace, workspace_bytes, stream);
}

pa_status pa_decode_partitions_step(void* out, const void* q, const void* key, const void* value,
                                    void* k_cache, void* v_cache, const int32_t* block_tables,
                                    const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                    int32_t max_blocks_per_seq, int64_t num_blocks, float scale,
                                    pa_dtype dtype, int32_t partition_tokens, uint32_t flags,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (num_seqs > 0 && (!key || !value)) return PA_ERR_NULL_PTR;
    return decode_partitions(out, q, key, value, k_cache, v_cache, block_tables, seq_lens, num_seqs,
                             num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                             scale, dtype, partition_tokens, flags, workspace, workspace_bytes, stream);
}

pa_status pa_decode_merge(void* out, const int32_t* seq_lens, int32_t num_seqs,
                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, int32_t max_blocks_per_seq, pa_dtype dtype,
                          int32_t partition_tokens, const void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
    const int32_t sh = block_shift(block_size);
    if (!supported_dtype(dtype) || sh < 0 || (head_dim != 64 && head_dim != 128))
        return PA_ERR_UNSUPPORTED;
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0 ||
        num_q_heads % num_kv_heads != 0 || num_q_heads / num_kv_heads > kMaxGroup ||
        (partition_tokens != PA_PARTITION_BALANCED && (partition_tokens < 0 || partition_tokens % 16 != 0)) ||
        (int64_t)max_blocks_per_seq * block_size > INT32_MAX)
        return PA_ERR_SHAPE;
    if (num_seqs == 0) return PA_OK;
    if (!out || !seq_lens) return PA_ERR_NULL_PTR;
    if (!aligned16(out)) return PA_ERR_ALIGNMENT;
    const DecodeShape shape = decode_shape(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                           max_blocks_per_seq << sh, partition_tokens, true);
    if (!shape.valid) return PA_ERR_SHAPE;
    const pa_status st = check_workspace(shape, workspace, workspace_bytes);
    if (st != PA_OK) return st;
    if (!shape.balanced && shape.num_parts <= 1) return PA_OK;
    const pa::DecodeArgs a = decode_args(out, nullptr, nullptr, nullptr, nullptr, seq_lens,
                                         num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                         max_blocks_per_seq, 1, 1.f, dtype, shape,
                                         const_cast<void*>(workspace), 0u);
    return pa::launch_decode_merge(a, stream) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_decode_partitions_fp8(void* out, const void* q, const void* k_cache,
                                   const void* v_cache, const float* k_scales,
                                   const float* v_scales, const int32_t* block_tables,
                                   const int32_t* seq_lens, int32_t num_seqs,
                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, int32_t max_blocks_per_seq,
                                   int64_t num_blocks, float scale, pa_dtype dtype,
                                   int32_t partition_tokens, uint32_t flags, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
    if (flags & ~kDecodeFlags) return PA_ERR_UNSUPPORTED;
    if (block_size != PA_BLOCK_SIZE) return PA_ERR_UNSUPPORTED;   // scales are per 16-token block
    pa_status st = check_decode(out, q, k_cache, v_cache, block_tables, seq_lens, num_seqs,
                                num_q_heads, num_kv_heads, head_dim, block_size,
                                max_blocks_per_seq, num_blocks, scale, dtype, partition_tokens);
    if (st != PA_OK || num_seqs == 0) return st;
    if (!k_scales || !v_scales) return PA_ERR_NULL_PTR;
    if (!aligned16(k_scales) || !aligned16(v_scales)) return PA_ERR_ALIGNMENT;
    const DecodeShape shape = decode_shape(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                           max_blocks_per_seq, partition_tokens, true);
    if (!shape.valid) return PA_ERR_SHAPE;
    st = check_workspace(shape, workspace, workspace_bytes);
    if (st != PA_OK) return st;
    pa::DecodeArgs a = decode_args(out, q, k_cache, v_cache, block_tables, seq_lens, num_seqs,
                                   num_q_heads, num_kv_heads, head_dim, block_size,
                                   max_blocks_per_seq, num_blocks, scale, dtype, shape, workspace,
                                   flags);
    if (!a.gqa_mfma && a.heads_per_wave > 4) {   // the FP8 vector kernel carries up to 4 heads
        a.heads_per_wave = 4;
        a.head_chunks = ceil_div(a.group, 4);
    }
    a.k_scales = k_scales;
    a.v_scales = v_scales;
    if (!decode_grids_fit(a)) return PA_ERR_SHAPE;
    if (!check_decode_bounds(a, stream)) return PA_ERR_HIP;
    return pa::launch_decode_partitions_fp8(a, stream) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_decode_fp8(void* out, const void* q, const void* k_cache, const void* v_cache,
                        const float* k_scales, const float* v_scales, const int32_t* block_tables,
                        const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                        int32_t max_blocks_per_seq, int64_t num_blocks, float scale,
                        pa_dtype dtype, int32_t partition_tokens, uint32_t flags,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (flags & ~kDecodeFlags) return PA_ERR_UNSUPPORTED;
    if ((flags & PA_DECODE_SHARED_PREFIX) && block_size == PA_BLOCK_SIZE) {
        if (!k_scales || !v_scales) return PA_ERR_NULL_PTR;
        const pa_status gst = decode_grouped(out, q, k_cache, v_cache, k_scales, v_scales, block_tables,
                                             seq_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                             max_blocks_per_seq, num_blocks, scale, dtype, partition_tokens,
                                             flags, workspace, workspace_bytes, stream);
        if (gst != kNotGrouped) return gst;
    }
    pa_status st = pa_decode_partitions_fp8(out, q, k_cache, v_cache, k_scales, v_scales,
                                            block_tables, seq_lens, num_seqs, num_q_heads,
                                            num_kv_heads, head_dim, block_size,
                                            max_blocks_per_seq, num_blocks, scale, dtype,
                                            partition_tokens, flags, workspace, workspace_bytes,
                                            stream);
    if (st != PA_OK || num_seqs == 0) return st;
    return pa_decode_merge(out, seq_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                           block_size, max_blocks_per_seq, dtype, partition_tokens, workspace,
                           workspace_bytes, stream);
}

pa_status pa_decode_multi(void* out, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                          int32_t q_per_seq, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                          int64_t num_blocks, float scale, pa_dtype dtype, int32_t partition_tokens,
                          uint32_t flags, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
    if (flags & ~kDecodeFlags) return PA_ERR_UNSUPPORTED;
    if (q_per_seq < 1 || q_per_seq > PA_MAX_QUERIES_PER_SEQ) return PA_ERR_SHAPE;
    pa_status st = check_decode(out, q, k_cache, v_cache, block_tables, seq_lens, num_seqs,
                                num_q_heads, num_kv_heads, head_dim, block_size,
                                max_blocks_per_seq, num_blocks, scale, dtype, partition_tokens);
    if (st != PA_OK || num_seqs == 0) return st;
    if ((int64_t)num_seqs * q_per_seq > INT32_MAX) return PA_ERR_SHAPE;
    // Default partition: with several queries the work of a block grows while
    // its bytes do not, and the matrix-core kernel (used from 3 columns per kv
    // head at head_dim 128) is faster with longer partitions (measured on the
    // LLaMA-2-7B-shaped layer with 4 queries: 1024 tokens 68% of HBM peak, 512
    // tokens 65%).  Twice the single-query default, at most 2048 tokens (one
    // query keeps the single-query default, so it stays identical to pa_decode); never
    // more partitions than the single-query default, so the workspace size
    // documented for it always suffices.
    const int32_t mb16 = max_blocks_per_seq << block_shift(block_size);
    // Several queries on matrix cores: the balanced split (partition 0 or
    // PA_PARTITION_BALANCED) where its partial states fit the workspace that
    // pa_decode_workspace_size documents for this call (num_seqs * q_per_seq
    // single-query sequences, the same partition_tokens), so that no caller
    // needs more; PA_PARTITION_BALANCED is refused otherwise (below).
    DecodeShape shape{};
    if (q_per_seq > 1 && (partition_tokens == 0 || partition_tokens == PA_PARTITION_BALANCED)) {
        const DecodeShape mb = multi_balanced_shape(num_seqs, num_q_heads, num_kv_heads, head_dim, mb16, q_per_seq);
        const size_t documented =
            std::max(decode_shape(num_seqs * q_per_seq, num_q_heads, num_kv_heads, head_dim, mb16, partition_tokens,
                                  true).ws_bytes,
                     decode_shape(num_seqs * q_per_seq, num_q_heads, num_kv_heads, head_dim, mb16, partition_tokens,
                                  false).ws_bytes);
        if (mb.valid && mb.ws_bytes <= documented) shape = mb;
    }
    if (!shape.valid) {
        if (partition_tokens == 0 && q_per_seq > 1 && head_dim == 128 &&
            q_per_seq * (num_q_heads / num_kv_heads) >= 3)
            partition_tokens = std::min<int32_t>(
                2 * default_partition(num_q_heads, num_kv_heads, head_dim, mb16), 2048);
        // the partial states are per (sequence, query, q head): the workspace of
        // num_seqs * q_per_seq single-query sequences
        shape = decode_shape(num_seqs * q_per_seq, num_q_heads, num_kv_heads, head_dim, mb16, partition_tokens,
                             q_per_seq == 1);
    }
    if (!shape.valid) return PA_ERR_SHAPE;
    st = check_workspace(shape, workspace, workspace_bytes);
    if (st != PA_OK) return st;
    const pa::DecodeArgs a = decode_args(out, q, k_cache, v_cache, block_tables, seq_lens,
                                         num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                         max_blocks_per_seq, num_blocks, scale, dtype, shape,
                                         workspace, flags, q_per_seq);
    if (!decode_grids_fit(a)) return PA_ERR_SHAPE;
    if (!check_decode_bounds(a, stream)) return PA_ERR_HIP;
    if (pa::launch_decode_partitions(a, stream) != hipSuccess) return PA_ERR_HIP;
    if (!shape.balanced && shape.num_parts <= 1) return PA_OK;
    return pa::launch_decode_merge(a, stream) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                    float scale, pa_dtype dtype, int32_t partition_tokens, uint32_t flags,
                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (flags & ~kDecodeFlags) return PA_ERR_UNSUPPORTED;
    if (flags & PA_DECODE_SHARED_PREFIX) {
        const pa_status st = decode_grouped(out, q, k_cache, v_cache, nullptr, nullptr, block_tables, seq_lens,
                                            num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                            max_blocks_per_seq, num_blocks, scale, dtype, partition_tokens, flags,
                                            workspace, workspace_bytes, stream);
        if (st != kNotGrouped) return st;
    }
    pa_status st = pa_decode_partitions(out, q, k_cache, v_cache, block_tables, seq_lens,
                                        num_seqs, num_q_heads, num_kv_heads, head_dim,
                                        block_size, max_blocks_per_seq, num_blocks, scale, dtype,
                                        partition_tokens, flags, workspace, workspace_bytes,
                                        stream);
    if (st != PA_OK || num_seqs == 0) return st;
    return pa_decode_merge(out, seq_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                           block_size, max_blocks_per_seq, dtype, partition_tokens, workspace,
                           workspace_bytes, stream);
}

pa_status pa_decode_step(void* out, const void* q, const void* key, const void* value, void* k_cache,
                         void* v_cache, const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         int32_t max_blocks_per_seq, int64_t num_blocks, float scale, pa_dtype dtype,
                         int32_t partition_tokens, uint32_t flags, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
    if (flags & ~kDecodeFlags) return PA_ERR_UNSUPPORTED;
    pa_status st = check_decode(out, q, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_q_heads,
                                num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, scale, dtype,
                                partition_tokens);
    if (st != PA_OK || num_seqs == 0) return st;
    if (!key || !value) return PA_ERR_NULL_PTR;
    if (!aligned16(key) || !aligned16(value)) return PA_ERR_ALIGNMENT;
    const int32_t spw = group_seqs(flags, num_q_heads, num_kv_heads, head_dim, partition_tokens);
    if (spw > 1) {
        const DecodeShape g = grouped_shape(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                            max_blocks_per_seq << block_shift(block_size), spw);
        if (g.valid) {   // sequence groups read the newest tokens from the pool: the write goes first
            st = check_workspace(g, workspace, workspace_bytes);
            if (st != PA_OK) return st;
            pa::ReshapeArgs w;
            w.key = key;
            w.value = value;
            w.k_cache = k_cache;
            w.v_cache = v_cache;
            w.slot_mapping = nullptr;
            w.num_tokens = num_seqs;
            w.num_slots = num_blocks * block_size;
            w.row_vecs = num_kv_heads * head_dim / 8;
            w.block_tables = block_tables;
            w.seq_lens = seq_lens;
            w.table_stride = max_blocks_per_seq;
            w.block_size = block_size;
            if (pa::launch_reshape_and_cache(w, stream) != hipSuccess) return PA_ERR_HIP;
            st = decode_grouped(out, q, k_cache, v_cache, nullptr, nullptr, block_tables, seq_lens, num_seqs,
                                num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                                scale, dtype, partition_tokens, flags, workspace, workspace_bytes, stream);
            if (st != kNotGrouped) return st;
            // (not reached: the checks above are the groups' own) the rows are written: decode them
            return pa_decode(out, q, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_q_heads, num_kv_heads,
                             head_dim, block_size, max_blocks_per_seq, num_blocks, scale, dtype, partition_tokens,
                             flags & ~PA_DECODE_SHARED_PREFIX, workspace, workspace_bytes, stream);
        }
    }
    st = decode_partitions(out, q, key, value, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_q_heads,
                           num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, scale, dtype,
                           partition_tokens, flags, workspace, workspace_bytes, stream);
    if (st != PA_OK) return st;
    return pa_decode_merge(out, seq_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                           max_blocks_per_seq, dtype, partition_tokens, workspace, workspace_bytes, stream);
}

pa_status pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                            int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                            float scale, pa_dtype dtype, int32_t partition_tokens, uint32_t flags,
                            hipStream_t stream) {
    if (flags & ~kDecodeFlags) return PA_ERR_UNSUPPORTED;
    const pa_status st = check_decode(out, q, k_cache, v_cache, block_tables, seq_lens, num_seqs,
                                      num_q_heads, num_kv_heads, head_dim, block_size,
                                      max_blocks_per_seq, num_blocks, scale, dtype,
                                      partition_tokens);
    if (st != PA_OK || num_seqs == 0) return st;
    const DecodeShape shape = decode_shape(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                           max_blocks_per_seq << block_shift(block_size),
                                           partition_tokens, true);
    if (!shape.valid) return PA_ERR_SHAPE;
    size_t need = shape.ws_bytes;
    const int32_t spw = group_seqs(flags, num_q_heads, num_kv_heads, head_dim, partition_tokens);
    if (spw > 1) {
        const DecodeShape g = grouped_shape(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                            max_blocks_per_seq << block_shift(block_size), spw);
        if (g.valid && g.ws_bytes <= PA_NOALLOC_SCRATCH_BYTES) {
            need = g.ws_bytes;
        } else {
            flags &= ~PA_DECODE_SHARED_PREFIX;   // a hint: without room for the groups, decode without them
        }
    }
    if (need > PA_NOALLOC_SCRATCH_BYTES) return PA_ERR_SCRATCH;
    // The partition kernels write every partial state (and, with sequence
    // groups, every private block count) that the merge reads, so the scratch
    // needs no clearing between calls.
    void* ws = nullptr;
    if (need) {
        ws = scratch_address();
        if (!ws) return PA_ERR_HIP;
    }
    return pa_decode(out, q, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_q_heads,
                     num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, scale, dtype,
                     partition_tokens, flags, ws, ws ? PA_NOALLOC_SCRATCH_BYTES : 0, stream);
}

static pa_status prefill_common(void* out, const void* q, const void* k_cache, const void* v_cache,
                                const float* k_scales, const float* v_scales, bool fp8,
                                const int32_t* block_tables, const int32_t* ctx_lens,
                                const int32_t* query_start_loc, int32_t num_seqs, int64_t num_tokens,
                                int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                                int64_t num_blocks, float scale, pa_dtype dtype, hipStream_t stream) {
    const int32_t sh = block_shift(block_size);
    if (!supported_dtype(dtype) || sh < 0 || (fp8 && sh != 0) || (head_dim != 64 && head_dim != 128))
        return PA_ERR_UNSUPPORTED;
    if (num_seqs < 0 || num_tokens < 0 || max_q_len < 0 || num_q_heads <= 0 ||
        num_kv_heads <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0 ||
        num_q_heads % num_kv_heads != 0 || !(scale > 0.f) || !isfinite(scale) ||
        (int64_t)max_blocks_per_seq * block_size > INT32_MAX || num_blocks > (INT64_C(1) << (31 - sh)))
        return PA_ERR_SHAPE;
    const int32_t group = num_q_heads / num_kv_heads;
    if (group > kMaxGroup) return PA_ERR_UNSUPPORTED;   // more q heads per kv head than a workgroup's rows
    if (num_seqs == 0 || num_tokens == 0 || max_q_len == 0) return PA_OK;
    if (!out || !q || !k_cache || !v_cache || !block_tables || !ctx_lens || !query_start_loc)
        return PA_ERR_NULL_PTR;
    if (fp8 && (!k_scales || !v_scales)) return PA_ERR_NULL_PTR;
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
        return PA_ERR_ALIGNMENT;
    if (fp8 && (!aligned16(k_scales) || !aligned16(v_scales))) return PA_ERR_ALIGNMENT;
    pa::PrefillArgs a;
    a.out = out;
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.ctx_lens = ctx_lens;
    a.query_start_loc = query_start_loc;
    a.num_seqs = num_seqs;
    a.num_tokens = num_tokens;
    a.max_q_len = max_q_len;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.group = group;
    a.max_blocks_per_seq = max_blocks_per_seq << sh;
    a.num_blocks = num_blocks << sh;
    a.table_stride = max_blocks_per_seq;
    a.block_shift = sh;
    a.scale_log2 = scale * kLog2e;
    a.dtype = dtype == PA_F16 ? pa::kF16 : pa::kBF16;
    a.head_dim = head_dim;
    a.k_scales = k_scales;
    a.v_scales = v_scales;
#ifdef PA_DEBUG_BOUNDS
    pa::BoundsArgs ba = bounds_args(pa::kBoundsPrefill, num_seqs, a.num_blocks);
    ba.block_tables = block_tables;
    ba.ctx_lens = ctx_lens;
    ba.query_start_loc = query_start_loc;
    ba.num_tokens = num_tokens;
    ba.max_q_len = max_q_len;
    ba.table_stride = a.table_stride;
    ba.block_shift = sh;
    ba.max_blocks16 = a.max_blocks_per_seq;
    if (!check_bounds(ba, stream)) return PA_ERR_HIP;
#endif
    const hipError_t e = fp8 ? pa::launch_prefill_fp8(a, stream) : pa::launch_prefill(a, stream);
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_prefill_paged_fp8(void* out, const void* q, const void* k_cache, const void* v_cache,
                               const float* k_scales, const float* v_scales,
                               const int32_t* block_tables, const int32_t* ctx_lens,
                               const int32_t* query_start_loc, int32_t num_seqs, int64_t num_tokens,
                               int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                               int64_t num_blocks, float scale, pa_dtype dtype, hipStream_t stream) {
    return prefill_common(out, q, k_cache, v_cache, k_scales, v_scales, true, block_tables, ctx_lens,
                          query_start_loc, num_seqs, num_tokens, max_q_len, num_q_heads,
                          num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, scale,
                          dtype, stream);
}

pa_status pa_prefill_paged(void* out, const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, const int32_t* ctx_lens,
                           const int32_t* query_start_loc, int32_t num_seqs, int64_t num_tokens,
                           int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                           int64_t num_blocks, float scale, pa_dtype dtype, hipStream_t stream) {
    return prefill_common(out, q, k_cache, v_cache, nullptr, nullptr, false, block_tables, ctx_lens,
                          query_start_loc, num_seqs, num_tokens, max_q_len, num_q_heads,
                          num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, scale,
                          dtype, stream);
}

pa_status pa_debug_bounds(uint32_t* word, int32_t clear, hipStream_t stream) {
#ifdef PA_DEBUG_BOUNDS
    if (!word) return PA_ERR_NULL_PTR;
    uint32_t* dev = debug_word_address();
    if (!dev) return PA_ERR_HIP;
    if (hipMemcpyAsync(word, dev, sizeof(uint32_t), hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return PA_ERR_HIP;
    if (clear && (hipMemsetAsync(dev, 0, sizeof(uint32_t), stream) != hipSuccess ||
                  hipStreamSynchronize(stream) != hipSuccess))
        return PA_ERR_HIP;
    return PA_OK;
#else
    (void)word;
    (void)clear;
    (void)stream;
    return PA_ERR_UNSUPPORTED;
#endif
}

}  // extern "C"
