// Debug-build checks of device-resident indices.
//
// Device data cannot be validated on the host without a read-back, so the
// kernels skip what is out of range and leave the results involving it
// unspecified.  A library built with PA_DEBUG_BOUNDS runs this kernel before a
// call's own and records what it finds in a device word, read after a
// synchronisation ("Hardware abstraction and portability", §六: asynchronous
// errors surface at synchronisation points, and validation covers shapes and
// indices, not only host arguments).  The checks mirror what the kernels
// assume: the table entries of every block a sequence uses name a block of the
// pool, a sequence (or a context plus its chunk) fits its table row, packed
// query rows lie in order within the batch, and a slot or copy pair names the
// pool.  Only whole-pool ranges are checked; two tokens writing one slot is
// not detected.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace pa {

namespace {

__device__ __forceinline__ void flag(uint32_t* word, uint32_t bits) {
    if (bits) __hip_atomic_fetch_or(word, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// block j (16-token units) of a table row: the pool block it names, or -1
__device__ __forceinline__ int64_t table_block(const BoundsArgs& a, int64_t row, int j) {
    const int32_t entry = a.block_tables[row * a.table_stride + (j >> a.block_shift)];
    return sub_block(entry, j, a.block_shift);
}

}  // namespace

constexpr int kBoundsThreads = 256;

// one workgroup per sequence (decode, prefill) or a grid-stride loop (slots, pairs)
__global__ __launch_bounds__(kBoundsThreads) void bounds_check_kernel(BoundsArgs a) {
    uint32_t bits = 0;
    if (a.kind == kBoundsSlots || a.kind == kBoundsPairs) {
        const int64_t stride = (int64_t)gridDim.x * kBoundsThreads;
        const int64_t n = a.kind == kBoundsSlots ? a.count : 2 * a.count;
        for (int64_t i = (int64_t)blockIdx.x * kBoundsThreads + threadIdx.x; i < n; i += stride)
            if (a.indices[i] >= a.limit) bits |= a.kind == kBoundsSlots ? kBoundsSlot : kBoundsBlockId;
        flag(a.word, bits);
        return;
    }
    const int64_t b = blockIdx.x;
    if (b >= a.count) return;
    const int max_tokens = a.max_blocks16 * kBlockSize;
    int64_t n;   // tokens whose blocks the call reads
    if (a.kind == kBoundsDecode) {
        n = a.seq_lens[b];
        if (n < 0 || n > max_tokens) bits |= kBoundsSeqLen;
    } else {
        const int64_t r0 = a.query_start_loc[b];
        const int64_t r1 = a.query_start_loc[b + 1];
        if (r0 < 0 || r1 < r0 || r1 > a.num_tokens || r1 - r0 > a.max_q_len) bits |= kBoundsQueryRange;
        const int64_t len = r1 > r0 ? r1 - r0 : 0;
        const int64_t ctx = a.ctx_lens[b];
        if (ctx < 0 || ctx + len > max_tokens) bits |= kBoundsSeqLen;
        n = (ctx > 0 ? ctx : 0) + len;
    }
    n = n < 0 ? 0 : (n > max_tokens ? max_tokens : n);
    const int nblk = (int)((n + kBlockSize - 1) / kBlockSize);
    for (int j = threadIdx.x; j < nblk; j += kBoundsThreads) {
        const int64_t pb = table_block(a, b, j);
        if (pb < 0 || pb >= a.limit) bits |= kBoundsBlockId;
    }
    flag(a.word, bits);
}

hipError_t launch_bounds_check(const BoundsArgs& a, hipStream_t s) {
    if (a.count <= 0) return hipSuccess;
    unsigned grid;
    if (a.kind == kBoundsSlots || a.kind == kBoundsPairs) {
        const int64_t n = a.kind == kBoundsSlots ? a.count : 2 * a.count;
        grid = (unsigned)std::min<int64_t>((n + kBoundsThreads - 1) / kBoundsThreads, 1024);
    } else {
        if (a.count > 0x7fffffff) return hipErrorInvalidValue;
        grid = (unsigned)a.count;
    }
    return launch(bounds_check_kernel, dim3(grid), dim3(kBoundsThreads), s, a);
}

}  // namespace pa
