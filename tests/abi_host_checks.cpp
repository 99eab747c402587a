// Host-side checks of the C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer around the ABI layer (tests/test_abi_sanitized.py
// compiles and runs it; no GPU is needed).  Every call below is refused on the
// host before anything touches HIP, so the sanitizers see the whole of the
// validation code: argument checks, the size arithmetic of workspaces and
// grids, and the status strings, including extreme sizes near the int32 and
// int64 limits where an unchecked product would overflow.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "pa.h"

namespace {

int failures = 0;

void expect(const char* what, long long got, long long want) {
    if (got != want) {
        std::printf("FAIL %s: got %lld, want %lld\n", what, got, want);
        ++failures;
    }
}

// 16-byte aligned, never dereferenced: every call here fails validation first
void* const F = reinterpret_cast<void*>(0x10000);
const int32_t* const FI = static_cast<const int32_t*>(F);
const int64_t* const FL = static_cast<const int64_t*>(F);
const float* const FF = static_cast<const float*>(F);

}  // namespace

int main() {
    // status strings: every status, and an unknown one
    for (int s = -8; s <= 1; ++s)
        if (!pa_status_string(static_cast<pa_status>(s)) || !*pa_status_string(static_cast<pa_status>(s)))
            expect("status string", s, 1000);

    expect("kv bytes", (long long)pa_kv_bytes_per_token(32, 32, 128, 2), 524288);
    expect("kv bytes, negative", (long long)pa_kv_bytes_per_token(-1, 32, 128, 2), 0);
    pa_kv_bytes_per_token(INT32_MAX, INT32_MAX, INT32_MAX, INT32_MAX);

    // size queries at the edges
    pa_decode_workspace_size(INT32_MAX, 128, 1, 128, 16, INT32_MAX, 0);
    pa_decode_workspace_size(INT32_MAX, 128, 1, 128, 32, INT32_MAX, PA_PARTITION_BALANCED);
    pa_decode_workspace_size(1, INT32_MAX, 1, 128, 16, 1, 16);
    expect("workspace, negative", (long long)pa_decode_workspace_size(-1, 8, 2, 128, 16, 10, 0), 0);
    pa_decode_split(INT32_MAX, 128, 1, 128, 16, INT32_MAX, 0);
    pa_decode_split(1, INT32_MAX, 1, 64, 32, INT32_MAX >> 1, PA_PARTITION_BALANCED);
    expect("split, odd partition", pa_decode_split(4, 8, 2, 128, 16, 10, 17), 0);
    pa_decode_default_partition(INT32_MAX, 1, 128, 16, INT32_MAX);
    pa_decode_default_partition(8, 2, 128, 32, INT32_MAX);

    // cache writes and block copies
    expect("reshape null", pa_reshape_and_cache(nullptr, F, F, F, FL, 4, 2, 128, 16, 8, PA_BF16, nullptr),
           PA_ERR_NULL_PTR);
    expect("reshape shape", pa_reshape_and_cache(F, F, F, F, FL, 4, 2, 128, 16, 0, PA_BF16, nullptr),
           PA_ERR_SHAPE);
    expect("reshape huge pool", pa_reshape_and_cache(F, F, F, F, FL, 4, 2, 128, 32, INT64_MAX, PA_BF16, nullptr),
           PA_ERR_SHAPE);
    expect("reshape dtype", pa_reshape_and_cache(F, F, F, F, FL, 4, 2, 128, 16, 8, static_cast<pa_dtype>(9), nullptr),
           PA_ERR_UNSUPPORTED);
    expect("reshape fp8 tokens", pa_reshape_and_cache_fp8(F, F, F, F, static_cast<float*>(F), static_cast<float*>(F),
                                                         FL, INT64_MAX, 8, 128, 16, 8, PA_F16, nullptr),
           PA_ERR_SHAPE);
    expect("copy null", pa_copy_blocks(F, F, nullptr, 3, 2, 128, 16, 8, PA_F16, nullptr), PA_ERR_NULL_PTR);
    expect("copy fp8 pairs", pa_copy_blocks_fp8(F, F, static_cast<float*>(F), static_cast<float*>(F), FL,
                                                INT64_MAX, 64, 128, 16, 8, nullptr),
           PA_ERR_SHAPE);

    // decode, all entry points, at the limits of the size checks
    expect("decode group", pa_decode(F, F, F, F, FI, FI, 2, 258, 2, 128, 16, 64, 128, 0.1f, PA_BF16, 0, 0, F,
                                     1 << 20, nullptr),
           PA_ERR_SHAPE);
    expect("decode table width", pa_decode(F, F, F, F, FI, FI, 2, 8, 2, 128, 32, INT32_MAX, 128, 0.1f, PA_BF16, 0,
                                           0, F, 1 << 20, nullptr),
           PA_ERR_SHAPE);
    expect("decode pool", pa_decode(F, F, F, F, FI, FI, 2, 8, 2, 128, 16, 64, INT64_MAX, 0.1f, PA_BF16, 0, 0, F,
                                    1 << 20, nullptr),
           PA_ERR_SHAPE);
    expect("decode workspace", pa_decode(F, F, F, F, FI, FI, INT32_MAX, 8, 2, 128, 16, 64, 128, 0.1f, PA_BF16, 64,
                                         0, F, 16, nullptr),
           PA_ERR_WORKSPACE);
    expect("decode flags", pa_decode(F, F, F, F, FI, FI, 2, 8, 2, 128, 16, 64, 128, 0.1f, PA_BF16, 0, 4u, F,
                                     1 << 20, nullptr),
           PA_ERR_UNSUPPORTED);
    expect("decode noalloc scratch", pa_decode_noalloc(F, F, F, F, FI, FI, INT32_MAX, 128, 1, 128, 16, 4096, 1 << 20,
                                                       0.1f, PA_BF16, 16, 0, nullptr),
           PA_ERR_SCRATCH);
    expect("decode multi queries", pa_decode_multi(F, F, F, F, FI, FI, 2, PA_MAX_QUERIES_PER_SEQ + 1, 8, 2, 128,
                                                   16, 64, 128, 0.1f, PA_BF16, 0, 0, F, 1 << 20, nullptr),
           PA_ERR_SHAPE);
    expect("decode multi rows", pa_decode_multi(F, F, F, F, FI, FI, INT32_MAX, 16, 8, 2, 128, 16, 64, 128, 0.1f,
                                                PA_BF16, 0, 0, F, 1 << 20, nullptr),
           PA_ERR_SHAPE);
    expect("decode fp8 block size", pa_decode_fp8(F, F, F, F, FF, FF, FI, FI, 2, 8, 2, 128, 32, 64, 128, 0.1f,
                                                  PA_BF16, 0, 0, F, 1 << 20, nullptr),
           PA_ERR_UNSUPPORTED);
    expect("merge partition", pa_decode_merge(F, FI, 2, 8, 2, 128, 16, 64, PA_BF16, 24, F, 1 << 20, nullptr),
           PA_ERR_SHAPE);
    expect("partitions scale", pa_decode_partitions(F, F, F, F, FI, FI, 2, 8, 2, 128, 16, 64, 128, -1.f, PA_BF16,
                                                    0, 0, F, 1 << 20, nullptr),
           PA_ERR_SHAPE);

    // the decode step (cache write inside the decode)
    expect("step key", pa_decode_step(F, F, nullptr, F, F, F, FI, FI, 2, 8, 2, 128, 16, 64, 128, 0.1f, PA_BF16, 0,
                                      0, F, 1 << 20, nullptr),
           PA_ERR_NULL_PTR);
    expect("step table width", pa_decode_partitions_step(F, F, F, F, F, F, FI, FI, 2, 8, 2, 128, 32, INT32_MAX,
                                                         128, 0.1f, PA_BF16, 0, 0, F, 1 << 20, nullptr),
           PA_ERR_SHAPE);

    // prefill
    expect("prefill null", pa_prefill_paged(F, F, F, F, FI, FI, nullptr, 2, 64, 40, 32, 8, 128, 16, 16, 64, 0.1f,
                                            PA_BF16, nullptr),
           PA_ERR_NULL_PTR);
    expect("prefill table width", pa_prefill_paged(F, F, F, F, FI, FI, FI, 2, 64, 40, 32, 8, 128, 32, INT32_MAX, 64,
                                                   0.1f, PA_BF16, nullptr),
           PA_ERR_SHAPE);
    expect("prefill group", pa_prefill_paged(F, F, F, F, FI, FI, FI, 2, 64, 40, 258, 2, 128, 16, 16, 64, 0.1f,
                                             PA_BF16, nullptr),
           PA_ERR_UNSUPPORTED);
    expect("prefill fp8 scales", pa_prefill_paged_fp8(F, F, F, F, nullptr, FF, FI, FI, FI, 2, 64, 40, 32, 8, 128,
                                                      16, 16, 64, 0.1f, PA_BF16, nullptr),
           PA_ERR_NULL_PTR);

    // the debug bounds word: refused by the normal layer, wants a pointer in a debug one
    uint32_t word = 0;
    const pa_status dbg = pa_debug_bounds(&word, 1, nullptr);
    if (dbg != PA_ERR_UNSUPPORTED) expect("debug bounds", dbg, PA_ERR_UNSUPPORTED);

    if (failures) {
        std::printf("%d check(s) failed\n", failures);
        return 1;
    }
    std::printf("all host checks passed\n");
    return 0;
}
