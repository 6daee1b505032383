// Sanitizer driver for the C ABI's host-side argument checks (test
// infrastructure): every entry point is called with arguments the library
// must reject before anything is enqueued, plus the size queries, under an
// AddressSanitizer / UndefinedBehaviorSanitizer build of the library's host
// code.  No kernel is launched and no device is needed.  Exit status 0 when
// every call returned the expected status.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "spec_verify.h"

static int failures = 0;

static void expect(const char* what, int got, int want) {
    if (got != want) {
        std::printf("FAIL %s: status %d, want %d\n", what, got, want);
        ++failures;
    }
}

int main() {
    void* P = reinterpret_cast<void*>(uintptr_t(4096));
    void* W = reinterpret_cast<void*>(uintptr_t(1) << 20);
    auto* I = static_cast<int32_t*>(P);
    auto* F = static_cast<float*>(P);
    const size_t ws = spec_verify_workspace_bytes(2, 7, 1000);
    expect("workspace query", ws > 0, 1);
    expect("workspace query B=0", spec_verify_workspace_bytes(0, 7, 1000) == 0, 1);
    expect("workspace query huge V", spec_verify_workspace_bytes(2, 7, 1 << 30) == 0, 1);
    expect("sample query", spec_sample_workspace_bytes(10, 1000) > 0, 1);
    for (int s = -1; s < 7; ++s) expect("status string", spec_status_string(s) != nullptr, 1);

    // greedy
    expect("greedy dtype", spec_verify_greedy(P, (spec_dtype)7, I, 2, 3, 1000, I, I, nullptr, nullptr, I, W, ws, nullptr), SPEC_EDTYPE);
    expect("greedy B", spec_verify_greedy(P, SPEC_BF16, I, 0, 3, 1000, I, I, nullptr, nullptr, I, W, ws, nullptr), SPEC_EINVAL);
    expect("greedy K", spec_verify_greedy(P, SPEC_BF16, I, 2, 64, 1000, I, I, nullptr, nullptr, I, W, ws, nullptr), SPEC_EINVAL);
    expect("greedy V", spec_verify_greedy(P, SPEC_BF16, I, 2, 3, -5, I, I, nullptr, nullptr, I, W, ws, nullptr), SPEC_EINVAL);
    expect("greedy null", spec_verify_greedy(nullptr, SPEC_BF16, I, 2, 3, 1000, I, I, nullptr, nullptr, I, W, ws, nullptr), SPEC_EINVAL);
    expect("greedy ws", spec_verify_greedy(P, SPEC_BF16, I, 2, 3, 1000, I, I, nullptr, nullptr, I, W, 16, nullptr), SPEC_EWORKSPACE);
    expect("greedy grid", spec_verify_greedy(P, SPEC_BF16, I, 65536, 7, 262144, I, I, nullptr, nullptr, I, W, ws, nullptr), SPEC_EINVAL);
    // exact, power, relaxed, tree
    expect("exact draft", spec_verify_exact(P, nullptr, SPEC_BF16, I, F, 2, 3, 1000, I, I, nullptr, nullptr, I, W, ws, nullptr), SPEC_EINVAL);
    expect("exact ws", spec_verify_exact(P, P, SPEC_BF16, I, F, 2, 3, 1000, I, I, nullptr, nullptr, I, nullptr, ws, nullptr), SPEC_EWORKSPACE);
    expect("power alpha", spec_verify_power(P, P, SPEC_BF16, I, F, 2, 3, 1000, -1.f, I, I, nullptr, nullptr, I, W, ws, nullptr), SPEC_EINVAL);
    expect("power nan", spec_verify_power(P, P, SPEC_BF16, I, F, 2, 3, 1000, NAN, I, I, nullptr, nullptr, I, W, ws, nullptr), SPEC_EINVAL);
    expect("relaxed tau", spec_verify_relaxed(P, SPEC_BF16, I, F, 2, 3, 1000, NAN, 4, I, I, nullptr, nullptr, I, W, ws, nullptr), SPEC_EINVAL);
    expect("relaxed k", spec_verify_relaxed(P, SPEC_BF16, I, F, 2, 3, 1000, 0.1f, -2, I, I, nullptr, nullptr, I, W, ws, nullptr), SPEC_EINVAL);
    expect("tree N", spec_verify_tree(P, SPEC_BF16, I, I, nullptr, 2, 65, 1000, I, I, I, nullptr, nullptr, I, W, ws, nullptr), SPEC_EINVAL);
    expect("tree parents", spec_verify_tree(P, SPEC_BF16, I, nullptr, nullptr, 2, 8, 1000, I, I, I, nullptr, nullptr, I, W, ws, nullptr), SPEC_EINVAL);
    expect("sampler rows", spec_sample_drafts(P, SPEC_F32, F, 0, 100, I, F, I, W, ws, nullptr), SPEC_EINVAL);
    expect("sampler ws", spec_sample_drafts(P, SPEC_F32, F, 4, 100, I, F, I, W, 8, nullptr), SPEC_EWORKSPACE);

    // vocabulary shards: sizes, then gathered inputs one byte short
    const int G = 4, B = 2, K = 3, V = 1000;
    const size_t rec = spec_shard_record_bytes(SPEC_BF16, B, 2 * K + 1, V, G);
    const size_t grec = spec_shard_record_bytes(SPEC_BF16, B, K + 1, V, G);
    const size_t sums = spec_shard_sums_bytes(B, V, G), sws = spec_shard_workspace_bytes(B);
    const size_t vals = spec_shard_values_bytes(B, K);
    expect("shard sizes", rec > 0 && grec > 0 && sums > 0 && sws > 0 && vals > 0, 1);
    expect("shard bad G", spec_shard_record_bytes(SPEC_BF16, B, 4, V, 7) == 0, 1);
    expect("stats shard index", spec_shard_stats_exact(P, P, SPEC_BF16, I, B, K, V, G, G, W, rec, nullptr), SPEC_EINVAL);
    expect("stats record", spec_shard_stats_exact(P, P, SPEC_BF16, I, B, K, V, G, 0, W, rec - 1, nullptr), SPEC_EWORKSPACE);
    expect("combine short", spec_shard_combine_greedy(W, G * grec - 1, SPEC_BF16, I, B, K, V, G, I, I, nullptr, nullptr, I, nullptr), SPEC_EWORKSPACE);
    expect("combine tree short", spec_shard_combine_tree(W, 8, SPEC_BF16, I, I, nullptr, B, 8, V, G, I, I, I, nullptr, nullptr, I, nullptr), SPEC_EWORKSPACE);
    expect("sweep short", spec_shard_sweep_exact(P, P, SPEC_BF16, W, G * rec - 1, I, F, B, K, V, G, 0, I, I, nullptr, nullptr, I, W, sums, W, sws, nullptr), SPEC_EWORKSPACE);
    expect("sweep power short", spec_shard_sweep_power(P, P, SPEC_BF16, W, 0, I, F, B, K, V, G, 0, 0.5f, I, I, nullptr, nullptr, I, W, sums, W, sws, nullptr), SPEC_EWORKSPACE);
    expect("sweep relaxed short", spec_shard_sweep_relaxed(P, SPEC_BF16, W, G * grec - 1, I, F, B, K, V, G, 0, 0.1f, 4, I, I, nullptr, nullptr, I, W, sums, W, sws, nullptr), SPEC_EWORKSPACE);
    expect("sample short", spec_shard_sample_exact(P, P, SPEC_BF16, W, G * sums - 1, F, B, K, V, G, 0, I, nullptr, nullptr, nullptr, W, sws, nullptr), SPEC_EWORKSPACE);
    expect("sample power short", spec_shard_sample_power(P, P, SPEC_BF16, W, 1, F, B, K, V, G, 0, I, nullptr, nullptr, nullptr, W, sws, nullptr), SPEC_EWORKSPACE);
    expect("sample relaxed short", spec_shard_sample_relaxed(P, SPEC_BF16, W, G * sums - 1, F, B, K, V, G, 0, I, nullptr, nullptr, nullptr, W, sws, nullptr), SPEC_EWORKSPACE);
    expect("values short", spec_shard_values_relaxed(P, SPEC_BF16, I, B, K, V, G, 0, W, vals - 1, nullptr), SPEC_EWORKSPACE);
    expect("stats relaxed short", spec_shard_stats_relaxed(P, SPEC_BF16, I, W, G * vals - 1, B, K, V, G, 0, W, grec, nullptr), SPEC_EWORKSPACE);
    expect("read ceiling", spec_read_ceiling(P, 100, static_cast<uint32_t*>(P), nullptr), SPEC_EINVAL);
    expect("read ceiling words", spec_read_ceiling_out_words(16400) == 2, 1);

    std::printf("abi sanitizer driver: %d failures\n", failures);
    return failures ? 1 : 0;
}
