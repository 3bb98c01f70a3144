// Host-sanitizer driver for the library's host code (test infrastructure).
// tests/test_host_sanitizers.py builds the C ABI layer (capi.cpp) with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host side, links it
// with launch_stubs.cpp in place of the kernels, and runs this driver.  It needs no GPU: it sweeps the workspace
// planners over a grid of shapes up to the documented limits (integer
// overflow in the size arithmetic is undefined behaviour the sanitizer
// reports), and calls every entry point with arguments each check must
// reject before anything is enqueued (so no pointer below is ever handed to
// a kernel), expecting a nonzero status and an error message.
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../include/spec_verify.h"

static int g_fail = 0;
#define EXPECT(cond, what)                                                                                   \
    do {                                                                                                     \
        if (!(cond)) {                                                                                       \
            std::fprintf(stderr, "FAIL: %s\n", what);                                                        \
            g_fail = 1;                                                                                      \
        }                                                                                                    \
    } while (0)

int main()
{
    EXPECT(sv_abi_version() == 1, "abi version");
    for (int s = -2; s < 12; ++s)
        EXPECT(sv_status_string(s) != nullptr, "status string");

    // Planner sweep (sizes only; nothing is enqueued).
    const int Bs[] = {1, 2, 3, 64, 1024, 1025};
    const int Ts[] = {1, 7, 8, 16};
    const int Gs[] = {1, 2, 4, 8};
    const int Hkvs[] = {1, 2, 6, 8, 15, 16};
    const int ds[] = {64, 128};
    const int mbs[] = {1, 17, 512, 8192, 65536};
    const int bpss[] = {-1, 0, 4, 64, 512};
    size_t checksum = 0;
    for (int B : Bs)
        for (int T : Ts)
            for (int G : Gs)
                for (int Hkv : Hkvs)
                    for (int d : ds)
                        for (int mb : mbs) {
                            const int Hq = G * Hkv;
                            checksum += spec_verify_attn_workspace_size(B, T, Hq, Hkv, d, mb);
                            for (int bps : bpss)
                                checksum += spec_verify_attn_workspace_size_ex(B, T, Hq, Hkv, d, mb, bps);
                        }
    const int Vs[] = {1, 1000, 32000, 128256, 1 << 20};
    for (int B : Bs)
        for (int K : Ts)
            for (int V : Vs) {
                checksum += spec_verify_sample_workspace_size(B, K, V);
                checksum += spec_verify_sample_tree_workspace_size(B, K, V);
            }
    EXPECT(checksum > 0, "planner sizes");
    EXPECT(spec_verify_attn_noalloc_max_bytes() > 0, "no-alloc maximum");
    EXPECT(spec_verify_probe_read_sink_floats() > 0, "probe sink size");

    // Argument checks: every call below must be rejected before anything is
    // enqueued, with a message.
    alignas(256) static unsigned char buf[1 << 16];
    void *p = buf;
    const float *f = reinterpret_cast<const float *>(buf);
    float *fo = reinterpret_cast<float *>(buf);
    const int32_t *i32 = reinterpret_cast<const int32_t *>(buf);
    int32_t *io = reinterpret_cast<int32_t *>(buf);
    auto rejected = [&](int status, const char *what) {
        EXPECT(status != 0, what);
        const char *m = sv_last_error();
        EXPECT(m != nullptr && std::strlen(m) > 0, "error message");
    };
    rejected(spec_verify_attn(nullptr, p, p, nullptr, nullptr, i32, i32, fo, 2, 5, 32, 8, 128, 16, 8, 16, 1, 0.1f,
                              p, 1 << 14, nullptr),
             "attention: null q");
    rejected(spec_verify_attn(f, p, p, nullptr, nullptr, i32, i32, fo, 2, 17, 32, 8, 128, 16, 8, 16, 1, 0.1f, p,
                              1 << 14, nullptr),
             "attention: T > 16");
    rejected(spec_verify_attn(f, p, p, nullptr, nullptr, i32, i32, fo, 2, 5, 32, 8, 96, 16, 8, 16, 1, 0.1f, p,
                              1 << 14, nullptr),
             "attention: d = 96");
    rejected(spec_verify_attn(f, p, p, nullptr, nullptr, i32, i32, fo, 2, 5, 32, 8, 128, 16, 8, 16, 1, 0.1f, p, 16,
                              nullptr),
             "attention: workspace too small");
    rejected(spec_verify_attn_ex(f, p, p, nullptr, nullptr, i32, i32, fo, 2, 5, 32, 8, 128, 16, 8, 16, 1, 0.1f, p,
                                 1 << 14, nullptr, 0, 10, nullptr),
             "attention: split not a multiple of 4");
    rejected(spec_verify_attn_ex(f, p, p, nullptr, nullptr, i32, i32, fo, 1025, 5, 32, 8, 128, 16, 8, 16, 1, 0.1f,
                                 p, 1 << 14, nullptr, 0, -1, nullptr),
             "attention: balanced shares beyond 1024 sequences");
    rejected(spec_verify_attn_tree(f, p, p, nullptr, nullptr, i32, i32, nullptr, fo, 2, 4, 8, 2, 64, 16, 4, 8, 1,
                                   0.125f, p, 1 << 14, nullptr, 0, 0),
             "tree attention: null mask");
    rejected(spec_verify_attn_noalloc(f, p, p, nullptr, nullptr, i32, i32, fo, 1024, 8, 32, 8, 128, 16, 8192,
                                      16, 1, 0.1f, nullptr),
             "no-alloc attention: plan beyond the static scratch");
    rejected(spec_verify_sample(nullptr, f, i32, f, io, io, nullptr, 2, 3, 100, p, 1 << 14, nullptr),
             "sampler: null logits");
    rejected(spec_verify_sample(f, f, i32, f, io, io, nullptr, 2, 16, 100, p, 1 << 14, nullptr),
             "sampler: K = 16");
    rejected(spec_verify_sample_ex(f, f, i32, f, nullptr, f, io, io, nullptr, 2, 3, 1 << 20, p, 1 << 30, nullptr),
             "sampler: top-p with V >= 2^20");
    rejected(spec_verify_sample_typical(f, i32, f, nullptr, -0.1, 0.3, io, io, nullptr, nullptr, 2, 3, 100, p,
                                        1 << 14, nullptr),
             "typical: negative eps");
    rejected(spec_verify_sample_tree(f, f, i32, i32, f, io, io, io, nullptr, 2, 17, 100, 2, p, 1 << 18, nullptr),
             "tree sampler: N > 16");
    rejected(spec_verify_kv_append(nullptr, f, p, p, nullptr, nullptr, i32, i32, 2, 5, 8, 128, 16, 8, 16, 1,
                                   nullptr),
             "append: null k_new");
    rejected(spec_verify_rollback(nullptr, io, io, 2, 3, nullptr), "rollback: null counts");
    rejected(spec_verify_tree_commit(nullptr, i32, p, p, nullptr, nullptr, i32, io, io, 2, 4, 8, 128, 16, 8, 16, 1,
                                     nullptr),
             "tree commit: null path");
    rejected(spec_verify_check_inputs(i32, i32, 5, 8, 16, nullptr, 0, 100, nullptr, 0, 0, io, nullptr),
             "check inputs: B = 0");
    rejected(spec_verify_probe_read(p, 1 << 10, fo, 1, nullptr), "probe: sink too small");

    if (g_fail)
        return 1;
    std::printf("ok %zu\n", checksum);
    return 0;
}
