// Host-only driver of the C-ABI layer (capi.hip) for sanitizer runs on the CPU.
//
// capi.hip is compiled for the host alone and linked against the stub launchers
// below instead of the GPU kernels, so every entry point's validation and
// dispatch runs under AddressSanitizer and UndefinedBehaviorSanitizer with no
// GPU.  Fake, never dereferenced device addresses are used; the stubs record
// what reached them.  Exit status 0 when every expectation holds.
#include <stdio.h>
#include <string.h>

#include "../../include/based_la.h"
#include "../../recurrent_lm_sequence_amd/csrc/common.h"

namespace {
int g_calls = 0;
bla::PrefillArgs g_pf;
int g_split = -1;
bla::DecodeArgs g_dec;
bla::SwaArgs g_swa;
}  // namespace

namespace bla {
hipError_t launch_prefill_sym(const PrefillArgs &a, int split_ok, hipStream_t)
{
    ++g_calls;
    g_pf = a;
    g_split = split_ok;
    return hipSuccess;
}
hipError_t launch_prefill_exact(const PrefillArgs &a, int, hipStream_t)
{
    ++g_calls;
    g_pf = a;
    return hipSuccess;
}
hipError_t launch_decode(const DecodeArgs &a, int, hipStream_t)
{
    ++g_calls;
    g_dec = a;
    return hipSuccess;
}
hipError_t launch_swa_prefill(const SwaArgs &a, hipStream_t)
{
    ++g_calls;
    g_swa = a;
    return hipSuccess;
}
hipError_t launch_swa_decode(const SwaArgs &a, int, hipStream_t)
{
    ++g_calls;
    g_swa = a;
    return hipSuccess;
}
}  // namespace bla

static int failures = 0;
#define EXPECT(cond)                                                      \
    do {                                                                  \
        if (!(cond)) {                                                    \
            fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__,  \
                    __LINE__, #cond);                                     \
            ++failures;                                                   \
        }                                                                 \
    } while (0)

static void *A(long long n) { return (void *)(uintptr_t)(n << 24); }  // 16 MiB apart, aligned
static float *F(long long n) { return (float *)A(n); }

int main()
{
    // status strings, dims
    for (int s = 0; s < 4; ++s) EXPECT(strncmp(bla_status_string((bla_status)s), "BLA_", 4) == 0);
    EXPECT(strstr(bla_status_string((bla_status)99), "unknown") != nullptr);
    EXPECT(bla_feature_dim(16) == 273 && bla_feature_dim(0) == -1 && bla_feature_dim(1 << 30) == -1);
    EXPECT(bla_compact_dim(16) == 153 && bla_compact_dim(-3) == -1);

    // a valid bf16 prefill reaches the chunked kernel with the call's arguments
    g_calls = 0;
    EXPECT(based_prefill(2, 3, 100, 16, 64, BLA_BF16, BLA_F32, 0.f, A(1), A(2), A(3), nullptr,
                         nullptr, A(4), F(5), F(6), nullptr) == BLA_OK);
    EXPECT(g_calls == 1 && g_pf.B == 2 && g_pf.H == 3 && g_pf.N == 100 && g_pf.M == 0 && g_pf.dv == 64);
    EXPECT(g_pf.y == A(4) && g_pf.S_out == F(5) && g_pf.z_out == F(6) && !g_pf.compact && g_split == 1);
    // in-place z keeps one workgroup per head
    EXPECT(based_prefill(2, 3, 100, 16, 64, BLA_BF16, BLA_F32, 0.f, A(1), A(2), A(3), F(5), F(6),
                         A(4), F(5), F(6), nullptr) == BLA_OK);
    EXPECT(g_split == 0);
    // N = 0: y is not produced, the state still is
    EXPECT(based_prefill(2, 3, 0, 16, 64, BLA_BF16, BLA_F32, 0.f, nullptr, nullptr, nullptr, F(5),
                         F(6), A(4), F(7), F(8), nullptr) == BLA_OK);
    EXPECT(g_pf.y == nullptr);
    // nothing to produce: no launch
    g_calls = 0;
    EXPECT(based_prefill(2, 3, 10, 16, 64, BLA_BF16, BLA_F32, 0.f, A(1), A(2), A(3), nullptr,
                         nullptr, nullptr, nullptr, nullptr, nullptr) == BLA_OK);
    EXPECT(g_calls == 0);
    // invalid arguments never launch
    EXPECT(based_prefill(0, 3, 10, 16, 64, BLA_BF16, BLA_F32, 0.f, A(1), A(2), A(3), nullptr, nullptr,
                         A(4), nullptr, nullptr, nullptr) == BLA_ERR_INVALID);
    EXPECT(based_prefill(2, 3, 10, 16, 64, (bla_dtype)7, BLA_F32, 0.f, A(1), A(2), A(3), nullptr, nullptr,
                         A(4), nullptr, nullptr, nullptr) == BLA_ERR_INVALID);
    EXPECT(based_prefill(2, 3, 10, 8, 64, BLA_BF16, BLA_F32, 0.f, A(1), A(2), A(3), nullptr, nullptr,
                         A(4), nullptr, nullptr, nullptr) == BLA_ERR_UNSUPPORTED);
    EXPECT(based_prefill(2, 3, 10, 16, 64, BLA_BF16, BLA_F32, 0.f, (char *)A(1) + 8, A(2), A(3), nullptr,
                         nullptr, A(4), nullptr, nullptr, nullptr) == BLA_ERR_INVALID);
    EXPECT(based_prefill(2, 3, 10, 16, 64, BLA_BF16, BLA_F32, 0.f, A(1), A(2), A(3), F(5), nullptr,
                         A(4), nullptr, nullptr, nullptr) == BLA_ERR_INVALID);
    EXPECT(based_prefill(2, 3, 10, 16, 64, BLA_BF16, BLA_F32, 0.f, A(1), A(2), A(3), F(5), F(6),
                         A(4), (float *)((char *)A(5) + 256), F(9), nullptr) == BLA_ERR_INVALID);
    EXPECT(based_prefill(1 << 12, 1 << 11, 1, 16, 64, BLA_BF16, BLA_F32, 0.f, A(1), A(2), A(3), nullptr,
                         nullptr, A(4), nullptr, nullptr, nullptr) == BLA_ERR_UNSUPPORTED);
    EXPECT(based_prefill((1 << 11) + 1, 1 << 10, 1, 16, 32, BLA_F32, BLA_F32, 0.f, A(1), A(2), A(3),
                         nullptr, nullptr, A(4), nullptr, nullptr, nullptr) == BLA_ERR_UNSUPPORTED);
    EXPECT(g_calls == 0);

    // fp32 inputs take the exact kernel; JRT passes M and the prefix pointers; compact layout
    EXPECT(based_prefill(1, 1, 256, 16, 16, BLA_F32, BLA_F32, 0.f, A(1), A(2), A(3), nullptr, nullptr,
                         A(4), nullptr, nullptr, nullptr) == BLA_OK);
    EXPECT(g_calls == 1 && g_pf.dv == 16);
    EXPECT(jrt_prefix_prefill(2, 2, 50, 30, 16, 64, BLA_BF16, BLA_F32, 0.f, A(1), A(2), A(3), A(10),
                              A(11), nullptr, nullptr, A(4), F(5), F(6), nullptr) == BLA_OK);
    EXPECT(g_pf.M == 30 && g_pf.ke == A(10) && g_pf.ve == A(11) && g_pf.prefix_len == nullptr);
    EXPECT(jrt_prefix_prefill(2, 2, 50, 30, 16, 64, BLA_BF16, BLA_F32, 0.f, A(1), A(2), A(3), nullptr,
                              A(11), nullptr, nullptr, A(4), F(5), F(6), nullptr) == BLA_ERR_INVALID);
    EXPECT(jrt_prefix_prefill_ex(2, 2, 50, 30, 16, 64, BLA_BF16, BLA_F32, 0.f, A(1), A(2), A(3), A(10),
                                 A(11), (const int *)A(12), nullptr, nullptr, A(4), F(5), F(6),
                                 BLA_STATE_COMPACT, nullptr) == BLA_OK);
    EXPECT(g_pf.compact == 1 && g_pf.prefix_len == (const int *)A(12));
    EXPECT(jrt_prefix_prefill_ex(2, 2, 50, 30, 16, 64, BLA_BF16, BLA_F32, 0.f, A(1), A(2), A(3), A(10),
                                 A(11), nullptr, nullptr, nullptr, A(4), F(5), F(6),
                                 (bla_state_layout)5, nullptr) == BLA_ERR_INVALID);
    EXPECT(based_prefill_compact(2, 2, 50, 16, 32, BLA_BF16, BLA_BF16, 0.f, A(1), A(2), A(3), nullptr,
                                 nullptr, A(4), F(5), F(6), nullptr) == BLA_OK);
    EXPECT(g_pf.compact == 1 && g_pf.y_bf16 == 1);

    // decode and its aliasing checks
    EXPECT(based_decode_step(4, 16, 16, 64, BLA_BF16, BLA_F32, 0.f, A(1), A(2), A(3), F(5), F(6), A(4),
                             nullptr) == BLA_OK);
    EXPECT(g_dec.B == 4 && g_dec.H == 16 && g_dec.S == F(5) && g_dec.z == F(6) && !g_dec.compact);
    EXPECT(based_decode_step_compact(4, 16, 16, 64, BLA_BF16, BLA_F32, 0.f, A(1), A(2), A(3), F(5),
                                     (float *)((char *)A(5) + 4096), A(4), nullptr) == BLA_ERR_INVALID);
    EXPECT(based_decode_step(4, 16, 16, 64, BLA_BF16, BLA_F32, 0.f, A(1), A(2), A(3), nullptr, F(6), A(4),
                             nullptr) == BLA_ERR_INVALID);

    // sliding-window attention
    EXPECT(swa_prefill(2, 2, 300, 64, 64, 128, BLA_BF16, BLA_F32, A(1), A(2), A(3), A(4), A(5), A(6),
                       nullptr) == BLA_OK);
    EXPECT(g_swa.window == 128 && g_swa.N == 300 && g_swa.k_cache == A(5));
    EXPECT(swa_prefill(2, 2, 300, 64, 64, 257, BLA_BF16, BLA_F32, A(1), A(2), A(3), A(4), nullptr,
                       nullptr, nullptr) == BLA_ERR_UNSUPPORTED);
    EXPECT(swa_decode_step(2, 2, 64, 64, 64, 70, BLA_F32, BLA_F32, A(1), A(2), A(3), A(5), A(6), A(4),
                           nullptr) == BLA_OK);
    EXPECT(g_swa.pos == 70);
    EXPECT(swa_decode_step(2, 2, 64, 64, 64, -1, BLA_F32, BLA_F32, A(1), A(2), A(3), A(5), A(6), A(4),
                           nullptr) == BLA_ERR_INVALID);

    if (failures) {
        fprintf(stderr, "%d expectation(s) failed\n", failures);
        return 1;
    }
    printf("capi driver: all expectations hold\n");
    return 0;
}
