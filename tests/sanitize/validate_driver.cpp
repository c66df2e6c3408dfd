// Exercises the C ABI's argument checks (cp_validate.hpp) and the launchers'
// segment planning (cp_plan.hpp) on the host, built
// with -fsanitize=address,undefined by tests/test_sanitizers.py.  Pointers are
// fake, 16-byte aligned addresses that are never dereferenced.  Prints one
// line per failed expectation and exits with the number of failures.
#include <stdint.h>
#include <stdio.h>

#include "cp_plan.hpp"
#include "cp_validate.hpp"

static int failures = 0;

static void expect(int got, int want, const char *what) {
    if (got != want) {
        printf("FAIL %s: got %d, want %d\n", what, got, want);
        ++failures;
    }
}

static const void *P(int n) { return reinterpret_cast<const void *>(uintptr_t(0x1000000000ull) + uintptr_t(n) * 0x100000000ull); }
static const float *F(int n) { return static_cast<const float *>(P(n)); }

// Properties of a segment plan: every row in exactly one non-empty segment,
// segments of whole chunks, at least kMinSegChunks chunks each, only when the
// slices leave CUs idle, and the kernels' ceil(L / seg_len) gives nseg back.
static void check_plan(int L, int NS, int groups, int C, int wpc) {
    const cp::SegPlan p = cp::plan_segments(L, NS, groups, C, wpc);
    char what[160];
    snprintf(what, sizeof what, "plan L=%d NS=%d groups=%d C=%d wpc=%d -> %d x %d", L, NS, groups, C, wpc, p.nseg,
             p.seg_len);
    bool ok = p.nseg >= 1 && p.seg_len >= 1;
    if (ok && p.nseg == 1) ok = p.seg_len == L;
    if (ok && p.nseg > 1) {
        const long long covered = (long long)p.nseg * p.seg_len, before_last = (long long)(p.nseg - 1) * p.seg_len;
        ok = p.seg_len % C == 0 && before_last < L && covered >= L && p.seg_len >= cp::kMinSegChunks * C &&
             (long long)NS * groups < cp::kCUs && ((long long)L + p.seg_len - 1) / p.seg_len == p.nseg;
    }
    expect(ok ? 1 : 0, 1, what);
}

int main() {
    using namespace cp;
    // valid calls over every dtype and tile size, ragged and tiny lengths
    for (int dt : {CP_F32, CP_BF16, CP_F16})
        for (int64_t E : {16, 32, 40, 64, 80, 128})
            for (int64_t M : {16, 32, 64, 96, 128})
                for (int64_t L : {1, 17, 4096}) {
                    expect(validate_fwd(P(0), P(1), P(2), P(3), nullptr, nullptr, 2, 3, L, E, M, dt), CP_OK, "fwd ok");
                    expect(validate_bwd(P(0), P(1), P(2), P(3), F(4), F(5), P(6), P(7), P(8), nullptr, 2, 3, L, E, M,
                                        dt), CP_OK, "bwd ok");
                    expect(validate_linattn_fwd(P(0), P(1), P(2), P(3), nullptr, nullptr, F(4), F(5), F(6), 2, 3, L,
                                                E, M, 1e-6f, 1, dt), CP_OK, "linattn ok");
                    expect(validate_linattn_bwd(P(0), P(1), P(2), P(3), P(4), F(5), nullptr, nullptr, F(6), F(12), P(7),
                                                P(8), P(9), F(10), F(11), 2, 3, L, E, M, 0, dt), CP_OK,
                           "linattn bwd ok");
                }
    // sizes
    const int64_t big = INT64_MAX;
    for (int64_t bad : {int64_t(0), int64_t(-1), big}) {
        expect(validate_fwd(P(0), P(1), P(2), P(3), nullptr, nullptr, bad, 3, 100, 64, 64, CP_BF16), CP_ERR_DIM, "N");
        expect(validate_fwd(P(0), P(1), P(2), P(3), nullptr, nullptr, 2, bad, 100, 64, 64, CP_BF16), CP_ERR_DIM, "H");
        expect(validate_fwd(P(0), P(1), P(2), P(3), nullptr, nullptr, 2, 3, bad, 64, 64, CP_BF16), CP_ERR_DIM, "L");
    }
    expect(validate_fwd(P(0), P(1), P(2), P(3), nullptr, nullptr, 2, 3, 100, big, 64, CP_BF16), CP_ERR_UNSUPPORTED, "E big");
    expect(validate_fwd(P(0), P(1), P(2), P(3), nullptr, nullptr, 2, 3, 100, 0, 64, CP_BF16), CP_ERR_DIM, "E 0");
    expect(validate_fwd(P(0), P(1), P(2), P(3), nullptr, nullptr, INT32_MAX, INT32_MAX, INT32_MAX, 128, 128, CP_F32),
           CP_ERR_DIM, "overflow");
    expect(validate_fwd(P(0), P(1), P(2), P(3), nullptr, nullptr, 1 << 16, 1 << 10, int64_t(1) << 30, 128, 128, CP_F32),
           CP_ERR_DIM, "bytes overflow");
    expect(validate_fwd(P(0), P(1), P(2), P(3), nullptr, nullptr, 2, 3, 100, 129, 64, CP_BF16), CP_ERR_UNSUPPORTED, "E 129");
    expect(validate_fwd(P(0), P(1), P(2), P(3), nullptr, nullptr, 2, 3, 100, 60, 64, CP_BF16), CP_ERR_UNSUPPORTED, "E 60 bf16");
    expect(validate_fwd(P(0), P(1), P(2), P(3), nullptr, nullptr, 2, 3, 100, 60, 64, CP_F32), CP_OK, "E 60 f32");
    expect(validate_fwd(P(0), P(1), P(2), P(3), nullptr, nullptr, 2, 3, 100, 64, 64, 7), CP_ERR_UNSUPPORTED, "dtype");
    // pointers
    expect(validate_fwd(nullptr, P(1), P(2), P(3), nullptr, nullptr, 2, 3, 100, 64, 64, CP_BF16), CP_ERR_NULL, "null Q");
    expect(validate_fwd(static_cast<const char *>(P(0)) + 8, P(1), P(2), P(3), nullptr, nullptr, 2, 3, 100, 64, 64,
                        CP_BF16), CP_ERR_ALIGN, "align Q");
    expect(validate_fwd(P(0), P(1), P(2), P(3), F(4) + 1, nullptr, 2, 3, 100, 64, 64, CP_BF16), CP_ERR_ALIGN,
           "align S0");
    // aliasing: output inside an input, two outputs overlapping, an address
    // range reaching the end of the address space
    expect(validate_fwd(P(0), P(1), P(2), static_cast<const char *>(P(2)) + 16, nullptr, nullptr, 2, 3, 100, 64, 64,
                        CP_BF16), CP_ERR_ALIAS, "alias out/v");
    expect(validate_bwd(P(0), P(1), P(2), P(3), nullptr, nullptr, P(6), P(6), P(8), nullptr, 2, 3, 100, 64, 64,
                        CP_BF16), CP_ERR_ALIAS, "alias dq/dk");
    const void *top = reinterpret_cast<const void *>(UINTPTR_MAX & ~uintptr_t(15));
    expect(validate_fwd(P(0), P(1), P(2), top, nullptr, nullptr, 2, 3, 100, 64, 64, CP_BF16), CP_OK, "top ok");
    expect(validate_fwd(top, P(1), P(2), static_cast<const char *>(top) - 32, nullptr, nullptr, 2, 3, 100, 64, 64,
                        CP_BF16), CP_ERR_ALIAS, "top alias");
    // a caller's workspace counts as an output: aligned, disjoint from every tensor
    expect(validate_fwd(P(0), P(1), P(2), P(3), nullptr, nullptr, 2, 3, 100, 64, 64, CP_BF16, P(11), 1 << 20), CP_OK,
           "ws ok");
    expect(validate_fwd(P(0), P(1), P(2), P(3), nullptr, nullptr, 2, 3, 100, 64, 64, CP_BF16,
                        static_cast<const char *>(P(11)) + 4, 64), CP_ERR_ALIGN, "ws align");
    expect(validate_bwd(P(0), P(1), P(2), P(3), nullptr, nullptr, P(6), P(7), P(8), nullptr, 2, 3, 100, 64, 64, CP_BF16,
                        static_cast<const char *>(P(7)) + 64, 64), CP_ERR_ALIAS, "ws over dk");
    expect(validate_linattn_fwd(P(0), P(1), P(2), P(3), nullptr, nullptr, nullptr, nullptr, F(4), 2, 3, 100, 64, 64,
                                1e-6f, 1, CP_BF16, P(4), 16), CP_ERR_ALIAS, "ws over den_out");
    expect(validate_linattn_bwd(P(0), P(1), P(2), P(3), P(4), F(5), nullptr, nullptr, nullptr, nullptr, P(7), P(8),
                                P(9), nullptr, nullptr, 2, 3, 100, 64, 64, 1, CP_BF16, P(3), 16), CP_ERR_ALIAS,
           "ws over out");
    // normalised form: flags and eps
    expect(validate_linattn_fwd(P(0), P(1), P(2), P(3), nullptr, nullptr, nullptr, nullptr, nullptr, 2, 3, 100, 64, 64,
                                -1.f, 1, CP_BF16), CP_ERR_UNSUPPORTED, "eps < 0");
    expect(validate_linattn_fwd(P(0), P(1), P(2), P(3), nullptr, nullptr, nullptr, nullptr, nullptr, 2, 3, 100, 64, 64,
                                1.f / 0.f, 1, CP_BF16), CP_ERR_UNSUPPORTED, "eps inf");
    expect(validate_linattn_fwd(P(0), P(1), P(2), P(3), nullptr, nullptr, nullptr, nullptr, nullptr, 2, 3, 100, 64, 64,
                                1e-6f, 2, CP_BF16), CP_ERR_UNSUPPORTED, "feature map");
    expect(validate_linattn_bwd(P(0), P(1), P(2), P(3), P(4), nullptr, nullptr, nullptr, nullptr, nullptr, P(7), P(8),
                                P(9), nullptr, nullptr, 2, 3, 100, 64, 64, 1, CP_BF16), CP_ERR_NULL, "den required");
    expect(validate_linattn_bwd(P(0), P(1), P(2), P(3), P(4), F(5), nullptr, nullptr, nullptr, nullptr, P(7), P(8),
                                P(9), F(5), nullptr, 2, 3, 100, 64, 64, 1, CP_BF16), CP_ERR_ALIAS, "dS0 over den");
    expect(validate_linattn_bwd(P(0), P(1), P(2), P(3), P(4), F(5), nullptr, nullptr, nullptr, F(11), P(7), P(8),
                                P(9), nullptr, F(11), 2, 3, 100, 64, 64, 1, CP_BF16), CP_ERR_ALIAS, "dz0 over z_final");
    for (int64_t x = -3; x <= 200; ++x) {
        const int t = tile_index(x);
        const int want = x < 1 ? -1 : x <= 16 ? 0 : x <= 32 ? 1 : x <= 64 ? 2 : x <= 128 ? 3 : -1;
        expect(t, want, "tile_index");
    }
    // segment plans over lengths, slice counts, groups, chunks and targets
    for (int C : {16, 32, 64, 128})
        for (int groups : {1, 2, 4})
            for (int wpc : {1, 2})
                for (int NS : {1, 2, 3, 7, 16, 33, 100, 127, 128, 255, 256, 1000})
                    for (long long L : {1LL, 63LL, 64LL, 65LL, 511LL, 512LL, 513LL, 1000LL, 1500LL, 2085LL, 4096LL,
                                        16384LL, 100003LL, 1LL << 24, (long long)INT32_MAX - 5, (long long)INT32_MAX})
                        check_plan((int)L, NS, groups, C, wpc);

    printf("%d failures\n", failures);
    return failures;
}
