// Sanitizer driver for the host side of the C ABI: validation, launch
// planning, workspace layout (favor_api.cpp, favor_plan.cpp, with the kernel
// launcher replaced by stub_launch.cpp) and the host projection generator
// (orf_omega.cpp), built with AddressSanitizer and UndefinedBehaviorSanitizer.
// Device pointers are fake addresses the library never dereferences; the
// projection generator writes exactly-sized heap buffers.  Exit status 0 and
// no sanitizer report mean success.  Test infrastructure only.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../../include/favor.h"

extern "C" {
extern const char* g_ws_base;
extern size_t g_ws_bytes;
extern int g_launches;
}

static int failures = 0;
#define EXPECT(c)                                                          \
    do {                                                                   \
        if (!(c)) {                                                        \
            std::fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #c); \
            ++failures;                                                    \
        }                                                                  \
    } while (0)

static void* fake(uintptr_t a) { return reinterpret_cast<void*>(a); }

int main() {
    const uintptr_t Q = 0x100000000ULL, K = 0x200000000ULL, V = 0x300000000ULL, O = 0x400000000ULL,
                    OM = 0x500000000ULL, WS = 0x600000000ULL;
    const int ds[] = {8, 16, 32, 48, 64, 128, 256};
    const int ms[] = {16, 32, 64, 96, 128, 160, 256, 320, 512, 544};
    const int Ls[] = {0, 1, 31, 32, 33, 63, 64, 65, 97, 1000, 4096, 8192, 65536};
    const int BHs[][2] = {{1, 1}, {1, 3}, {2, 8}, {4, 8}, {1, 16}, {3, 5}};
    const int segs[] = {0, 1, 2, 3, 7, 64, 255, 256};
    const int chunks[] = {0, 32, 64, 16};
    long calls = 0;
    for (int dtype = 0; dtype < 2; ++dtype)
        for (int feature = 0; feature < 2; ++feature)
            for (int d : ds)
                for (int m : ms)
                    for (auto& bh : BHs)
                        for (int L : Ls)
                            for (int per_head = 0; per_head < 2; ++per_head) {
                                favor_shape s{bh[0], bh[1], L, d, m, (favor_dtype)dtype,
                                              per_head ? (long long)m * d : 0, feature};
                                for (int op = 0; op < 3; ++op)
                                    for (int seg : segs)
                                        for (int chunk : chunks) {
                                            if (op != 2 && chunk != 0) continue;
                                            favor_plan pl{chunk, seg};
                                            const size_t need = favor_workspace_bytes_plan(op, &s, &pl);
                                            g_ws_base = reinterpret_cast<const char*>(WS);
                                            g_ws_bytes = need;
                                            const int before = g_launches;
                                            favor_status st;
                                            if (op == 0)
                                                st = favor_features(&s, fake(Q), (const float*)fake(OM), (float*)fake(O),
                                                                    (float*)fake(K), 1, fake(WS), need, nullptr);
                                            else if (op == 1)
                                                st = favor_bidir_plan(&s, fake(Q), fake(K), fake(V), (const float*)fake(OM),
                                                                      fake(O), &pl, fake(WS), need, nullptr);
                                            else
                                                st = favor_causal_plan(&s, fake(Q), fake(K), fake(V), (const float*)fake(OM),
                                                                       fake(O), &pl, fake(WS), need, nullptr);
                                            ++calls;
                                            // a call is accepted exactly when the workspace query accepts the shape
                                            // and plan (L = 0 is a no-op either way)
                                            if (need > 0) {
                                                EXPECT(st == FAVOR_OK);
                                                EXPECT(g_launches == before + (L > 0 ? 1 : 0));
                                                if (need >= 256 && L > 0) {
                                                    // one byte short is refused before any launch
                                                    const int b2 = g_launches;
                                                    favor_status s2 =
                                                        op == 1 ? favor_bidir_plan(&s, fake(Q), fake(K), fake(V),
                                                                                   (const float*)fake(OM), fake(O), &pl,
                                                                                   fake(WS), need - 1, nullptr)
                                                        : op == 2 ? favor_causal_plan(&s, fake(Q), fake(K), fake(V),
                                                                                      (const float*)fake(OM), fake(O), &pl,
                                                                                      fake(WS), need - 1, nullptr)
                                                                  : FAVOR_ERR_WORKSPACE;
                                                    EXPECT(s2 == FAVOR_ERR_WORKSPACE);
                                                    EXPECT(g_launches == b2);
                                                }
                                            } else {
                                                EXPECT(st != FAVOR_OK || L == 0);
                                                EXPECT(g_launches == before);
                                            }
                                        }
                            }
    // carried-state entry point and the profiled ones over a smaller grid
    for (int L : Ls) {
        favor_shape s{2, 8, L, 64, 256, FAVOR_BF16, 0, 0};
        const size_t need = favor_workspace_bytes(FAVOR_OP_CAUSAL, &s, 0);
        g_ws_base = reinterpret_cast<const char*>(WS);
        g_ws_bytes = need;
        favor_status st = favor_causal_state(&s, fake(Q), fake(K), fake(V), (const float*)fake(OM), fake(O), 0,
                                             (const float*)fake(0x700000000ULL), (float*)fake(0x780000000ULL),
                                             fake(WS), need, nullptr);
        EXPECT(st == FAVOR_OK);
        void* ev[4] = {fake(1), fake(2), fake(3), fake(4)};
        st = favor_causal_profiled(&s, fake(Q), fake(K), fake(V), (const float*)fake(OM), fake(O), 0, fake(WS), need,
                                   nullptr, ev, 4);
        EXPECT(st == FAVOR_OK);
        EXPECT(favor_causal_profiled(&s, fake(Q), fake(K), fake(V), (const float*)fake(OM), fake(O), 0, fake(WS),
                                     need, nullptr, ev, 3) == FAVOR_ERR_INVALID_ARG);
    }
    // features over the Hadamard projection by transforms (no workspace)
    for (int d : ds)
        for (int m : ms)
            for (int L : Ls)
                for (int stab = 0; stab < 2; ++stab) {
                    favor_shape s{2, 3, L, d, m, FAVOR_BF16, (long long)m * d, 0};
                    const int before = g_launches;
                    const favor_status st = favor_features_hadamard(&s, fake(Q), 5, (float*)fake(O),
                                                                    stab ? (float*)fake(K) : nullptr, stab, nullptr);
                    const bool shape_ok = (d == 16 || d == 32 || d == 64 || d == 128) && m % 32 == 0 && m <= 512 &&
                                          (m <= 256 || m % 64 == 0);
                    EXPECT(st == (shape_ok ? FAVOR_OK : FAVOR_ERR_UNSUPPORTED));
                    EXPECT(g_launches == before + (shape_ok && L > 0 ? 1 : 0));
                    ++calls;
                }
    {
        favor_shape s{1, 1, 64, 64, 256, FAVOR_BF16, 0, 0};
        EXPECT(favor_features_hadamard(&s, fake(Q), 5, (float*)fake(Q), nullptr, 0, nullptr) == FAVOR_ERR_INVALID_ARG);
        EXPECT(favor_features_hadamard(&s, fake(Q), 5, (float*)fake(O), nullptr, 1, nullptr) == FAVOR_ERR_INVALID_ARG);
        EXPECT(favor_features_hadamard(nullptr, fake(Q), 5, (float*)fake(O), nullptr, 0, nullptr) ==
               FAVOR_ERR_INVALID_ARG);
    }
    // extreme dimensions: no overflow in the size computations (UBSan)
    {
        favor_shape big{1 << 16, 1 << 8, 1 << 8, 64, 256, FAVOR_BF16, 0, 0};
        EXPECT(favor_workspace_bytes(FAVOR_OP_CAUSAL, &big, 0) == 0);
        favor_shape huge{2147483647, 2147483647, 2147483647, 128, 512, FAVOR_BF16, 0, 0};
        EXPECT(favor_workspace_bytes(FAVOR_OP_BIDIR, &huge, 0) == 0);
        EXPECT(favor_bidir(&huge, fake(Q), fake(K), fake(V), (const float*)fake(OM), fake(O), fake(WS), 1, nullptr) ==
               FAVOR_ERR_UNSUPPORTED);
        favor_shape neg{1, 1, -2147483647 - 1, 64, 256, FAVOR_BF16, 0, 0};
        EXPECT(favor_workspace_bytes(FAVOR_OP_CAUSAL, &neg, 0) == 0);
    }
    // host projection generator: exactly-sized heap buffers
    for (int d : {1, 2, 3, 4, 16, 17, 64, 128})
        for (int m : {1, 5, 16, 33, 256, 512})
            for (int H : {1, 3}) {
                std::vector<float> out((size_t)H * m * d);
                EXPECT(favor_orf_omega(7, H, m, d, out.data()) == FAVOR_OK);
                for (float x : out) EXPECT(x == x);
            }
    EXPECT(favor_orf_omega(0, 1, 4, 4, nullptr) == FAVOR_ERR_INVALID_ARG);
    for (int c = -1; c <= 6; ++c) EXPECT(favor_status_string((favor_status)c) != nullptr);
    std::printf("abi_driver: %ld planned calls, %d launches, %d failures\n", calls, g_launches, failures);
    return failures == 0 ? 0 : 1;
}
