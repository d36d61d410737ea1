// Host-side checks of libtlg's plan logic under AddressSanitizer and
// UndefinedBehaviorSanitizer: argument validation, variant choice, plan geometry,
// describe strings, the no-alloc entry point's refusals and destroy.  Only calls
// that return before any device work are made, so no GPU is needed.
#include <cstdio>
#include <cstdint>
#include <cstring>

#include "../../include/tlg.h"

static int fails = 0;
#define CHECK(c)                                                       \
    do {                                                               \
        if (!(c)) {                                                    \
            std::printf("FAIL %s:%d %s\n", __FILE__, __LINE__, #c);    \
            ++fails;                                                   \
        }                                                              \
    } while (0)

int main()
{
    const int64_t shapes[][3] = {{0, 5, 7},       {1, 1, 1},        {16, 16384, 8192}, {1000, 1500, 777},
                                 {4600, 4350, 4100}, {8192, 8192, 8192}, {1024, 1024, 4096}, {255, 257, 0},
                                 {1 << 24, 1, 1},  {3, 1 << 24, 64}};
    int plans = 0;
    for (const auto& s : shapes)
        for (int v = 0; v <= 12; ++v)
            for (int ab = 1; ab <= 6; ++ab)
                for (int tA = 0; tA <= 1; ++tA)
                    for (int tB = 0; tB <= 1; ++tB) {
                        tlg_plan_info info;
                        std::memset(&info, 0x5A, sizeof(info));
                        const tlg_status st = tlg_gemm_select(&info, s[0], s[1], s[2], ab, 1, tA, tB, 1, 0, v);
                        if (st != TLG_OK) continue;
                        CHECK(info.grid >= 0 && info.k_tiles >= 0 && info.splits >= 1);
                        // plans that own no workspace are made and destroyed without a device
                        if (info.workspace_bytes == 0) {
                            tlg_gemm_t p = nullptr;
                            const tlg_status cs = v == 0 ? tlg_gemm_create(&p, s[0], s[1], s[2], ab, 1, tA, tB, 1, 0)
                                                         : tlg_gemm_create_variant(&p, s[0], s[1], s[2], ab, 1, tA,
                                                                                   tB, 1, 0, v);
                            CHECK(cs == TLG_OK && p != nullptr);
                            const char* d = tlg_gemm_describe(p);
                            CHECK(d != nullptr && std::strlen(d) > 10 && std::strlen(d) < 256);
                            tlg_plan_info q;
                            CHECK(tlg_gemm_query(p, &q) == TLG_OK && q.variant == info.variant && q.grid == info.grid);
                            // runs refused before any launch: null or overlapping buffers
                            if (q.variant != TLG_VARIANT_EMPTY && (ab == 1 || ab == 2)) {
                                CHECK(tlg_gemm_run(p, nullptr, nullptr, nullptr, nullptr) == TLG_ERR_NULL);
                                if (s[2] > 0) {
                                    char* a = reinterpret_cast<char*>(uintptr_t(1) << 20);
                                    CHECK(tlg_gemm_run(p, a, a + (uintptr_t(1) << 34), a, nullptr) ==
                                          TLG_ERR_INVALID_ARG);
                                }
                            }
                            CHECK(tlg_gemm_destroy(p) == TLG_OK);
                            ++plans;
                        }
                    }
    CHECK(tlg_gemm_destroy(nullptr) == TLG_OK);
    CHECK(std::strcmp(tlg_status_string(-7), "TLG_ERR_TOO_LARGE") == 0);
    CHECK(std::strcmp(tlg_status_string(12345), "TLG_ERR_UNKNOWN") == 0);
    CHECK(tlg_gemm_run_noalloc(-1, 1, 1, 1, 1, 0, 0, 1, 0, nullptr, nullptr, nullptr, nullptr) == TLG_ERR_INVALID_ARG);
    CHECK(tlg_gemm_run_noalloc(4, 4, 128, 6, 1, 0, 1, 1, 0, nullptr, nullptr, nullptr, nullptr) == TLG_ERR_UNSUPPORTED);
    CHECK(tlg_gemm_run_noalloc(0, 4, 4, 1, 1, 0, 0, 1, 0, nullptr, nullptr, nullptr, nullptr) == TLG_OK);
    std::printf("host checks: %d plans made and destroyed, %d failures\n", plans, fails);
    return fails ? 1 : 0;
}
