// Host-side driver for the address and undefined-behaviour sanitizer build of
// the library's host code (built and run by tests/test_host_sanitize.py on the
// CPU).  It sizes many descriptors, valid and invalid, checks the plan's
// invariants, and calls every entry point with arguments its validation
// refuses, so that no call reaches a launch.  Exit status 0 when every check
// holds; the sanitizers abort the run on the first error they find.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../include/lighthouse.h"

namespace {

int g_failures = 0;

void check(bool ok, const char* what, int line) {
    if (!ok) {
        fprintf(stderr, "check failed at line %d: %s\n", line, what);
        ++g_failures;
    }
}
#define CHECK(x) check((x), #x, __LINE__)

void* fake(uintptr_t off = 0) { return reinterpret_cast<void*>(uintptr_t(0x100000) + off); }

lh_desc make(int64_t B, int64_t H, int64_t N, int64_t d, int p, int L, int k, int dtype) {
    lh_desc x;
    memset(&x, 0, sizeof x);
    x.B = B; x.H = H; x.N = N; x.d = d; x.p = p; x.L = L; x.k = k; x.dtype = dtype; x.scale = 0.f;
    return x;
}

// Invariants of a successful plan (the entry counts of the pyramid and the
// sub-sequence length the header documents).
void check_plan(const lh_desc& x, const lh_plan& P) {
    int64_t pw = 1, off = 0, S = 0;
    for (int l = 0; l < x.L; ++l) {
        CHECK(P.M[l] == x.N / pw);
        CHECK(P.level_off[l] == off);
        CHECK(P.k_eff[l] >= 0 && P.k_eff[l] <= P.M[l]);
        if (l >= 1) S += (int64_t)x.p * P.k_eff[l];
        off += P.M[l];
        pw *= x.p;
    }
    S += P.M[x.L - 1];
    CHECK(P.level_off[x.L] == off && P.M_total == off);
    CHECK(P.S == S && P.S <= P.M_total);
    CHECK(P.S_pad % 64 == 0 && P.S_pad >= P.S && P.S_pad < P.S + 64);
    for (int i = 1; i < 8; ++i) CHECK(P.fwd_off[i] >= P.fwd_off[i - 1] && P.fwd_off[i] % 256 == 0);
    for (int i = 1; i < 7; ++i) CHECK(P.bwd_off[i] >= P.bwd_off[i - 1] && P.bwd_off[i] % 256 == 0);
    CHECK(P.fwd_ws_bytes > P.fwd_off[7] && P.bwd_ws_bytes > P.bwd_off[6]);
    CHECK((P.sel_ws_bytes > 0) == (x.L > 1));   // L = 1 selects nothing
    CHECK(P.dense_fwd_ws_bytes > 0 && P.dense_bwd_ws_bytes > 0);
}

void sweep_plans() {
    const int64_t Ns[] = {1, 2, 3, 16, 64, 100, 729, 1000, 1024, 4096, 8192, 65536, 98304, 524288,
                          (int64_t)1 << 20, ((int64_t)1 << 25) - 64, (int64_t)1 << 25, (int64_t)1 << 40};
    const int64_t ds[] = {0, 8, 60, 64, 96, 128, 256};
    const int ps[] = {0, 1, 2, 3, 4, 5, 8};
    const int Ls[] = {0, 1, 2, 3, 4, 6, 8, 9};
    const int ks[] = {-1, 0, 1, 7, 1536, 1 << 20};
    const int dts[] = {0, 1, 7};
    int ok = 0, refused = 0;
    for (int64_t N : Ns)
        for (int64_t d : ds)
            for (int p : ps)
                for (int L : Ls)
                    for (int k : ks)
                        for (int dt : dts) {
                            const lh_desc x = make(1, 2, N, d, p, L, k, dt);
                            lh_plan P;
                            memset(&P, 0xab, sizeof P);
                            const lh_status s = lh_make_plan(&x, &P);
                            if (s == LH_OK) {
                                ++ok;
                                check_plan(x, P);
                            } else {
                                ++refused;
                                CHECK(s == LH_E_ARG || s == LH_E_UNSUPPORTED);
                            }
                        }
    CHECK(ok > 100 && refused > 100);
    // batch and head counts, including products that overflow 32 bits
    const int64_t BHs[][2] = {{0, 1}, {1, 0}, {-1, 1}, {3, 5}, {64, 64}, {1 << 20, 1 << 20}};
    for (const auto& bh : BHs) {
        const lh_desc x = make(bh[0], bh[1], 4096, 64, 4, 3, 64, 1);
        lh_plan P;
        const lh_status s = lh_make_plan(&x, &P);
        if (s == LH_OK) check_plan(x, P);
    }
    CHECK(lh_make_plan(nullptr, nullptr) == LH_E_ARG);
    const lh_desc x = make(1, 1, 64, 64, 2, 2, 1, 1);
    CHECK(lh_make_plan(&x, nullptr) == LH_E_ARG);
}

void refuse_entry_points() {
    const lh_desc x = make(1, 2, 4096, 64, 4, 3, 64, 1);
    lh_plan P;
    CHECK(lh_make_plan(&x, &P) == LH_OK);
    int32_t* gi = static_cast<int32_t*>(fake());
    // null, misaligned and short buffers
    CHECK(lh_pyramid(&x, nullptr, fake(), fake(), fake(), P.pyr_bytes, nullptr) == LH_E_ARG);
    CHECK(lh_pyramid(&x, fake(2), fake(), fake(), fake(), P.pyr_bytes, nullptr) == LH_E_ARG);
    CHECK(lh_pyramid(&x, fake(), fake(), fake(), fake(), P.pyr_bytes - 1, nullptr) == LH_E_WORKSPACE);
    CHECK(lh_score_topk(&x, nullptr, fake(), nullptr, gi, gi, fake(), P.sel_ws_bytes, nullptr) == LH_E_ARG);
    CHECK(lh_score_topk(&x, fake(), fake(), fake(4), gi, gi, fake(), P.sel_ws_bytes, nullptr) == LH_E_ARG);
    CHECK(lh_score_topk(&x, fake(), fake(), nullptr, gi, gi, fake(), P.sel_ws_bytes - 1, nullptr) ==
          LH_E_WORKSPACE);
    CHECK(lh_forward(&x, fake(), fake(), fake(), fake(), gi, gi, nullptr, fake(), P.fwd_ws_bytes, nullptr) ==
          LH_E_ARG);
    CHECK(lh_forward(&x, fake(), fake(), fake(), fake(), gi, gi, fake(), fake(), P.fwd_ws_bytes - 1, nullptr) ==
          LH_E_WORKSPACE);
    CHECK(lh_backward(&x, gi, gi, fake(), fake(), fake(), fake(), nullptr, fake(), P.bwd_ws_bytes, nullptr) ==
          LH_E_ARG);
    CHECK(lh_backward(&x, gi, gi, fake(), fake(), fake(), fake(), fake(), fake(), P.bwd_ws_bytes - 1, nullptr) ==
          LH_E_WORKSPACE);
    CHECK(dense_causal_attn(&x, fake(), fake(), fake(), fake(), static_cast<float*>(fake(4)), fake(),
                            P.dense_fwd_ws_bytes, nullptr) == LH_E_ARG);
    CHECK(dense_causal_attn(&x, fake(), fake(), fake(), fake(), static_cast<float*>(fake()), fake(),
                            P.dense_fwd_ws_bytes - 1, nullptr) == LH_E_WORKSPACE);
    CHECK(dense_causal_attn_backward(&x, fake(), fake(), fake(), static_cast<float*>(fake()), fake(), fake(),
                                     fake(), fake(), fake(), fake(), P.dense_bwd_ws_bytes - 1,
                                     nullptr) == LH_E_WORKSPACE);
    // a descriptor the plan refuses, at every entry point
    const lh_desc bad = make(1, 2, 4095, 64, 4, 3, 64, 1);
    CHECK(lh_pyramid(&bad, fake(), fake(), fake(), fake(), (size_t)1 << 40, nullptr) == LH_E_ARG);
    CHECK(lh_score_topk(&bad, fake(), fake(), nullptr, gi, gi, fake(), (size_t)1 << 40, nullptr) == LH_E_ARG);
    CHECK(lh_score_topk_noalloc(&bad, fake(), fake(), nullptr, gi, gi, nullptr) == LH_E_ARG);
    CHECK(lh_forward(&bad, fake(), fake(), fake(), fake(), gi, gi, fake(), fake(), (size_t)1 << 40, nullptr) ==
          LH_E_ARG);
    CHECK(lh_backward(&bad, gi, gi, fake(), fake(), fake(), fake(), fake(), fake(), (size_t)1 << 40, nullptr) ==
          LH_E_ARG);
    CHECK(lh_pyramid(nullptr, fake(), fake(), fake(), fake(), 0, nullptr) == LH_E_ARG);
    // the allocation-free selection refuses a selection larger than its static array before any device call
    const lh_desc big = make(1, 16, 524288, 64, 4, 6, 1536, 1);
    CHECK(lh_score_topk_noalloc(&big, fake(), fake(), nullptr, gi, gi, nullptr) == LH_E_WORKSPACE);
    CHECK(lh_score_topk_noalloc(&x, fake(2), fake(), nullptr, gi, gi, nullptr) == LH_E_ARG);
    // projections
    size_t ws = 0;
    lh_proj_desc pd = {1, 4096, 1024, 16, 64};
    CHECK(lh_qkv_plan(&pd, &ws) == LH_OK && ws > 0);
    CHECK(lh_qkv_plan(&pd, nullptr) != LH_OK);
    CHECK(lh_qkv_plan(nullptr, &ws) != LH_OK);
    lh_proj_desc bad_pd = {1, 4096, 1000, 16, 64};
    CHECK(lh_qkv_plan(&bad_pd, &ws) != LH_OK);
    CHECK(lh_qkv_forward(&pd, nullptr, fake(), fake(), fake(), fake(), nullptr) != LH_OK);
    CHECK(lh_qkv_backward(&pd, fake(), fake(), fake(), fake(), fake(), fake(), static_cast<float*>(fake()), fake(),
                          0, nullptr) != LH_OK);
    // measurement hooks: bad arguments refused, switching off always allowed
    CHECK(lh_set_probe(LH_KERNEL_COUNT, fake(), fake()) == LH_E_ARG);
    CHECK(lh_set_probe(-2, nullptr, nullptr) == LH_E_ARG);
    CHECK(lh_set_probe(-1, nullptr, nullptr) == LH_OK);
    CHECK(lh_set_probe_flush(nullptr, 0) == LH_OK);
    CHECK(lh_peak_hbm(3, fake(), fake(), 16, nullptr) == LH_E_ARG);
    CHECK(lh_peak_hbm(0, fake(), fake(), 15, nullptr) == LH_E_ARG);
    CHECK(lh_peak_mfma(nullptr, 1, nullptr) == LH_E_ARG);
    for (int s = -3; s < 20; ++s) CHECK(lh_status_string(s) != nullptr && lh_status_string(s)[0] != 0);
}

}  // namespace

int main() {
    sweep_plans();
    refuse_entry_points();
    if (g_failures) {
        fprintf(stderr, "%d checks failed\n", g_failures);
        return 1;
    }
    printf("host sanitizer driver: all checks passed\n");
    return 0;
}
