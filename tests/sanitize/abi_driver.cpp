// Calls every entry point of include/deltanet.h with host buffers of exactly
// the sizes its contract states (inputs, outputs and workspace), against the
// host stand-ins of launch_stubs.cpp. Built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_sanitizers.py; exits non-zero on
// the first unexpected status, and the sanitizers abort on any out-of-bounds
// access or undefined behaviour.
#include "deltanet.h"

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

int stub_launch_count();
void stub_set_capturing(bool c);

namespace {

int failures = 0;

// Exactly `bytes` bytes, 16-byte aligned (the redzone starts right after).
struct Buf {
    void *p = nullptr;
    explicit Buf(size_t bytes) {
        if (bytes && posix_memalign(&p, 16, bytes) != 0) p = nullptr;
        if (p) std::memset(p, 0, bytes);
    }
    ~Buf() { std::free(p); }
    Buf(const Buf &) = delete;
    Buf &operator=(const Buf &) = delete;
    template <typename T> T *as() const { return static_cast<T *>(p); }
};

void expect(int got, int want, const char *what) {
    if (got != want) {
        std::fprintf(stderr, "FAIL %s: status %d, expected %d\n", what, got, want);
        ++failures;
    } else {
        std::printf("ok   %s\n", what);
    }
}

void fwd_dense(int B, int H, int T, int dk, int dv, int dtype, int cp, bool s0, bool sf, int gated, int nh = 1) {
    const size_t e = dtype == DN_BF16 ? 2 : 4;
    const size_t real = (size_t)B * T, steps = real * nh;
    Buf q(real * H * dk * e), k(steps * H * dk * e), v(steps * H * dv * e), beta(steps * H * e);
    Buf o(real * H * dv * e), S0(s0 ? (size_t)B * H * dv * dk * 4 : 0), Sf(sf ? (size_t)B * H * dv * dk * 4 : 0);
    Buf g(gated ? real * H * 4 : 0);
    const size_t need = deltanet_workspace_bytes(B, H, T * nh, dk, dv, 64, cp);
    Buf ws(need);
    char what[160];
    std::snprintf(what, sizeof what, "fwd%s B%d H%d T%d nh%d dk%d dv%d %s cp%d ws=%zu", gated ? "(gated)" : "", B, H,
                  T, nh, dk, dv, dtype == DN_BF16 ? "bf16" : "f32", cp, need);
    int st;
    if (nh > 1)
        st = deltanet_gdp_fwd(q.p, k.p, v.p, beta.p, g.as<float>(), S0.as<float>(), o.p, Sf.as<float>(), B, H, T, nh,
                              dk, dv, 64, dtype, cp, ws.p, need, nullptr);
    else if (gated)
        st = deltanet_gated_fwd(q.p, k.p, v.p, beta.p, g.as<float>(), S0.as<float>(), o.p, Sf.as<float>(), B, H, T,
                                dk, dv, 64, dtype, cp, ws.p, need, nullptr);
    else
        st = deltanet_fwd(q.p, k.p, v.p, beta.p, S0.as<float>(), o.p, Sf.as<float>(), B, H, T, dk, dv, 64, dtype, cp,
                          ws.p, need, nullptr);
    expect(st, DN_OK, what);
    if (need > 16) { // one byte short of the contract is refused before any launch
        const int before = stub_launch_count();
        st = deltanet_fwd(q.p, k.p, v.p, beta.p, S0.as<float>(), o.p, Sf.as<float>(), B, H, T * nh, dk, dv, 64,
                          dtype, cp, ws.p, need - 1, nullptr);
        expect(st == DN_ERR_WORKSPACE && stub_launch_count() == before ? 0 : 1, 0, "  short workspace refused");
    }
}

void kda_dense(int B, int H, int T, int dk, int dv, int cp) {
    const size_t n = (size_t)B * T * H;
    Buf q(n * dk * 2), k(n * dk * 2), v(n * dv * 2), beta(n * 2), g(n * dk * 4), o(n * dv * 2);
    Buf S0((size_t)B * H * dv * dk * 4), Sf((size_t)B * H * dv * dk * 4);
    const size_t need = deltanet_workspace_bytes(B, H, T, dk, dv, 64, cp);
    Buf ws(need);
    char what[128];
    std::snprintf(what, sizeof what, "kda B%d H%d T%d dk%d dv%d cp%d ws=%zu", B, H, T, dk, dv, cp, need);
    expect(deltanet_kda_fwd(q.p, k.p, v.p, beta.p, g.as<float>(), S0.as<float>(), o.p, Sf.as<float>(), B, H, T, dk,
                            dv, 64, DN_BF16, cp, ws.p, need, nullptr),
           DN_OK, what);
}

std::vector<int32_t> cu_of(const std::vector<int> &lens) {
    std::vector<int32_t> cu(lens.size() + 1, 0);
    for (size_t i = 0; i < lens.size(); ++i) cu[i + 1] = cu[i] + lens[i];
    return cu;
}

void fwd_varlen(const std::vector<int> &lens, int H, int dk, int dv, int dtype, int mode) {
    const std::vector<int32_t> cuv = cu_of(lens);
    const int N = (int)lens.size(), T = cuv.back();
    const size_t e = dtype == DN_BF16 ? 2 : 4;
    Buf cu((N + 1) * 4), order(N * 4);
    std::memcpy(cu.p, cuv.data(), (N + 1) * 4);
    for (int n = 0; n < N; ++n) order.as<int32_t>()[n] = N - 1 - n;
    Buf q((size_t)T * H * dk * e), k((size_t)T * H * dk * e), v((size_t)T * H * dv * e), beta((size_t)T * H * e);
    Buf o((size_t)T * H * dv * e), S0((size_t)N * H * dv * dk * 4), Sf((size_t)N * H * dv * dk * 4);
    Buf g((size_t)T * H * 4), gk((size_t)T * H * dk * 4);
    char what[128];
    std::snprintf(what, sizeof what, "fwd_varlen mode%d N%d T%d H%d dk%d dv%d", mode, N, T, H, dk, dv);
    int st;
    if (mode == 0)
        st = deltanet_fwd_varlen(q.p, k.p, v.p, beta.p, S0.as<float>(), o.p, Sf.as<float>(), cu.as<int32_t>(),
                                 order.as<int32_t>(), N, T, H, dk, dv, 64, dtype, nullptr);
    else if (mode == 1)
        st = deltanet_gated_fwd_varlen(q.p, k.p, v.p, beta.p, g.as<float>(), S0.as<float>(), o.p, Sf.as<float>(),
                                       cu.as<int32_t>(), nullptr, N, T, H, dk, dv, 64, dtype, nullptr);
    else
        st = deltanet_kda_fwd_varlen(q.p, k.p, v.p, beta.p, gk.as<float>(), S0.as<float>(), o.p, Sf.as<float>(),
                                     cu.as<int32_t>(), order.as<int32_t>(), N, T, H, dk, dv, 64, DN_BF16, nullptr);
    expect(st, DN_OK, what);
}

// mode 0 DeltaNet, 1 gated, 2 GDP (nh substeps), 3 DeltaNet and 4 gated with
// context parallelism (nh: the group count, 0 automatic)
void bwd_dense(int B, int H, int T, int dk, int dv, int mode, int nh = 1) {
    const size_t real = (size_t)B * T, steps = mode >= 3 ? real : real * nh;
    Buf q(real * H * dk * 2), k(steps * H * dk * 2), v(steps * H * dv * 2), beta(steps * H * 2), dO(real * H * dv * 2);
    Buf dq(real * H * dk * 2), dk_(steps * H * dk * 2), dv_(steps * H * dv * 2), db(steps * H * 2);
    Buf g(real * H * 4), dg(real * H * 4);
    Buf S0((size_t)B * H * dv * dk * 4), dSf((size_t)B * H * dv * dk * 4), dS0((size_t)B * H * dv * dk * 4);
    size_t need;
    int st;
    if (mode == 0) {
        need = deltanet_bwd_workspace_bytes(B, H, T, dk, dv, 64);
        Buf ws(need);
        st = deltanet_bwd(q.p, k.p, v.p, beta.p, S0.as<float>(), dO.p, dSf.as<float>(), dq.p, dk_.p, dv_.p, db.p,
                          dS0.as<float>(), B, H, T, dk, dv, 64, DN_BF16, ws.p, need, nullptr);
    } else if (mode == 1) {
        need = deltanet_gated_bwd_workspace_bytes(B, H, T, dk, dv, 64);
        Buf ws(need);
        st = deltanet_gated_bwd(q.p, k.p, v.p, beta.p, g.as<float>(), S0.as<float>(), dO.p, dSf.as<float>(), dq.p,
                                dk_.p, dv_.p, db.p, dg.as<float>(), dS0.as<float>(), B, H, T, dk, dv, 64, DN_BF16,
                                ws.p, need, nullptr);
    } else if (mode == 4) {
        need = deltanet_gated_bwd_cp_workspace_bytes(B, H, T, dk, dv, 64, nh);
        Buf ws(need);
        st = deltanet_gated_bwd_cp(q.p, k.p, v.p, beta.p, g.as<float>(), S0.as<float>(), dO.p, dSf.as<float>(), dq.p,
                                   dk_.p, dv_.p, db.p, dg.as<float>(), dS0.as<float>(), B, H, T, dk, dv, 64, DN_BF16, nh,
                                   ws.p, need, nullptr);
    } else if (mode == 3) {
        need = deltanet_bwd_cp_workspace_bytes(B, H, T, dk, dv, 64, nh);
        Buf ws(need);
        st = deltanet_bwd_cp(q.p, k.p, v.p, beta.p, S0.as<float>(), dO.p, dSf.as<float>(), dq.p, dk_.p, dv_.p, db.p,
                             dS0.as<float>(), B, H, T, dk, dv, 64, DN_BF16, nh, ws.p, need, nullptr);
    } else {
        need = deltanet_gdp_bwd_workspace_bytes(B, H, T, nh, dk, dv, 64);
        Buf ws(need);
        st = deltanet_gdp_bwd(q.p, k.p, v.p, beta.p, g.as<float>(), nullptr, dO.p, nullptr, dq.p, dk_.p, dv_.p, db.p,
                              dg.as<float>(), dS0.as<float>(), B, H, T, nh, dk, dv, 64, DN_BF16, ws.p, need, nullptr);
    }
    char what[128];
    std::snprintf(what, sizeof what, "bwd mode%d B%d H%d T%d nh%d dk%d dv%d ws=%zu", mode, B, H, T, nh, dk, dv, need);
    expect(st, DN_OK, what);
}

void bwd_varlen(const std::vector<int> &lens, int H, int dk, int dv, bool gated) {
    const std::vector<int32_t> cuv = cu_of(lens);
    const int N = (int)lens.size(), T = cuv.back();
    Buf cu((N + 1) * 4);
    std::memcpy(cu.p, cuv.data(), (N + 1) * 4);
    const size_t n = (size_t)T * H;
    Buf q(n * dk * 2), k(n * dk * 2), v(n * dv * 2), beta(n * 2), dO(n * dv * 2);
    Buf dq(n * dk * 2), dk_(n * dk * 2), dv_(n * dv * 2), db(n * 2), g(n * 4), dg(n * 4);
    Buf S0((size_t)N * H * dv * dk * 4), dSf((size_t)N * H * dv * dk * 4), dS0((size_t)N * H * dv * dk * 4);
    const size_t need = gated ? deltanet_gated_bwd_varlen_workspace_bytes(N, T, H, dk, dv, 64)
                              : deltanet_bwd_varlen_workspace_bytes(N, T, H, dk, dv, 64);
    Buf ws(need);
    int st;
    if (gated)
        st = deltanet_gated_bwd_varlen(q.p, k.p, v.p, beta.p, g.as<float>(), S0.as<float>(), dO.p, dSf.as<float>(),
                                       dq.p, dk_.p, dv_.p, db.p, dg.as<float>(), dS0.as<float>(), cu.as<int32_t>(),
                                       nullptr, N, T, H, dk, dv, 64, DN_BF16, ws.p, need, nullptr);
    else
        st = deltanet_bwd_varlen(q.p, k.p, v.p, beta.p, S0.as<float>(), dO.p, dSf.as<float>(), dq.p, dk_.p, dv_.p,
                                 db.p, dS0.as<float>(), cu.as<int32_t>(), nullptr, N, T, H, dk, dv, 64, DN_BF16, ws.p,
                                 need, nullptr);
    char what[128];
    std::snprintf(what, sizeof what, "bwd_varlen%s N%d T%d H%d dk%d dv%d ws=%zu", gated ? "(gated)" : "", N, T, H, dk,
                  dv, need);
    expect(st, DN_OK, what);
}

void decode(int B, int H, int dk, int dv, int dtype, int mode) {
    const size_t e = dtype == DN_BF16 ? 2 : 4, n = (size_t)B * H;
    Buf q(n * dk * e), k(n * dk * e), v(n * dv * e), beta(n * e), o(n * dv * e), S(n * dv * dk * 4);
    Buf g(n * 4), gk(n * dk * 4);
    char what[96];
    std::snprintf(what, sizeof what, "decode mode%d B%d H%d dk%d dv%d", mode, B, H, dk, dv);
    int st;
    if (mode == 2)
        st = deltanet_kda_decode_step(q.p, k.p, v.p, beta.p, gk.as<float>(), S.as<float>(), o.p, B, H, dk, dv, dtype,
                                      nullptr);
    else
        st = deltanet_decode_step(q.p, k.p, v.p, beta.p, mode ? g.as<float>() : nullptr, S.as<float>(), o.p, B, H, dk,
                                  dv, dtype, nullptr);
    expect(st, DN_OK, what);
}

void rejected() {
    Buf a(1 << 16);
    const int before = stub_launch_count();
    expect(deltanet_fwd(a.p, a.p, a.p, a.p, nullptr, a.p, nullptr, 1, 1, 64, 96, 64, 64, DN_BF16, 1, nullptr, 0,
                        nullptr),
           DN_ERR_UNSUPPORTED, "dk = 96 refused");
    expect(deltanet_fwd(a.p, a.p, a.p, a.p, nullptr, a.p, nullptr, 1, 1, 64, 64, 64, 32, DN_BF16, 1, nullptr, 0,
                        nullptr),
           DN_ERR_UNSUPPORTED, "chunk = 32 refused");
    expect(deltanet_fwd(a.p, a.p, a.p, a.p, nullptr, a.p, nullptr, 0, 1, 64, 64, 64, 64, DN_BF16, 1, nullptr, 0,
                        nullptr),
           DN_ERR_INVALID, "B = 0 refused");
    expect(deltanet_fwd(a.as<char>() + 2, a.p, a.p, a.p, nullptr, a.p, nullptr, 1, 1, 64, 64, 64, 64, DN_BF16, 1,
                        nullptr, 0, nullptr),
           DN_ERR_INVALID, "misaligned q refused");
    expect(deltanet_fwd(a.p, a.p, a.p, a.p, nullptr, a.p, nullptr, 1, 1, 640, 64, 64, 64, DN_BF16, 4, nullptr, 0,
                        nullptr),
           DN_ERR_WORKSPACE, "missing workspace refused");
    expect(deltanet_bwd(a.p, a.p, a.p, a.p, nullptr, a.p, nullptr, a.p, a.p, a.p, a.p, nullptr, 1, 1, 64, 64, 64, 64,
                        DN_F32, a.p, 1 << 16, nullptr),
           DN_ERR_UNSUPPORTED, "fp32 backward refused");
    expect(stub_launch_count() == before ? 0 : 1, 0, "refused calls launched nothing");
    expect(std::strcmp(deltanet_status_string(12345), "unknown status") == 0 ? 0 : 1, 0, "status string");
}

} // namespace

int main() {
    // dk = dv = 128: group 0 ahead of the transitions, on two streams and (as
    // under capture) on one; 18 chunks give group 0 fewer chunks than the
    // later groups for 3 and 4 groups, and an even split for 9
    for (bool cap : {false, true}) {
        stub_set_capturing(cap);
        for (int cp : {3, 4, 9}) fwd_dense(1, 2, 17 * 64 + 5, 128, 128, DN_BF16, cp, true, true, 0);
        fwd_dense(1, 2, 17 * 64 + 5, 128, 128, DN_BF16, 4, false, true, 1);
        fwd_dense(1, 2, 17 * 64 + 5, 128, 128, DN_BF16, 3, true, false, 1, 2);
    }
    stub_set_capturing(false);
    for (int dtype : {DN_BF16, DN_F32}) {
        const int dk = 64;
        for (int cp : {1, 0, 2, 3, 7}) fwd_dense(2, 3, 7 * 64 + 20, dk, 128, dtype, cp, true, true, 0);
        fwd_dense(1, 2, 0, dk, 64, dtype, 1, true, true, 0);
        fwd_dense(1, 2, 1, dk, 64, dtype, 2, false, false, 0);
        fwd_varlen({0, 1, 63, 64, 65, 300}, 3, dk, 64, dtype, 0);
        fwd_varlen({70, 5, 128}, 2, dk, 128, dtype, 1);
    }
    for (int dk : {64, 128})
        for (int dv : {64, 128}) {
            fwd_dense(1, 2, 5 * 64 + 1, dk, dv, DN_BF16, 3, true, true, 1);
            fwd_dense(2, 1, 150, dk, dv, DN_BF16, 2, false, true, 1, 2);
            kda_dense(1, 2, 6 * 64 + 5, dk, dv, 1);
            kda_dense(1, 2, 6 * 64 + 5, dk, dv, 3);
            kda_dense(1, 2, 0, dk, dv, 1);
            fwd_varlen({0, 33, 129}, 2, dk, dv, DN_BF16, 2);
            bwd_dense(2, 2, 200, dk, dv, 0);
            bwd_dense(1, 3, 130, dk, dv, 1);
            bwd_dense(1, 2, 70, dk, dv, 2, 3);
            bwd_dense(1, 2, 0, dk, dv, 0);
            bwd_dense(2, 3, 700, dk, dv, 3, 4);
            bwd_dense(1, 2, 1100, dk, dv, 3, 0);
            bwd_dense(2, 3, 700, dk, dv, 4, 4);
            bwd_varlen({0, 1, 64, 65, 190}, 2, dk, dv, false);
            bwd_varlen({3, 128, 77}, 2, dk, dv, true);
            for (int mode = 0; mode < 3; ++mode) decode(3, 2, dk, dv, DN_BF16, mode);
            decode(2, 2, dk, dv, DN_F32, 1);
        }
    rejected();
    std::printf("%d launches, %d failures\n", stub_launch_count(), failures);
    return failures ? 1 : 0;
}
