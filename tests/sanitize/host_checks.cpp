// host_checks.cpp -- the host side of libspecverify (argument checks and
// workspace geometry, sv_host.cpp) under AddressSanitizer and
// UndefinedBehaviorSanitizer, without a GPU: every entry point's checks with
// valid arguments and with each failure its declaration documents, the
// workspace sizes over a grid of shapes (never shrinking as a size grows, no
// overflow at the library limits), and every workspace layout inside the
// bytes the size query returns.  Prints "host ok" and exits 0 when all hold.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>

#include "sv_host.h"

using namespace sv;

static int g_fail = 0;
#define EXPECT(c)                                                          \
    do {                                                                   \
        if (!(c)) {                                                        \
            std::fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #c); \
            ++g_fail;                                                      \
        }                                                                  \
    } while (0)

// Stand-ins for device pointers: only compared with null and tested for
// alignment, never dereferenced.
alignas(256) static unsigned char g_buf[4096];
static const void *const P = g_buf;
static const int32_t *const I = reinterpret_cast<const int32_t *>(g_buf);
static const float *const F = reinterpret_cast<const float *>(g_buf);
static int32_t *const O = reinterpret_cast<int32_t *>(g_buf);
static const uint64_t *const U64 = reinterpret_cast<const uint64_t *>(g_buf);
static const int64_t *const I64 = reinterpret_cast<const int64_t *>(g_buf);

static void greedy_and_tree() {
    bool go = true;
    const size_t need = sv_workspace_bytes_greedy(4, 5, 1000);
    EXPECT(need > 0);
    EXPECT(check_greedy(P, SV_BF16, I, 4, 5, 1000, O, O, P, need, &go) == SV_OK && go);
    EXPECT(check_greedy(P, SV_F32, I, 0, 5, 1000, O, O, P, need, &go) == SV_OK && !go);
    EXPECT(check_greedy(P, 7, I, 4, 5, 1000, O, O, P, need, &go) == SV_ERR_UNSUPPORTED_DTYPE && !go);
    EXPECT(check_greedy(P, SV_BF16, I, -1, 5, 1000, O, O, P, need, &go) == SV_ERR_INVALID_ARG);
    EXPECT(check_greedy(P, SV_BF16, I, 4, -1, 1000, O, O, P, need, &go) == SV_ERR_INVALID_ARG);
    EXPECT(check_greedy(P, SV_BF16, I, 4, 5, 0, O, O, P, need, &go) == SV_ERR_INVALID_ARG);
    EXPECT(check_greedy(P, SV_BF16, I, 4, SV_MAX_GAMMA + 1, 1000, O, O, P, need, &go) == SV_ERR_TOO_LARGE);
    EXPECT(check_greedy(P, SV_BF16, I, 4, 5, SV_MAX_VOCAB + 1, O, O, P, need, &go) == SV_ERR_TOO_LARGE);
    EXPECT(check_greedy(nullptr, SV_BF16, I, 4, 5, 1000, O, O, P, need, &go) == SV_ERR_INVALID_ARG);
    EXPECT(check_greedy(P, SV_BF16, nullptr, 4, 5, 1000, O, O, P, need, &go) == SV_ERR_INVALID_ARG);
    EXPECT(check_greedy(P, SV_BF16, nullptr, 4, 0, 1000, O, O, P, sv_workspace_bytes_greedy(4, 0, 1000), &go) ==
               SV_OK && go);
    EXPECT(check_greedy(P, SV_BF16, I, 4, 5, 1000, nullptr, O, P, need, &go) == SV_ERR_INVALID_ARG);
    EXPECT(check_greedy(P, SV_BF16, I, 4, 5, 1000, O, O, nullptr, need, &go) == SV_ERR_INVALID_ARG);
    EXPECT(check_greedy(g_buf + 1, SV_BF16, I, 4, 5, 1000, O, O, P, need, &go) == SV_ERR_INVALID_ARG);
    EXPECT(check_greedy(g_buf + 2, SV_F32, I, 4, 5, 1000, O, O, P, need, &go) == SV_ERR_INVALID_ARG);
    EXPECT(check_greedy(g_buf + 2, SV_BF16, I, 4, 5, 1000, O, O, P, need, &go) == SV_OK && go);
    EXPECT(check_greedy(P, SV_BF16, I, 4, 5, 1000, O, O, P, 256, &go) == SV_ERR_WORKSPACE_TOO_SMALL && !go);
    // the limits: sizes stay finite and the grid check speaks
    const size_t big = sv_workspace_bytes_greedy(std::numeric_limits<int32_t>::max(), SV_MAX_GAMMA, SV_MAX_VOCAB);
    EXPECT(big > 0);
    const sv_status s = check_greedy(P, SV_BF16, I, std::numeric_limits<int32_t>::max(), SV_MAX_GAMMA, SV_MAX_VOCAB,
                                     O, O, P, big, &go);
    EXPECT(s == SV_ERR_TOO_LARGE || s == SV_OK);

    const size_t nt = sv_workspace_bytes_tree(3, 32, 4099);
    EXPECT(nt > 0);
    EXPECT(check_tree(P, SV_F32, I, I, 3, 32, 4099, O, O, O, P, nt, &go) == SV_OK && go);
    EXPECT(check_tree(P, SV_F32, I, I, 3, 0, 4099, O, O, O, P, nt, &go) == SV_ERR_INVALID_ARG);
    EXPECT(check_tree(P, SV_F32, I, I, 3, SV_MAX_TREE_NODES + 1, 4099, O, O, O, P, nt, &go) == SV_ERR_TOO_LARGE);
    EXPECT(check_tree(P, SV_F32, I, nullptr, 3, 32, 4099, O, O, O, P, nt, &go) == SV_ERR_INVALID_ARG);
    EXPECT(check_tree(P, SV_F32, I, I, 0, 32, 4099, nullptr, nullptr, nullptr, nullptr, 0, &go) == SV_OK && !go);
}

static void sample() {
    bool go = true;
    WorkspaceLayout L;
    int32_t ct, cd, tl, nt;
    for (float top_p : {0.9f, 1.0f}) {
        const size_t need = sv_workspace_bytes_sample(8, 5, 32000, 32000, top_p);
        EXPECT(need > 0);
        EXPECT(check_sample(P, SV_BF16, P, SV_BF16, I, nullptr, F, F, 8, 5, 32000, 32000, 0.8f, top_p, O, O, P, need,
                            &L, &ct, &cd, &tl, &nt, &go) == SV_OK && go);
        EXPECT(check_sample(P, SV_F32, P, SV_F32, I, nullptr, F, F, 8, 5, 32000, 32000, 0.8f, top_p, O, O, P, need,
                            &L, &ct, &cd, &tl, &nt, &go) == SV_OK && go);
        EXPECT(L.counter_bytes <= counter_region(need) && L.data_bytes <= need - counter_region(need));
    }
    const size_t need = sv_workspace_bytes_sample(8, 5, 32000, 16000, 0.9f);
    auto call = [&](const int32_t *d2t, int32_t Vd, float T, float top_p, size_t ws) {
        return check_sample(P, SV_BF16, P, SV_BF16, I, d2t, F, F, 8, 5, 32000, Vd, T, top_p, O, O, P, ws, &L, &ct,
                            &cd, &tl, &nt, &go);
    };
    EXPECT(call(I, 16000, 0.8f, 0.9f, need) == SV_OK);
    EXPECT(call(nullptr, 16000, 0.8f, 0.9f, need) == SV_ERR_INVALID_ARG);      // Vd != Vt needs a map
    EXPECT(call(I, 32001, 0.8f, 0.9f, need) == SV_ERR_INVALID_ARG);          // a map needs Vd <= Vt
    EXPECT(call(I, 16000, 0.0f, 0.9f, need) == SV_ERR_INVALID_ARG);
    EXPECT(call(I, 16000, NAN, 0.9f, need) == SV_ERR_INVALID_ARG);
    EXPECT(call(I, 16000, INFINITY, 0.9f, need) == SV_ERR_INVALID_ARG);
    EXPECT(call(I, 16000, 0.8f, 0.0f, need) == SV_ERR_INVALID_ARG);
    EXPECT(call(I, 16000, 0.8f, NAN, need) == SV_ERR_INVALID_ARG);
    EXPECT(call(I, 16000, 0.8f, 0.9f, 512) == SV_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(check_sample(P, SV_BF16, nullptr, SV_BF16, nullptr, nullptr, nullptr, F, 8, 0, 32000, 32000, 1.0f, 0.9f,
                        O, O, P, sv_workspace_bytes_sample(8, 0, 32000, 32000, 0.9f), &L, &ct, &cd, &tl, &nt,
                        &go) == SV_OK && go);                             // gamma 0: no draft side
    EXPECT(check_sample(P, SV_BF16, nullptr, SV_BF16, I, nullptr, F, F, 8, 3, 32000, 32000, 1.0f, 0.9f, O, O, P,
                        need, &L, &ct, &cd, &tl, &nt, &go) == SV_ERR_INVALID_ARG);
    EXPECT(check_sample(P, 3, P, SV_BF16, I, nullptr, F, F, 8, 5, 32000, 32000, 1.0f, 0.9f, O, O, P, need, &L, &ct,
                        &cd, &tl, &nt, &go) == SV_ERR_UNSUPPORTED_DTYPE);
    // the limits
    for (float top_p : {0.5f, 1.0f}) {
        const size_t big = sv_workspace_bytes_sample(std::numeric_limits<int32_t>::max(), SV_MAX_GAMMA, SV_MAX_VOCAB,
                                                     SV_MAX_VOCAB, top_p);
        EXPECT(big > 0);
    }
}

static void draft_count_fanout() {
    bool go = true;
    DraftLayout L;
    int32_t C;
    const size_t need = sv_workspace_bytes_draft(64, 151936);
    EXPECT(need > 0);
    EXPECT(check_draft(P, SV_BF16, F, 64, 151936, 0.8f, 0.9f, O, P, need, &L, &C, &go) == SV_OK && go);
    EXPECT(C >= 1 && C <= kDraftMaxChunks);
    EXPECT(L.counter_bytes <= counter_region(need) && L.data_bytes <= need - counter_region(need));
    EXPECT(check_draft(P, SV_BF16, F, 64, 151936, -1.0f, 0.9f, O, P, need, &L, &C, &go) == SV_ERR_INVALID_ARG);
    EXPECT(check_draft(P, SV_BF16, F, 64, 0, 0.8f, 0.9f, O, P, need, &L, &C, &go) == SV_ERR_INVALID_ARG);
    EXPECT(check_draft(P, SV_BF16, nullptr, 64, 151936, 0.8f, 0.9f, O, P, need, &L, &C, &go) == SV_ERR_INVALID_ARG);
    EXPECT(check_draft(P, SV_BF16, F, 64, 151936, 0.8f, 0.9f, O, P, 1024, &L, &C, &go) ==
           SV_ERR_WORKSPACE_TOO_SMALL);

    EXPECT(check_count(I, 16, 7, U64, &go) == SV_OK && go);
    EXPECT(check_count(I, 16, 7, reinterpret_cast<const uint64_t *>(g_buf + 4), &go) == SV_ERR_INVALID_ARG);
    EXPECT(check_count(I, 16, SV_MAX_GAMMA + 1, U64, &go) == SV_ERR_TOO_LARGE);
    EXPECT(check_count(nullptr, 0, 7, nullptr, &go) == SV_OK && !go);

    EXPECT(check_fanout(I, I, I, I, 16, 7, 3, 8, O, O, U64, &go) == SV_OK && go);
    EXPECT(check_fanout(I, I, I, nullptr, 16, 7, 3, 8, O, O, U64, &go) == SV_ERR_INVALID_ARG);
    EXPECT(check_fanout(I, I, I, nullptr, 16, 7, 3, 8, O, nullptr, U64, &go) == SV_OK && go);
    EXPECT(check_fanout(I, I, I, I, 16, 7, 0, 8, O, O, U64, &go) == SV_ERR_INVALID_ARG);
    EXPECT(check_fanout(I, I, I, I, 16, 7, SV_MAX_FANOUT + 1, 8, O, O, U64, &go) == SV_ERR_TOO_LARGE);
    EXPECT(check_fanout(I, I, I, I, 16, 7, 3, SV_MAX_BRANCH_DRAFTS + 1, O, O, U64, &go) == SV_ERR_TOO_LARGE);
    EXPECT(check_fanout(I, I, I, I, std::numeric_limits<int32_t>::max(), 7, 3, 8, O, O, nullptr, &go) == SV_OK);
}

static void trim() {
    bool go = true;
    for (int32_t Vt : {1, 2, 7, 8, 77, 1000, 32768, 32769, 128256, 151936, 1 << 20, SV_MAX_VOCAB}) {
        const size_t need = sv_workspace_bytes_vocab_trim(Vt);
        EXPECT(need > 0);
        EXPECT(check_trim(I, 1 << 20, Vt, 0.95f, O, O, I64, P, need, &go) == SV_OK && go);
        // the layout stays inside the workspace
        unsigned char *ws = static_cast<unsigned char *>(std::malloc(need));
        EXPECT(ws != nullptr);
        if (!ws) continue;
        TrimArgs a;
        std::memset(&a, 0, sizeof(a));
        a.Vt = Vt;
        char *base = reinterpret_cast<char *>(ws);
        char *data = base + counter_region(need);
        trim_layout(a, base, data);
        auto inside = [&](const void *p, size_t bytes) {
            const char *c = static_cast<const char *>(p);
            return c >= data && c + bytes <= base + need;
        };
        EXPECT(a.R >= 1 && (a.R & (a.R - 1)) == 0 && a.KB % 8 == 0 && a.KB <= kTrimBins);
        EXPECT((int64_t)a.R * a.KB >= Vt);
        // 16-bit bins, two per word
        EXPECT(inside(a.part, sizeof(uint16_t) * (size_t)a.S * a.R * a.KB));
        EXPECT(reinterpret_cast<char *>(a.part) + sizeof(uint16_t) * (size_t)a.S * a.R * a.KB <=
               reinterpret_cast<char *>(a.counts));
        // the overflow counts sit in the counter region, after the totals and arrival counters
        EXPECT(reinterpret_cast<char *>(a.ovf) >= reinterpret_cast<char *>(a.arrive) + 2 * sizeof(uint32_t));
        EXPECT(reinterpret_cast<char *>(a.ovf) + sizeof(uint32_t) * (size_t)Vt <= base + trim_counter_bytes(Vt));
        EXPECT(base + trim_counter_bytes(Vt) <= data);
        EXPECT(inside(a.counts, sizeof(uint32_t) * (size_t)Vt));
        EXPECT(inside(a.hist_n, sizeof(uint32_t) * kTrimBuckets));
        EXPECT(inside(a.hist_m, sizeof(unsigned long long) * kTrimBuckets));
        EXPECT(inside(a.h2, sizeof(uint32_t) * kTrimFine));
        EXPECT(inside(a.list, sizeof(uint32_t) * kTrimList));
        EXPECT(inside(a.blockdef, sizeof(uint32_t) * (size_t)a.nblocks));
        EXPECT(inside(a.blocktie, sizeof(uint32_t) * (size_t)a.nblocks));
        EXPECT(inside(a.state, sizeof(TrimState)));
        EXPECT(reinterpret_cast<char *>(a.arrive) + 2 * sizeof(uint32_t) <= data);
        std::free(ws);
    }
    const size_t need = sv_workspace_bytes_vocab_trim(1000);
    EXPECT(check_trim(nullptr, 0, 1000, 0.95f, O, O, nullptr, P, need, &go) == SV_OK && go);
    EXPECT(check_trim(nullptr, 5, 1000, 0.95f, O, O, nullptr, P, need, &go) == SV_ERR_INVALID_ARG);
    EXPECT(check_trim(I, 5, 1000, 0.0f, O, O, nullptr, P, need, &go) == SV_ERR_INVALID_ARG);
    EXPECT(check_trim(I, 5, 1000, NAN, O, O, nullptr, P, need, &go) == SV_ERR_INVALID_ARG);
    EXPECT(check_trim(I, (int64_t)INT32_MAX + 1, 1000, 0.95f, O, O, nullptr, P, need, &go) == SV_ERR_TOO_LARGE);
    EXPECT(check_trim(I, 5, 1000, 0.95f, O, O, reinterpret_cast<const int64_t *>(g_buf + 4), P, need, &go) ==
           SV_ERR_INVALID_ARG);
    EXPECT(check_trim(I, 5, 1000, 0.95f, O, O, nullptr, P, 4096, &go) == SV_ERR_WORKSPACE_TOO_SMALL);
}

static void lmhead() {
    bool go = true;
    const size_t need = sv_workspace_bytes_lmhead(128 * 8, 128256);
    EXPECT(need > 0);
    EXPECT(check_lmhead(P, P, I, nullptr, false, 128, 8, 4096, 128256, nullptr, O, O, P, need, &go) == SV_OK && go);
    EXPECT(check_lmhead(P, P, I, I, true, 128, 8, 4096, 128256, O, O, O, P, need, &go) == SV_OK && go);
    EXPECT(check_lmhead(P, P, I, nullptr, false, 128, 8, 4100, 128256, nullptr, O, O, P, need, &go) ==
           SV_ERR_INVALID_ARG);                                             // d % 8 != 0
    EXPECT(check_lmhead(g_buf + 8, P, I, nullptr, false, 128, 8, 4096, 128256, nullptr, O, O, P, need, &go) ==
           SV_ERR_INVALID_ARG);                                             // 16-byte alignment
    EXPECT(check_lmhead(P, P, I, nullptr, false, 128, 0, 4096, 128256, nullptr, O, O, P, need, &go) ==
           SV_ERR_INVALID_ARG);                                             // gamma < 0
    EXPECT(check_lmhead(P, P, I, nullptr, false, 128, SV_MAX_GAMMA + 2, 4096, 128256, nullptr, O, O, P, need, &go) ==
           SV_ERR_TOO_LARGE);
    EXPECT(check_lmhead(P, P, I, I, true, 128, SV_MAX_TREE_NODES + 1, 4096, 128256, O, O, O, P, need, &go) ==
           SV_ERR_TOO_LARGE);
    EXPECT(check_lmhead(P, P, I, nullptr, true, 128, 8, 4096, 128256, O, O, O, P, need, &go) == SV_ERR_INVALID_ARG);
    EXPECT(check_lmhead(P, P, I, nullptr, false, 128, 8, 4096, 128256, nullptr, O, O, P, 1024, &go) ==
           SV_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(check_lmhead(P, P, I, nullptr, false, std::numeric_limits<int32_t>::max(), 8, 4096, 128256, nullptr, O, O,
                        P, need, &go) == SV_ERR_TOO_LARGE);                 // B R past int32
}

// Workspace sizes never shrink as one size grows (a workspace sized for the
// largest call serves the smaller ones): every size query along dense sweeps
// of each argument, the others held at a few values.
template <typename F>
static void sweep(const char *what, int32_t lo, int32_t hi, int32_t step, F &&size_of) {
    size_t prev = 0;
    for (int64_t x = lo; x <= hi; x += step) {
        const size_t n = size_of((int32_t)x);
        if (n < prev) {
            std::fprintf(stderr, "FAIL %s: size %zu at %lld below %zu before\n", what, n, (long long)x, prev);
            ++g_fail;
            return;
        }
        prev = n;
    }
}

static void monotone() {
    const int32_t Vs[] = {1, 9, 777, 4099, 16385, 32000, 49152, 128256, 151936, 1 << 20};
    const int32_t gs[] = {0, 1, 3, 7, 31};
    const int32_t Bs[] = {1, 3, 16, 64, 300};
    for (int32_t V : Vs) {
        for (int32_t g : gs) {
            sweep("greedy/B", 0, 1200, 1, [&](int32_t B) { return sv_workspace_bytes_greedy(B, g, V); });
            sweep("tree/B", 0, 1200, 1, [&](int32_t B) { return sv_workspace_bytes_tree(B, g + 1, V); });
            for (float tp : {0.9f, 1.0f})
                sweep("sample/B", 0, 1200, 1, [&](int32_t B) { return sv_workspace_bytes_sample(B, g, V, V, tp); });
        }
        for (int32_t B : Bs) {
            sweep("greedy/gamma", 0, SV_MAX_GAMMA, 1, [&](int32_t g) { return sv_workspace_bytes_greedy(B, g, V); });
            sweep("tree/N", 1, 600, 1, [&](int32_t N) { return sv_workspace_bytes_tree(B, N, V); });
            for (float tp : {0.9f, 1.0f})
                sweep("sample/gamma", 0, SV_MAX_GAMMA, 1,
                      [&](int32_t g) { return sv_workspace_bytes_sample(B, g, V, V, tp); });
        }
        sweep("draft/B", 0, 3000, 1, [&](int32_t B) { return sv_workspace_bytes_draft(B, V); });
        sweep("lmhead/M", 0, 5000, 7, [&](int32_t M) { return sv_workspace_bytes_lmhead(M, V); });
    }
    for (int32_t B : Bs)
        for (int32_t g : gs) {
            sweep("greedy/V", 1, 400000, 61, [&](int32_t V) { return sv_workspace_bytes_greedy(B, g, V); });
            for (float tp : {0.9f, 1.0f}) {
                sweep("sample/Vt", 1, 400000, 61, [&](int32_t V) { return sv_workspace_bytes_sample(B, g, V, V, tp); });
                sweep("sample/Vd", 1, 160000, 61,
                      [&](int32_t V) { return sv_workspace_bytes_sample(B, g, 160000, V, tp); });
            }
            sweep("draft/V", 1, 400000, 61, [&](int32_t V) { return sv_workspace_bytes_draft(B, V); });
        }
    sweep("trim/Vt", 1, 600000, 97, [&](int32_t Vt) { return sv_workspace_bytes_vocab_trim(Vt); });
    sweep("lmhead/V", 1, 400000, 61, [&](int32_t V) { return sv_workspace_bytes_lmhead(1024, V); });
    EXPECT(sv_workspace_bytes_greedy(-1, 1, 10) == 0 && sv_workspace_bytes_sample(1, 1, 10, 10, 0.0f) == 0 &&
           sv_workspace_bytes_draft(1, 0) == 0 && sv_workspace_bytes_vocab_trim(0) == 0 &&
           sv_workspace_bytes_lmhead(-1, 10) == 0 && sv_workspace_bytes_tree(1, 0, 10) == 0);
    EXPECT(std::strcmp(spec_verify_strerror(SV_OK), "ok") == 0);
    EXPECT(std::strcmp(spec_verify_strerror(static_cast<sv_status>(99)), "unknown status") == 0);
}

int main() {
    greedy_and_tree();
    sample();
    draft_count_fanout();
    trim();
    lmhead();
    monotone();
    if (g_fail) {
        std::fprintf(stderr, "%d check(s) failed\n", g_fail);
        return 1;
    }
    std::printf("host ok\n");
    return 0;
}
