// Host-only run of the C ABI layer (combine_moe_layout_02_amd/csrc/moe_api.cpp) built with the
// address and undefined-behaviour sanitizers against the stand-in launchers of abi_stubs.cpp:
// the size arithmetic at the largest accepted sizes and at hostile int64 arguments, a rejected
// call for every entry point, and which launchers a valid call reaches (for example that
// moe_layout_dispatch takes the one-kernel path only for small tables, and each moe_layout_path
// value reaches its launcher). Pointers are fake device
// addresses that nothing dereferences. Prints "abi_asan ok" and returns 0 when every check holds.
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "abi_stubs.h"
#include "moe.h"

static int failures = 0;

static void expect(bool cond, const char *what) {
    if (!cond) {
        std::printf("FAIL: %s\n", what);
        ++failures;
    }
}

static bool only(stubs::Launcher a, int na, stubs::Launcher b = stubs::kLaunchers, int nb = 0) {
    for (int i = 0; i < stubs::kLaunchers; ++i) {
        const int want = i == a ? na : (i == b ? nb : 0);
        if (stubs::calls[i] != want) return false;
    }
    return true;
}

int main() {
    char *base = reinterpret_cast<char *>(uintptr_t{1} << 20);  // 512-byte aligned, never touched
    void *A = base;
    int32_t *I = reinterpret_cast<int32_t *>(base);
    uint8_t *U = reinterpret_cast<uint8_t *>(base);
    float *F = reinterpret_cast<float *>(base);
    const int64_t big = INT64_MAX;

    // host functions at the limits
    expect(moe_slot_bytes(7168) == 14848, "slot bytes at H=7168");
    expect(moe_window_bytes(MOE_MAX_TOKENS, MOE_MAX_K, MOE_MAX_HIDDEN) ==
               (int64_t)MOE_MAX_TOKENS * MOE_MAX_K * 33280,
           "window bytes at the largest sizes");
    expect(moe_window_bytes(MOE_MAX_TOKENS + 1, 1, 16) == MOE_ERR_UNSUPPORTED, "S above the limit");
    expect(moe_dedup_window_bytes(MOE_MAX_TOKENS, MOE_MAX_K, MOE_MAX_RANKS, MOE_MAX_HIDDEN) ==
               (int64_t)MOE_MAX_TOKENS * MOE_MAX_K * 33280,
           "dedup window bytes at the largest sizes");
    expect(moe_slot_offsets(MOE_MAX_HIDDEN, MOE_QUANT_FP8_E4M3_DYN, nullptr, nullptr, nullptr, nullptr) ==
               MOE_OK,
           "slot offsets with no outputs");
    for (int st = -6; st <= 1; ++st) expect(moe_status_string(st) != nullptr, "status string");

    // rejected calls: hostile sizes and int64 extremes
    stubs::reset();
    expect(moe_layout(I, 64, 8, 256, 8, 65, U, I, I, I, I, I, I, I, I, nullptr) == MOE_ERR_ARG, "layout C > S");
    expect(moe_dispatch(A, I, 64, 7168, 8, 0, 0, A, -1, nullptr) == MOE_ERR_WINDOW, "dispatch negative window");
    expect(moe_layout_dispatch(I, 64, 8, 256, 8, 16, U, I, I, I, I, I, I, I, I, A, 7168, 1, 0, A, 0, nullptr) ==
               MOE_ERR_WINDOW,
           "layout_dispatch empty window");
    expect(moe_combine(A, big - 15, 1 << 20, I, F, 64, 7168, 8, A, nullptr) == MOE_ERR_ARG,
           "combine row extent beyond int64");
    expect(moe_combine(A, 14336, -1, I, F, 64, 7168, 8, A, nullptr) == MOE_ERR_ARG, "combine negative rows");
    expect(moe_combine_scatter(A, 14336, 512, I, I, 64, 8, 7168, A, big - 15, big, nullptr) == MOE_ERR_WINDOW,
           "scatter huge staging stride");
    expect(moe_combine_scatter(A, big - 15, 512, I, I, 64, 8, 7168, A, 14336, big, nullptr) == MOE_ERR_ARG,
           "scatter row extent beyond int64");
    expect(moe_combine_scatter(A, 14336, 512, I, I, 64, 8, 7168, A, 14336, -5, nullptr) == MOE_ERR_WINDOW,
           "scatter negative staging bytes");
    expect(moe_combine_staged(A, 100, big, I, F, 64, 7168, 8, A, nullptr) == MOE_ERR_ARG, "staged short stride");
    expect(moe_combine_staged(A, big - 15, big, I, F, 64, 7168, 8, A, nullptr) == MOE_ERR_WINDOW,
           "staged huge staging stride");
    expect(moe_combine_staged(A, 14336, -5, I, F, 64, 7168, 8, A, nullptr) == MOE_ERR_WINDOW,
           "staged negative staging bytes");
    expect(moe_layout_ex(I, 64, 8, 256, 8, 16, U, I, I, I, I, I, I, I, I, 3, nullptr) == MOE_ERR_ARG,
           "layout_ex unknown path");
    expect(moe_layout_ex(I, 513, 8, 256, 8, 16, U, I, I, I, I, I, I, I, I, MOE_LAYOUT_SINGLE, nullptr) ==
               MOE_ERR_UNSUPPORTED,
           "layout_ex single launch at S*K = 4104");
    expect(moe_layout_ex(I, 2048, 2, 16, 4, 1025, U, I, I, I, I, I, I, I, I, MOE_LAYOUT_SINGLE, nullptr) ==
               MOE_ERR_UNSUPPORTED,
           "layout_ex single launch with C above 1024");
    expect(moe_layout_dispatch_ex(I, 513, 8, 256, 8, 16, U, I, I, I, I, I, I, I, I, A, 7168, 0, 0, A,
                                  moe_window_bytes(513, 8, 7168), MOE_LAYOUT_SINGLE, nullptr) == MOE_ERR_UNSUPPORTED,
           "layout_dispatch_ex single launch at S*K = 4104");
    expect(moe_layout_dispatch_ex(I, 64, 8, 256, 8, 16, U, I, I, I, I, I, I, I, I, A, 7168, 0, 0, A,
                                  moe_window_bytes(64, 8, 7168), -1, nullptr) == MOE_ERR_ARG,
           "layout_dispatch_ex negative path");
    expect(moe_unpack(A, big, I, 64, 8, 7168, 1, A, nullptr, I, nullptr) == MOE_ERR_ARG, "unpack fp8 without scales");
    expect(moe_unpack_padded(A, big, I, 256, 64, 8, 7168, 0, 16, big, A, nullptr, I, I, I, nullptr) == MOE_ERR_ARG,
           "unpack_padded out_rows beyond the limit");
    expect(moe_rank_rows(I, 64, 8, 250, 8, 16, I, I, I, I, nullptr) == MOE_ERR_UNSUPPORTED, "rank rows E % P");
    expect(moe_dispatch_dedup(A, I, I, 64, 7168, 8, 256, 8, 0, 0, A, 1, nullptr) == MOE_ERR_WINDOW,
           "dedup small window");
    expect(moe_expand_dedup(A, big, I, I, I, 64, 8, 0, 7168, 0, A, nullptr, I, nullptr) == MOE_ERR_ARG,
           "expand P = 0");
    {
        const int64_t wsb = moe_dispatch_workspace_bytes(4096, 8, 0);
        const int64_t wbig = moe_window_bytes(4096, 8, 7168);
        expect(wsb == 8LL * 4 * 128 * 8 * 8, "dispatch workspace bytes at S=4096, K=8");
        expect(moe_dispatch_workspace_bytes(MOE_MAX_TOKENS, MOE_MAX_K, 0) == 8LL * 128 * 64 * 16 * 8,
               "dispatch workspace bytes at the largest sizes");
        expect(moe_dispatch_ws(A, I, 4096, 7168, 8, 0, 0, A, wbig, nullptr, wsb, nullptr) == MOE_ERR_ARG,
               "dispatch_ws without a workspace");
        expect(moe_dispatch_ws(A, I, 4096, 7168, 8, 0, 0, A, wbig, A, wsb - 1, nullptr) == MOE_ERR_WINDOW,
               "dispatch_ws one workspace byte short");
        expect(moe_dispatch_ws(A, I, 4096, 7168, 8, 0, 0, A, wbig, base + 8, wsb, nullptr) == MOE_ERR_ALIGN,
               "dispatch_ws misaligned workspace");
        expect(moe_dispatch_ws(A, I, 4096, 7168, 8, 0, 0, A, wbig, A, -big, nullptr) == MOE_ERR_WINDOW,
               "dispatch_ws negative workspace bytes");
    }
    expect(only(stubs::kLaunchers, 0), "no launcher reached by a rejected call");

    // valid calls and the launchers they reach
    const int64_t win = moe_window_bytes(512, 8, 7168);
    stubs::reset();
    expect(moe_layout(I, 64, 8, 256, 8, 16, U, I, I, I, I, I, I, I, I, nullptr) == MOE_OK &&
               only(stubs::kLayoutSmall, 1),
           "layout at S*K = 512 -> the single launch");
    stubs::reset();
    expect(moe_layout(I, 513, 8, 256, 8, 16, U, I, I, I, I, I, I, I, I, nullptr) == MOE_OK &&
               only(stubs::kLayout, 1),
           "layout at S*K = 4104 -> the multi-launch form");
    stubs::reset();
    expect(moe_layout(I, 2048, 2, 16, 4, 1025, U, I, I, I, I, I, I, I, I, nullptr) == MOE_OK &&
               only(stubs::kLayout, 1),
           "layout with C above 1024 -> the multi-launch form");
    stubs::reset();
    expect(moe_layout_ex(I, 64, 8, 256, 8, 16, U, I, I, I, I, I, I, I, I, MOE_LAYOUT_AUTO, nullptr) == MOE_OK &&
               only(stubs::kLayoutSmall, 1),
           "layout_ex auto at S*K = 512 -> the single launch");
    stubs::reset();
    expect(moe_layout_ex(I, 64, 8, 256, 8, 16, U, I, I, I, I, I, I, I, I, MOE_LAYOUT_MULTI, nullptr) == MOE_OK &&
               only(stubs::kLayout, 1),
           "layout_ex multi at S*K = 512 -> the multi-launch form");
    stubs::reset();
    expect(moe_layout_ex(I, 512, 8, 256, 8, 128, U, I, I, I, I, I, I, I, I, MOE_LAYOUT_SINGLE, nullptr) ==
                   MOE_OK &&
               only(stubs::kLayoutSmall, 1),
           "layout_ex single at S*K = 4096 -> the single launch");
    stubs::reset();
    expect(moe_layout_ex(I, 513, 8, 256, 8, 16, U, I, I, I, I, I, I, I, I, MOE_LAYOUT_AUTO, nullptr) == MOE_OK &&
               only(stubs::kLayout, 1),
           "layout_ex auto at S*K = 4104 -> the multi-launch form");
    stubs::reset();
    expect(moe_layout_dispatch(I, 512, 8, 256, 8, 128, U, I, I, I, I, I, I, I, I, A, 7168, 0, 0, A, win,
                               nullptr) == MOE_OK &&
               only(stubs::kLayoutDispatchSmall, 1),
           "layout_dispatch at S*K = 4096 -> one kernel");
    stubs::reset();
    expect(moe_layout_dispatch(I, 513, 8, 256, 8, 128, U, I, I, I, I, I, I, I, I, A, 7168, 1, 0, A,
                               moe_window_bytes(513, 8, 7168), nullptr) == MOE_OK &&
               only(stubs::kLayout, 1, stubs::kPack, 1),
           "layout_dispatch at S*K = 4104 -> layout + pack");
    stubs::reset();
    expect(moe_layout_dispatch(I, 64, 8, 256, 8, 64, U, I, I, I, I, I, I, I, I, A, 7168, 2, 0, A, win, nullptr) ==
                   MOE_OK &&
               only(stubs::kLayoutDispatchSmall, 1),
           "layout_dispatch small, int8");
    stubs::reset();
    expect(moe_layout_dispatch(I, 2048, 2, 16, 4, 1025, U, I, I, I, I, I, I, I, I, A, 16, 0, 0, A,
                               moe_window_bytes(2048, 2, 16), nullptr) == MOE_OK &&
               only(stubs::kLayout, 1, stubs::kPack, 1),
           "layout_dispatch with C above 1024 -> layout + pack");
    stubs::reset();
    expect(moe_layout_dispatch_ex(I, 64, 8, 256, 8, 16, U, I, I, I, I, I, I, I, I, A, 7168, 0, 0, A, win,
                                  MOE_LAYOUT_MULTI, nullptr) == MOE_OK &&
               only(stubs::kLayout, 1, stubs::kPack, 1),
           "layout_dispatch_ex multi at S*K = 512 -> layout + pack");
    stubs::reset();
    expect(moe_layout_dispatch_ex(I, 64, 8, 256, 8, 16, U, I, I, I, I, I, I, I, I, A, 7168, 1, 0, A, win,
                                  MOE_LAYOUT_SINGLE, nullptr) == MOE_OK &&
               only(stubs::kLayoutDispatchSmall, 1),
           "layout_dispatch_ex single at S*K = 512 -> one kernel");
    stubs::reset();
    expect(moe_layout_dispatch_ex(I, 64, 8, 256, 8, 16, U, I, I, I, I, I, I, I, I, A, 7168, 2, 0, A, win,
                                  MOE_LAYOUT_AUTO, nullptr) == MOE_OK &&
               only(stubs::kLayoutDispatchSmall, 1),
           "layout_dispatch_ex auto at S*K = 512 -> one kernel");
    stubs::reset();
    expect(moe_dispatch(A, I, 64, 7168, 8, 1, 3, A, win, nullptr) == MOE_OK && only(stubs::kPack, 1),
           "dispatch -> launch_pack");
    {
        const int64_t wbig = moe_window_bytes(4096, 8, 7168);
        const int64_t wsb = moe_dispatch_workspace_bytes(4096, 8, 0);
        stubs::reset();
        expect(moe_dispatch_ws(A, I, 4096, 7168, 8, 0, 0, A, wbig, A, wsb, nullptr) == MOE_OK &&
                   only(stubs::kPackPlanned, 1),
               "dispatch_ws bf16 at S*K = 32768 -> planned pack");
        stubs::reset();
        expect(moe_dispatch_ws(A, I, 1024, 7168, 8, 0, 0, A, moe_window_bytes(1024, 8, 7168), A,
                               moe_dispatch_workspace_bytes(1024, 8, 0), nullptr) == MOE_OK &&
                   only(stubs::kPackPlanned, 1),
               "dispatch_ws bf16 at S*K = 8192 -> planned pack");
        stubs::reset();
        expect(moe_dispatch_ws(A, I, 1023, 7168, 8, 0, 0, A, moe_window_bytes(1023, 8, 7168), nullptr, 0,
                               nullptr) == MOE_OK &&
                   only(stubs::kPack, 1),
               "dispatch_ws bf16 at S*K = 8184 -> token-order pack, no workspace needed");
        stubs::reset();
        expect(moe_dispatch_ws(A, I, 4096, 7168, 8, 1, 0, A, wbig, nullptr, 0, nullptr) == MOE_OK &&
                   only(stubs::kPack, 1),
               "dispatch_ws fp8 -> token-order quantised pack, no workspace needed");
    }
    {
        // moe_layout_dispatch_ws: every part of the workspace inside it, 256-byte aligned, apart and
        // as large as its kernel writes; the plan first, where moe_dispatch_planned finds it.
        struct Case {
            int S, K, E, P, C, quant;
            stubs::Launcher launcher;
            const char *what;
        };
        const Case cases[] = {
            {4096, 8, 256, 8, 128, 0, stubs::kPackFromPlan, "layout_dispatch_ws bf16, 256 entries a channel -> plan by the layout"},
            {8192, 8, 256, 128, 128, 0, stubs::kPackFromPlan, "layout_dispatch_ws bf16, 512 entries a channel"},
            {4096, 8, 256, 8, 16, 0, stubs::kPackPlanned, "layout_dispatch_ws bf16, 2048 entries a channel -> plan kernel"},
            {4096, 8, 256, 8, 1, 0, stubs::kPackPlanned, "layout_dispatch_ws bf16, one channel"},
            {65536, 16, 512, 256, 4096, 0, stubs::kPackFromPlan, "layout_dispatch_ws at the maxima"},
            {65536, 16, 384, 384, 1, 0, stubs::kPackPlanned, "layout_dispatch_ws at the maxima, one channel"},
            {4096, 8, 256, 8, 128, 1, stubs::kPack, "layout_dispatch_ws fp8 -> token-order pack"},
            {1000, 8, 64, 8, 128, 0, stubs::kPack, "layout_dispatch_ws bf16 below 8192 entries -> token-order pack"},
        };
        for (const Case &c : cases) {
            const int64_t wsb = moe_layout_dispatch_workspace_bytes(c.S, c.K, c.E, c.P, c.C, c.quant, 0);
            const int64_t wb = moe_window_bytes(c.S, c.K, 64);
            const uintptr_t ws = 0x40000000;
            void *wsp = reinterpret_cast<void *>(ws);
            stubs::reset();
            const int st = moe_layout_dispatch_ws(I, c.S, c.K, c.E, c.P, c.C, U, I, I, I, I, I, I, I, I, A, 64,
                                                  c.quant, 0, A, wb, MOE_LAYOUT_AUTO, wsp, wsb, nullptr);
            bool ok = st == MOE_OK && only(stubs::kLayoutWs, 1, c.launcher, 1);
            const moe::LayoutWorkspace w = stubs::last_ws;
            const void *plan = stubs::last_plan;
            const moe::PackChunks pc = stubs::last_chunks;
            auto at = [&](const void *p) { return (int64_t)(reinterpret_cast<uintptr_t>(p) - ws); };
            const int64_t o_col = at(w.colexcl), o_bucket = at(w.bucket), o_chan = at(w.chan);
            int64_t plan_end = 0;
            if (c.launcher == stubs::kPackFromPlan) {
                plan_end = 64LL * pc.nsx * pc.cap;
                ok = ok && w.plan != nullptr && at(w.plan) == 0 && plan == w.plan && 8LL * pc.nsx >= pc.nsub &&
                     (int64_t)pc.cpc * ((c.S + c.C - 1) / c.C) * c.K <= pc.cap &&
                     (1 << pc.lt) >= pc.cpc * ((c.S + c.C - 1) / c.C);
            } else if (c.launcher == stubs::kPackPlanned) {
                plan_end = moe_dispatch_workspace_bytes(c.S, c.K, 0);
                ok = ok && w.plan == nullptr && at(plan) == 0;
            } else {
                ok = ok && w.plan == nullptr;
            }
            ok = ok && o_col >= plan_end && o_col % 256 == 0 && o_bucket >= o_col + (int64_t)c.E * c.C * 4 &&
                 o_bucket % 256 == 0 && o_chan >= o_bucket + (int64_t)c.S * c.K * 4 && o_chan % 256 == 0 &&
                 o_chan + 2LL * c.C * 4 <= wsb;
            expect(ok, c.what);
            expect(moe_layout_dispatch_ws(I, c.S, c.K, c.E, c.P, c.C, U, I, I, I, I, I, I, I, I, A, 64, c.quant, 0, A,
                                          wb, MOE_LAYOUT_AUTO, wsp, wsb - 1, nullptr) == MOE_ERR_WINDOW,
                   "layout_dispatch_ws one workspace byte short");
            // the same work as two calls: the layout, then the pack from the plan it left
            stubs::reset();
            ok = moe_layout_ws(I, c.S, c.K, c.E, c.P, c.C, U, I, I, I, I, I, I, I, I, c.quant, 0, wsp, wsb, nullptr) ==
                     MOE_OK &&
                 only(stubs::kLayoutWs, 1) && (stubs::last_ws.plan == nullptr) == (c.launcher != stubs::kPackFromPlan);
            expect(ok, "layout_ws alone");
            stubs::reset();
            ok = moe_dispatch_planned(A, I, c.S, 64, c.K, c.C, c.quant, 0, A, wb, wsp, plan_end, nullptr) == MOE_OK &&
                 only(c.launcher, 1) && (c.launcher == stubs::kPack || stubs::last_plan == wsp);
            expect(ok, "dispatch_planned with exactly the plan's bytes");
            if (plan_end > 0)
                expect(moe_dispatch_planned(A, I, c.S, 64, c.K, c.C, c.quant, 0, A, wb, wsp, plan_end - 1, nullptr) ==
                           MOE_ERR_WINDOW,
                       "dispatch_planned one plan byte short");
        }
        stubs::reset();
        expect(moe_layout_dispatch_workspace_bytes(64, 8, 256, 8, 16, 0, MOE_LAYOUT_AUTO) == 0 &&
                   moe_layout_dispatch_ws(I, 64, 8, 256, 8, 16, U, I, I, I, I, I, I, I, I, A, 7168, 0, 0, A, win,
                                          MOE_LAYOUT_AUTO, nullptr, 0, nullptr) == MOE_OK &&
                   only(stubs::kLayoutDispatchSmall, 1),
               "layout_dispatch_ws on a small table -> one kernel, no workspace");
    }
    stubs::reset();
    expect(moe_combine(A, 14848, 512, I, F, 64, 7168, 8, A, nullptr) == MOE_OK && only(stubs::kCombine, 1),
           "combine -> launch_combine");
    stubs::reset();
    expect(moe_combine_scatter(A, 14336, 512, I, I, 64, 8, 7168, A, 14336, 512LL * 14336, nullptr) == MOE_OK &&
               only(stubs::kCombineScatter, 1),
           "combine_scatter with exactly S*K rows of staging");
    expect(moe_combine_scatter(A, 14336, 512, I, I, 64, 8, 7168, A, 14336, 512LL * 14336 - 1, nullptr) ==
               MOE_ERR_WINDOW,
           "combine_scatter one byte short");
    stubs::reset();
    expect(moe_combine_staged(A, 14336, 511LL * 14336 + 14336, I, F, 64, 7168, 8, A, nullptr) == MOE_OK &&
               only(stubs::kCombineStaged, 1),
           "combine_staged with exactly S*K rows of staging");
    expect(moe_combine_staged(A, 14336, 511LL * 14336 + 14335, I, F, 64, 7168, 8, A, nullptr) == MOE_ERR_WINDOW,
           "combine_staged one byte short");
    expect(moe_combine_staged(A, 16384, 511LL * 16384 + 14336, I, F, 64, 7168, 8, A, nullptr) == MOE_OK,
           "combine_staged: the last row needs only 2H bytes");
    stubs::reset();
    expect(moe_unpack(A, win, I, 64, 8, 7168, 1, A, F, I, nullptr) == MOE_OK && only(stubs::kUnpack, 1),
           "unpack");
    stubs::reset();
    expect(moe_unpack_padded(A, win, I, 256, 64, 8, 7168, 0, 16, MOE_MAX_OUT_ROWS, A, nullptr, I, I, I,
                             nullptr) == MOE_OK &&
               only(stubs::kUnpackPadded, 1),
           "unpack_padded at the largest out_rows");
    stubs::reset();
    expect(moe_rank_rows(I, 64, 8, 256, 8, 16, I, I, I, I, nullptr) == MOE_OK && only(stubs::kRankRows, 1),
           "rank_rows");
    stubs::reset();
    expect(moe_dispatch_dedup(A, I, I, 64, 7168, 8, 256, 8, 1, 0, A, moe_dedup_window_bytes(64, 8, 8, 7168),
                              nullptr) == MOE_OK &&
               only(stubs::kPackDedup, 1),
           "dispatch_dedup");
    stubs::reset();
    expect(moe_expand_dedup(A, moe_dedup_window_bytes(64, 8, 8, 7168), I, I, I, 64, 8, 8, 7168, 2, A, F, I,
                            nullptr) == MOE_OK &&
               only(stubs::kExpandDedup, 1),
           "expand_dedup");

    // pre-validated calls reach the same launchers as the direct calls
    {
        moe_plan plan;
        stubs::reset();
        expect(moe_plan_layout(&plan, I, 64, 8, 256, 8, 16, U, I, I, I, I, I, I, I, I, MOE_LAYOUT_AUTO) == MOE_OK &&
                   only(stubs::kLaunchers, 0),
               "plan_layout checks without launching");
        expect(moe_plan_run(&plan, nullptr) == MOE_OK && only(stubs::kLayoutSmall, 1), "plan_run layout small");
        stubs::reset();
        expect(moe_plan_layout(&plan, I, 513, 8, 256, 8, 16, U, I, I, I, I, I, I, I, I, MOE_LAYOUT_AUTO) == MOE_OK &&
                   moe_plan_run(&plan, nullptr) == MOE_OK && only(stubs::kLayout, 1),
               "plan_run layout multi");
        stubs::reset();
        expect(moe_plan_layout_dispatch(&plan, I, 64, 8, 256, 8, 16, U, I, I, I, I, I, I, I, I, A, 7168, 1, 0, A,
                                        win, MOE_LAYOUT_AUTO) == MOE_OK &&
                   moe_plan_run(&plan, nullptr) == MOE_OK && moe_plan_run(&plan, nullptr) == MOE_OK &&
                   only(stubs::kLayoutDispatchSmall, 2),
               "plan_run layout_dispatch twice -> one kernel each");
        stubs::reset();
        expect(moe_plan_layout_dispatch(&plan, I, 513, 8, 256, 8, 128, U, I, I, I, I, I, I, I, I, A, 7168, 0, 0, A,
                                        moe_window_bytes(513, 8, 7168), MOE_LAYOUT_AUTO) == MOE_OK &&
                   moe_plan_run(&plan, nullptr) == MOE_OK && only(stubs::kLayout, 1, stubs::kPack, 1),
               "plan_run layout_dispatch large -> layout + pack");
        const int64_t wbig = moe_window_bytes(4096, 8, 7168);
        stubs::reset();
        expect(moe_plan_dispatch_ws(&plan, A, I, 4096, 7168, 8, 0, 0, A, wbig, A,
                                    moe_dispatch_workspace_bytes(4096, 8, 0)) == MOE_OK &&
                   moe_plan_run(&plan, nullptr) == MOE_OK && only(stubs::kPackPlanned, 1),
               "plan_run dispatch_ws -> planned pack");
        stubs::reset();
        expect(moe_plan_combine(&plan, A, 14848, 512, I, F, 64, 7168, 8, A) == MOE_OK &&
                   moe_plan_run(&plan, nullptr) == MOE_OK && only(stubs::kCombine, 1),
               "plan_run combine");
        stubs::reset();
        expect(moe_plan_combine(&plan, A, 100, 512, I, F, 64, 7168, 8, A) == MOE_ERR_ARG &&
                   moe_plan_run(&plan, nullptr) == MOE_ERR_ARG && only(stubs::kLaunchers, 0),
               "a failed plan cannot be run");
    }

    if (failures == 0) std::printf("abi_asan ok\n");
    return failures == 0 ? 0 : 1;
}
