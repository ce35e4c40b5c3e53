// Native consumer of include/moe.h on the GPU: no Python, no torch. Reads a routing table, x,
// weights and expert rows from the binary input file, runs the layout and the pack, then
// moe_combine, on hipMalloc'd buffers through libmoe.so, and writes slot_idx, the dispatched slot
// regions and y to the output file for the test to compare with the oracle. `mode` picks the calls:
//   0  moe_layout -> moe_dispatch -> moe_combine
//   1  moe_layout_dispatch -> moe_combine
//   2  moe_layout_ws -> moe_dispatch_planned -> moe_combine (workspace of
//      moe_layout_dispatch_workspace_bytes bytes)
//   3  the calls of mode 2 as pre-validated plans (moe_plan_layout_ws, moe_plan_dispatch_planned,
//      moe_plan_combine), each run by moe_plan_run
//
// Input file: int32 S, K, H, E, P, C, quant, mode; int32 topk[S*K]; uint16 x[S*H];
//             float w[S*K]; uint16 expert_out[S*K*H].
// Output file: int32 status; int32 slot_idx[S*K]; uint8 window[S*K*slot_bytes]; uint16 y[S*H].
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <vector>

#include "moe.h"

#define CHECK_HIP(x)                                                                  \
    do {                                                                              \
        hipError_t e_ = (x);                                                          \
        if (e_ != hipSuccess) {                                                       \
            std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));       \
            return 2;                                                                 \
        }                                                                             \
    } while (0)
#define CHECK_MOE(x)                                                                  \
    do {                                                                              \
        int s_ = (x);                                                                 \
        if (s_ != MOE_OK) {                                                           \
            std::fprintf(stderr, "%s failed: %s\n", #x, moe_status_string(s_));       \
            return 3;                                                                 \
        }                                                                             \
    } while (0)

template <typename T>
static bool read_n(FILE *f, std::vector<T> &v, size_t n) {
    v.resize(n);
    return std::fread(v.data(), sizeof(T), n, f) == n;
}

int main(int argc, char **argv) {
    if (argc != 3) {
        std::fprintf(stderr, "usage: %s input output\n", argv[0]);
        return 1;
    }
    FILE *in = std::fopen(argv[1], "rb");
    if (!in) return 1;
    int32_t hdr[8];
    if (std::fread(hdr, sizeof(int32_t), 8, in) != 8) return 1;
    const int32_t S = hdr[0], K = hdr[1], H = hdr[2], E = hdr[3], P = hdr[4], C = hdr[5], quant = hdr[6];
    const int mode = hdr[7];
    if (mode < 0 || mode > 3) return 1;
    std::vector<int32_t> topk;
    std::vector<uint16_t> x, eo;
    std::vector<float> w;
    if (!read_n(in, topk, (size_t)S * K) || !read_n(in, x, (size_t)S * H) || !read_n(in, w, (size_t)S * K) ||
        !read_n(in, eo, (size_t)S * K * H))
        return 1;
    std::fclose(in);

    const int64_t slot_bytes = moe_slot_bytes(H);
    const int64_t window_bytes = moe_window_bytes(S, K, H);
    if (slot_bytes < 0 || window_bytes < 0) return 4;

    hipStream_t stream;
    CHECK_HIP(hipStreamCreate(&stream));
    int32_t *d_topk, *d_npr, *d_npe, *d_rpm, *d_epm, *d_rsb, *d_esb, *d_slot, *d_status;
    uint8_t *d_in_rank, *d_window;
    void *d_x, *d_eo, *d_y;
    float *d_w;
    CHECK_HIP(hipMalloc(&d_topk, sizeof(int32_t) * S * K));
    CHECK_HIP(hipMalloc(&d_in_rank, (size_t)S * P));
    CHECK_HIP(hipMalloc(&d_npr, sizeof(int32_t) * P));
    CHECK_HIP(hipMalloc(&d_npe, sizeof(int32_t) * E));
    CHECK_HIP(hipMalloc(&d_rpm, sizeof(int32_t) * P * C));
    CHECK_HIP(hipMalloc(&d_epm, sizeof(int32_t) * E * C));
    CHECK_HIP(hipMalloc(&d_rsb, sizeof(int32_t) * (P + 1)));
    CHECK_HIP(hipMalloc(&d_esb, sizeof(int32_t) * (E + 1)));
    CHECK_HIP(hipMalloc(&d_slot, sizeof(int32_t) * S * K));
    CHECK_HIP(hipMalloc(&d_status, sizeof(int32_t)));
    CHECK_HIP(hipMalloc(&d_window, window_bytes));
    CHECK_HIP(hipMalloc(&d_x, sizeof(uint16_t) * S * H));
    CHECK_HIP(hipMalloc(&d_eo, sizeof(uint16_t) * S * K * H));
    CHECK_HIP(hipMalloc(&d_y, sizeof(uint16_t) * S * H));
    CHECK_HIP(hipMalloc(&d_w, sizeof(float) * S * K));
    CHECK_HIP(hipMemcpy(d_topk, topk.data(), sizeof(int32_t) * S * K, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_x, x.data(), sizeof(uint16_t) * S * H, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_eo, eo.data(), sizeof(uint16_t) * S * K * H, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_w, w.data(), sizeof(float) * S * K, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemset(d_window, 0xAB, window_bytes));

    void *d_ws = nullptr;
    const int64_t ws_bytes = moe_layout_dispatch_workspace_bytes(S, K, E, P, C, quant, MOE_LAYOUT_AUTO);
    if (ws_bytes < 0) return 4;
    if (ws_bytes > 0) CHECK_HIP(hipMalloc(&d_ws, ws_bytes));
    if (mode == 1) {
        CHECK_MOE(moe_layout_dispatch(d_topk, S, K, E, P, C, d_in_rank, d_npr, d_npe, d_rpm, d_epm, d_rsb, d_esb,
                                      d_slot, d_status, d_x, H, quant, 0, d_window, window_bytes, stream));
    } else if (mode == 2) {
        CHECK_MOE(moe_layout_ws(d_topk, S, K, E, P, C, d_in_rank, d_npr, d_npe, d_rpm, d_epm, d_rsb, d_esb, d_slot,
                                d_status, quant, MOE_LAYOUT_AUTO, d_ws, ws_bytes, stream));
        CHECK_MOE(moe_dispatch_planned(d_x, d_slot, S, H, K, C, quant, 0, d_window, window_bytes, d_ws, ws_bytes,
                                       stream));
    } else if (mode == 3) {
        moe_plan plans[3];
        CHECK_MOE(moe_plan_layout_ws(&plans[0], d_topk, S, K, E, P, C, d_in_rank, d_npr, d_npe, d_rpm, d_epm, d_rsb,
                                     d_esb, d_slot, d_status, quant, MOE_LAYOUT_AUTO, d_ws, ws_bytes));
        CHECK_MOE(moe_plan_dispatch_planned(&plans[1], d_x, d_slot, S, H, K, C, quant, 0, d_window, window_bytes, d_ws,
                                            ws_bytes));
        CHECK_MOE(moe_plan_combine(&plans[2], d_eo, 2 * (int64_t)H, (int64_t)S * K, d_slot, d_w, S, H, K, d_y));
        for (const moe_plan &p : plans) CHECK_MOE(moe_plan_run(&p, stream));
    } else {
        CHECK_MOE(moe_layout(d_topk, S, K, E, P, C, d_in_rank, d_npr, d_npe, d_rpm, d_epm, d_rsb, d_esb, d_slot,
                             d_status, stream));
        CHECK_MOE(moe_dispatch(d_x, d_slot, S, H, K, quant, 0, d_window, window_bytes, stream));
    }
    if (mode != 3)
        CHECK_MOE(moe_combine(d_eo, 2 * (int64_t)H, (int64_t)S * K, d_slot, d_w, S, H, K, d_y, stream));
    CHECK_HIP(hipStreamSynchronize(stream));

    int32_t status = 0;
    std::vector<int32_t> slot((size_t)S * K);
    std::vector<uint8_t> window((size_t)window_bytes);
    std::vector<uint16_t> y((size_t)S * H);
    CHECK_HIP(hipMemcpy(&status, d_status, sizeof(int32_t), hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(slot.data(), d_slot, sizeof(int32_t) * S * K, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(window.data(), d_window, window_bytes, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(y.data(), d_y, sizeof(uint16_t) * S * H, hipMemcpyDeviceToHost));

    FILE *out = std::fopen(argv[2], "wb");
    if (!out) return 1;
    std::fwrite(&status, sizeof(int32_t), 1, out);
    std::fwrite(slot.data(), sizeof(int32_t), slot.size(), out);
    std::fwrite(window.data(), 1, window.size(), out);
    std::fwrite(y.data(), sizeof(uint16_t), y.size(), out);
    std::fclose(out);

    void *bufs[] = {d_topk, d_in_rank, d_npr, d_npe, d_rpm, d_epm, d_rsb, d_esb, d_slot, d_status, d_window,
                    d_x, d_eo, d_y, d_w};
    for (void *b : bufs) CHECK_HIP(hipFree(b));
    if (d_ws) CHECK_HIP(hipFree(d_ws));
    CHECK_HIP(hipStreamDestroy(stream));
    std::printf("abi_gpu ok: S=%d K=%d H=%d E=%d P=%d C=%d quant=%d mode=%d\n", S, K, H, E, P, C, quant, mode);
    return 0;
}
