// Stand-ins for the kernel launchers of combine_moe_layout_02_amd/csrc (moe_internal.h), for a host
// build of the C ABI layer (moe_api.cpp) with the address and undefined-behaviour sanitizers:
// nothing runs on a GPU, each launcher only records that it was called and returns success.
#include "abi_stubs.h"

namespace stubs {
int calls[kLaunchers];
moe::LayoutWorkspace last_ws;
const void *last_plan;
moe::PackChunks last_chunks;
void reset() {
    for (int &c : calls) c = 0;
    last_ws = moe::LayoutWorkspace{};
    last_plan = nullptr;
    last_chunks = moe::PackChunks{};
}
}  // namespace stubs

namespace moe {
using stubs::calls;

hipError_t launch_layout(const int32_t *, int32_t, int32_t, int32_t, int32_t, int32_t, uint8_t *, int32_t *,
                         int32_t *, int32_t *, int32_t *, int32_t *, int32_t *, int32_t *, int32_t *,
                         hipStream_t) {
    ++calls[stubs::kLayout];
    return hipSuccess;
}
hipError_t launch_layout_ws(const int32_t *, int32_t, int32_t, int32_t, int32_t, int32_t, uint8_t *, int32_t *,
                            int32_t *, int32_t *, int32_t *, int32_t *, int32_t *, int32_t *, int32_t *,
                            const LayoutWorkspace &ws, hipStream_t) {
    ++calls[stubs::kLayoutWs];
    stubs::last_ws = ws;
    return hipSuccess;
}
hipError_t launch_pack_from_plan(const void *, const void *plan, const PackChunks &pc, int32_t, int32_t, int32_t,
                                 int32_t, void *, hipStream_t) {
    ++calls[stubs::kPackFromPlan];
    stubs::last_plan = plan;
    stubs::last_chunks = pc;
    return hipSuccess;
}
hipError_t launch_layout_small(const int32_t *, int32_t, int32_t, int32_t, int32_t, int32_t, uint8_t *,
                               int32_t *, int32_t *, int32_t *, int32_t *, int32_t *, int32_t *, int32_t *,
                               int32_t *, hipStream_t) {
    ++calls[stubs::kLayoutSmall];
    return hipSuccess;
}
hipError_t launch_layout_dispatch_small(const int32_t *, int32_t, int32_t, int32_t, int32_t, int32_t,
                                        uint8_t *, int32_t *, int32_t *, int32_t *, int32_t *, int32_t *,
                                        int32_t *, int32_t *, int32_t *, const void *, int32_t, int32_t,
                                        int32_t, void *, hipStream_t) {
    ++calls[stubs::kLayoutDispatchSmall];
    return hipSuccess;
}
hipError_t launch_rank_rows(const int32_t *, int32_t, int32_t, int32_t, int32_t, int32_t, const int32_t *,
                            const int32_t *, int32_t *, int32_t *, hipStream_t) {
    ++calls[stubs::kRankRows];
    return hipSuccess;
}
hipError_t launch_pack_dedup(const void *, const int32_t *, const int32_t *, int32_t, int32_t, int32_t,
                             int32_t, int32_t, int32_t, int32_t, void *, hipStream_t) {
    ++calls[stubs::kPackDedup];
    return hipSuccess;
}
hipError_t launch_expand_dedup(const void *, const int32_t *, const int32_t *, const int32_t *, int32_t,
                               int32_t, int32_t, int32_t, int32_t, void *, float *, int32_t *,
                               hipStream_t) {
    ++calls[stubs::kExpandDedup];
    return hipSuccess;
}
hipError_t launch_pack(const void *, const int32_t *, int32_t, int32_t, int32_t, int32_t, int32_t, void *,
                       hipStream_t) {
    ++calls[stubs::kPack];
    return hipSuccess;
}
hipError_t launch_pack_planned(const void *, const int32_t *, int32_t, int32_t, int32_t, int32_t, void *,
                               void *workspace, hipStream_t) {
    ++calls[stubs::kPackPlanned];
    stubs::last_plan = workspace;
    return hipSuccess;
}
hipError_t launch_combine(const void *, int64_t, int64_t, const int32_t *, const float *, int32_t, int32_t,
                          int32_t, void *, hipStream_t) {
    ++calls[stubs::kCombine];
    return hipSuccess;
}
hipError_t launch_combine_scatter(const void *, int64_t, int64_t, const int32_t *, const int32_t *, int32_t,
                                  int32_t, int32_t, void *, int64_t, hipStream_t) {
    ++calls[stubs::kCombineScatter];
    return hipSuccess;
}
hipError_t launch_combine_staged(const void *, int64_t, const int32_t *, const float *, int32_t, int32_t,
                                 int32_t, void *, hipStream_t) {
    ++calls[stubs::kCombineStaged];
    return hipSuccess;
}
hipError_t launch_unpack_padded(const void *, const int32_t *, int32_t, int32_t, int32_t, int32_t, int32_t,
                                int32_t, int64_t, void *, float *, int32_t *, int32_t *, int32_t *,
                                hipStream_t) {
    ++calls[stubs::kUnpackPadded];
    return hipSuccess;
}
hipError_t launch_unpack(const void *, const int32_t *, int32_t, int32_t, int32_t, int32_t, void *, float *,
                         int32_t *, hipStream_t) {
    ++calls[stubs::kUnpack];
    return hipSuccess;
}
}  // namespace moe
