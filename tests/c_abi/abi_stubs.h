// Call counters of the stand-in launchers in abi_stubs.cpp.
#pragma once

#include "moe_internal.h"

namespace stubs {
enum Launcher {
    kLayout, kLayoutWs, kPackFromPlan, kLayoutSmall, kLayoutDispatchSmall, kRankRows, kPackDedup, kExpandDedup, kPack, kPackPlanned, kCombine,
    kCombineScatter, kCombineStaged, kUnpackPadded, kUnpack, kLaunchers
};
extern int calls[kLaunchers];
extern moe::LayoutWorkspace last_ws;  // what launch_layout_ws was last given
extern const void *last_plan;         // the plan launch_pack_from_plan / launch_pack_planned last read
extern moe::PackChunks last_chunks;   // the chunks launch_pack_from_plan was last given
void reset();
}  // namespace stubs
