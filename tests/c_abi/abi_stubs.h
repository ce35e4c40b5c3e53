// Call counters of the stand-in launchers in abi_stubs.cpp.
#pragma once

#include "moe_internal.h"

namespace stubs {
enum Launcher {
    kLayout, kLayoutSmall, kLayoutDispatchSmall, kRankRows, kPackDedup, kExpandDedup, kPack, kPackPlanned, kCombine,
    kCombineScatter, kCombineStaged, kUnpackPadded, kUnpack, kLaunchers
};
extern int calls[kLaunchers];
void reset();
}  // namespace stubs
