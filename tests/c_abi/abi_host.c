/* Plain C consumer of include/moe.h: links libmoe.so and calls the host-only entry points and the
 * host-side validation of the device entry points (fake, never dereferenced device addresses).
 * Built and run by tests/test_c_abi.py; prints one line per check and exits non-zero on failure. */
#include <stdio.h>
#include <stdint.h>
#include <string.h>

#include "moe.h"

static int failures = 0;

static void check(int ok, const char *what) {
    printf("%s %s\n", ok ? "ok  " : "FAIL", what);
    if (!ok) failures++;
}

int main(void) {
    void *dev = (void *)(uintptr_t)0x10000; /* 512-byte aligned fake device address */
    int64_t payload = 0, scale_off = 0, triple_off = 0, tail_end = 0;

    check(moe_slot_bytes(7168) == 14848, "moe_slot_bytes(7168) == 14848");
    check(moe_window_bytes(4096, 8, 7168) == (int64_t)4096 * 8 * 14848, "moe_window_bytes at S=4096");
    check(moe_dedup_window_bytes(128, 8, 4, 7168) == (int64_t)128 * 4 * 14848, "moe_dedup_window_bytes");
    check(moe_slot_offsets(7168, MOE_QUANT_FP8_E4M3_DYN, &payload, &scale_off, &triple_off, &tail_end) == MOE_OK &&
              payload == 7168 && scale_off == 7168 && triple_off == 7200 && tail_end == 7296,
          "moe_slot_offsets fp8 at H=7168");
    check(moe_slot_bytes(1000) == MOE_ERR_UNSUPPORTED, "H % 16 != 0 is unsupported");
    check(moe_layout(NULL, 64, 8, 256, 8, 16, dev, dev, dev, dev, dev, dev, dev, dev, dev, NULL) == MOE_ERR_ARG,
          "moe_layout rejects a null topk_idx");
    check(moe_layout(dev, 64, 8, 250, 8, 16, dev, dev, dev, dev, dev, dev, dev, dev, dev, NULL) ==
              MOE_ERR_UNSUPPORTED,
          "moe_layout rejects E % P != 0");
    check(moe_dispatch(dev, dev, 64, 7168, 8, MOE_QUANT_NONE, 0, dev, 100, NULL) == MOE_ERR_WINDOW,
          "moe_dispatch rejects a small window");
    check(moe_layout_dispatch(dev, 64, 8, 256, 8, 16, dev, dev, dev, dev, dev, dev, dev, dev, dev, dev,
                              7168, MOE_QUANT_FP8_E4M3_DYN, 0, dev, 100, NULL) == MOE_ERR_WINDOW,
          "moe_layout_dispatch rejects a small window");
    check(moe_combine(dev, 14336, 512, dev, dev, 64, 7168, 8, (char *)dev + 8, NULL) == MOE_ERR_ALIGN,
          "moe_combine rejects a misaligned y");
    {
        const int64_t ws = moe_layout_dispatch_workspace_bytes(4096, 8, 256, 8, 128, MOE_QUANT_NONE, MOE_LAYOUT_AUTO);
        moe_plan plan;
        memset(&plan, 0, sizeof(plan));
        check(ws == 525312, "moe_layout_dispatch_workspace_bytes at S=4096, C=128");
        check(moe_layout_dispatch_workspace_bytes(64, 8, 256, 8, 16, MOE_QUANT_NONE, MOE_LAYOUT_AUTO) == 0,
              "no workspace for a table the single kernel takes");
        check(moe_layout_ws(dev, 4096, 8, 256, 8, 128, dev, dev, dev, dev, dev, dev, dev, dev, dev, MOE_QUANT_NONE,
                            MOE_LAYOUT_AUTO, dev, ws - 1, NULL) == MOE_ERR_WINDOW,
              "moe_layout_ws rejects a short workspace");
        check(moe_dispatch_planned(dev, dev, 4096, 7168, 8, 128, MOE_QUANT_NONE, 0, dev,
                                   moe_window_bytes(4096, 8, 7168), NULL, 0, NULL) == MOE_ERR_ARG,
              "moe_dispatch_planned needs the workspace for a planned table");
        check(moe_plan_layout_ws(&plan, dev, 4096, 8, 256, 8, 128, dev, dev, dev, dev, dev, dev, dev, dev, dev,
                                 MOE_QUANT_NONE, MOE_LAYOUT_AUTO, NULL, ws) == MOE_ERR_ARG &&
                  moe_plan_run(&plan, NULL) == MOE_ERR_ARG,
              "a plan that failed its checks is refused");
    }
    check(strlen(moe_status_string(MOE_ERR_WINDOW)) > 0, "moe_status_string");
    printf("%d failure(s)\n", failures);
    return failures ? 1 : 0;
}
