/* A plain C99 caller of the DyT C ABI (include/dyt.h): compiled with gcc
 * against libdyt.so by tests/test_abi_cpu.py. Uses only calls that never
 * reach the GPU: version, status strings, plans, workspace sizes and
 * argument validation (which runs before anything is enqueued). Prints one
 * line per check; exits non-zero on the first mismatch. */
#include <stdio.h>
#include <string.h>

#include "dyt.h"

static int fails = 0;

static void expect(int cond, const char* what) {
    printf("%s %s\n", cond ? "ok" : "FAIL", what);
    if (!cond) ++fails;
}

int main(void) {
    dyt_plan p;
    expect(dyt_abi_version() == DYT_ABI_VERSION, "abi version matches the header");
    expect(strcmp(dyt_status_string(DYT_OK), "DYT_OK") == 0, "status string of DYT_OK");
    expect(strlen(dyt_build_id()) == 16, "build id of 16 hex digits");
    expect(dyt_get_plan(32768, 4096, DYT_BF16, DYT_F32, 1, &p) == DYT_OK, "backward plan");
    expect(p.vec == 8 && p.block == 256 && p.ws_bytes > 0, "plan fields");
    expect(dyt_backward_workspace_size(32768, 4096, DYT_BF16, DYT_F32) >= (size_t)p.ws_bytes,
           "workspace size covers the plan");
    expect(dyt_get_forward_plan(4, 4, 99, DYT_F32, 1, &p) == DYT_ERR_UNSUPPORTED_DTYPE,
           "unknown dtype code");
    expect(dyt_forward(NULL, NULL, NULL, NULL, NULL, 4, 4, DYT_F32, DYT_F32, NULL) ==
               DYT_ERR_INVALID_ARG, "null pointers rejected before any launch");
    expect(dyt_forward(NULL, NULL, NULL, NULL, NULL, -1, 4, DYT_F32, DYT_F32, NULL) ==
               DYT_ERR_INVALID_ARG, "negative M");
    expect(dyt_forward(NULL, NULL, NULL, NULL, NULL, 0, 4, DYT_F32, DYT_F32, NULL) == DYT_OK,
           "empty problem is a no-op");
    return fails == 0 ? 0 : 1;
}
