/* A plain C99 consumer of the C ABI: the header compiles as C and the library links.  Only calls that end in
 * host-side validation run here (no device is touched), so it runs on a machine without a GPU. */
#include <stdio.h>
#include <string.h>

#include "lowbit.h"

static int failures = 0;

static void expect(int ok, const char *what)
{
    if (!ok) {
        printf("FAIL %s\n", what);
        failures++;
    }
}

int main(void)
{
    /* a 16-byte-aligned stand-in address, never dereferenced: every call below fails validation first */
    void *p = (void *)(size_t)(1u << 20);

    expect(strcmp(lowbit_status_str(LB_OK), "LB_OK") == 0, "status string of LB_OK");
    expect(lowbit_weight_bytes(LB_Q1_0, 4096, 4096) == 2359296, "Q1_0 bytes of 4096 x 4096");
    expect(lowbit_weight_bytes(LB_Q2_0_G64, 4096, 4096) == 4718592, "Q2_0_g64 bytes of 4096 x 4096");
    expect(lowbit_weight_bytes(LB_TERNARY_PLANAR, 6912, 2560) == 4423680, "planar bytes of 6912 x 2560");

    expect(lowbit_gemm(LB_Q2_0_G64, p, 8, 64, 1.0f, LB_ACT_Q8_0, p, p, -1, (float *)p, NULL) == LB_ESHAPE,
           "negative M is LB_ESHAPE");
    expect(strncmp(lowbit_last_error(), "lowbit_gemm: ", 13) == 0, "the last error names the call");
    expect(lowbit_matvec(LB_Q2_0_G64, p, 8, 96, 1.0f, LB_ACT_Q8_0, (const int8_t *)p, p, (float *)p, NULL) ==
               LB_ESHAPE, "K not a multiple of the block is LB_ESHAPE");
    expect(lowbit_matvec(LB_TERNARY_PLANAR, p, 8, 64, 1.0f, LB_ACT_Q8_0, (const int8_t *)p, p, (float *)p, NULL) ==
               LB_EINVAL, "a mismatched activation format is LB_EINVAL");

    lb_batch *b = (lb_batch *)p;
    expect(lowbit_batch_create(NULL, 1, &b) == LB_EINVAL && b == NULL, "a null work list is LB_EINVAL");
    lowbit_batch_destroy(NULL);

    if (failures == 0)
        printf("ok\n");
    return failures == 0 ? 0 : 1;
}
