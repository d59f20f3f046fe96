/* A plain C caller of libaarms.so: includes the public header, links the
 * library and drives the argument checks that run before any HIP call, so
 * it needs no GPU.  Device pointers are integers that are never
 * dereferenced.  Exit status 0 when every check returns what the header
 * documents, else the number of the first failing check. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "aarms.h"

#define P(k) ((void *)(uintptr_t)(0x10000ull + ((uint64_t)(k) << 32)))

static int n_check = 0;

static int expect(int got, int want, const char *what)
{
    ++n_check;
    if (got != want) {
        fprintf(stderr, "check %d (%s): got %d (%s), want %d\n", n_check, what, got,
                aarms_status_string(got), want);
        return 1;
    }
    return 0;
}

int main(void)
{
    int bad = 0;
    const void *x = P(1), *res = P(2), *w = P(3), *gu = P(4);
    void *out = P(5), *res_out = P(6);
    float *scale_out = (float *)P(7);

    if (aarms_status_string(AARMS_OK) == NULL || strlen(aarms_status_string(AARMS_ERR_ALIAS)) == 0)
        return 100;
    bad |= expect(fused_add_rmsnorm(out, res_out, x, res, w, 0, 1536, 1e-6f, 0), AARMS_OK, "zero tokens");
    bad |= expect(fused_add_rmsnorm(NULL, res_out, x, res, w, 4, 1536, 1e-6f, 0), AARMS_ERR_NULL_POINTER, "null out");
    bad |= expect(fused_add_rmsnorm(out, res_out, x, res, w, 4, 1540, 1e-6f, 0), AARMS_ERR_BAD_SHAPE, "width % 8");
    bad |= expect(fused_add_rmsnorm(out, res_out, x, res, w, 4, 1536, -1.0f, 0), AARMS_ERR_BAD_EPS, "negative eps");
    bad |= expect(fused_add_rmsnorm(out, out, x, res, w, 4, 1536, 1e-6f, 0), AARMS_ERR_ALIAS, "out == residual_out");
    bad |= expect(fused_add_rmsnorm((char *)out + 8, res_out, x, res, w, 4, 1536, 1e-6f, 0), AARMS_ERR_MISALIGNED,
                  "misaligned out");
    bad |= expect(fused_add_rmsnorm_ex(out, res_out, x, res, w, 4, 16384, 1e-6f, 0, 0), AARMS_ERR_BAD_VARIANT,
                  "variant too narrow");
    bad |= expect(swiglu(out, gu, 4, 8964, 0), AARMS_ERR_BAD_SHAPE, "inter % 8");
    bad |= expect(swiglu(out, gu, 0, 8960, 0), AARMS_OK, "swiglu zero tokens");
    bad |= expect(swiglu_quant_fp8(out, gu, NULL, 4, 8960, 0), AARMS_ERR_NULL_POINTER, "null scale");
    bad |= expect(fused_add_rmsnorm_quant_fp8(out, NULL, res_out, x, res, w, 4, 16384, 1e-5f, 0),
                  AARMS_ERR_NULL_POINTER, "null scale_out");
    bad |= expect(fused_add_rmsnorm_quant_fp8_group(out, scale_out, res_out, x, res, w, 4, 16392, 1e-5f, 0),
                  AARMS_ERR_BAD_SHAPE, "group width % 128");
    bad |= expect(swiglu_quant_nvfp4(out, (uint8_t *)scale_out, gu, NULL, 4, 8960, 0), AARMS_ERR_NULL_POINTER,
                  "null tensor scale");
    bad |= expect(aarms_pick_variant(0, 16, 1536, 0) >= 0, 1, "a norm variant for [16, 1536]");
    bad |= expect(aarms_variant_name(0, aarms_variant_count(0)) == NULL, 1, "no name past the table");
    if (bad) return 1;
    printf("%d checks passed\n", n_check);
    return 0;
}
