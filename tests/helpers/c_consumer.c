/*
 * A C consumer of libnvfp4rq (test helper, GPU): draws a Student-t x
 * log-normal bf16 tensor with the seeded generator library, quantizes it on
 * the device through the C ABI only (HIP runtime C API for memory, no
 * PyTorch), and compares codes, scales, global scale and amax with the CPU
 * oracle byte for byte.  Prints one line and exits 0 on agreement.
 *
 *   c_consumer ROWS COLS
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "nvfp4rq.h"

int synth_t3_lognormal(uint64_t seed, int64_t rows, int64_t cols, uint16_t *out);
int oracle_quantize(const void *x, int is_f32, int64_t rows, int64_t cols, int rotate, uint8_t *q,
                    uint8_t *s, float *g_out, float *amax_out, int nthreads);

#define HIP_OK(call)                                                              \
    do {                                                                          \
        hipError_t e_ = (call);                                                   \
        if (e_ != hipSuccess) {                                                   \
            printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            return 2;                                                             \
        }                                                                         \
    } while (0)

int main(int argc, char **argv)
{
    if (argc != 3)
        return 64;
    const int64_t rows = atoll(argv[1]), cols = atoll(argv[2]), n = rows * cols;
    uint16_t *x = malloc((size_t)n * 2);
    uint8_t *q = malloc((size_t)n / 2), *s = malloc((size_t)n / 16);
    uint8_t *oq = malloc((size_t)n / 2), *os = malloc((size_t)n / 16);
    if (!x || !q || !s || !oq || !os || synth_t3_lognormal(7, rows, cols, x) != 0)
        return 3;
    void *dx, *dq, *ds, *dg, *da;
    HIP_OK(hipMalloc(&dx, (size_t)n * 2));
    HIP_OK(hipMalloc(&dq, (size_t)n / 2));
    HIP_OK(hipMalloc(&ds, (size_t)n / 16));
    HIP_OK(hipMalloc(&dg, 4));
    HIP_OK(hipMalloc(&da, 4));
    HIP_OK(hipMemcpy(dx, x, (size_t)n * 2, hipMemcpyHostToDevice));
    nvfp4_status st = nvfp4_rotquant(dx, rows, cols, 1, dq, ds, dg, da, 0);
    if (st != NVFP4_OK) {
        printf("nvfp4_rotquant: %s\n", nvfp4_status_string(st));
        return 4;
    }
    float g, a, og, oa;
    HIP_OK(hipMemcpy(q, dq, (size_t)n / 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(s, ds, (size_t)n / 16, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(&g, dg, 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(&a, da, 4, hipMemcpyDeviceToHost));
    if (oracle_quantize(x, 0, rows, cols, 1, oq, os, &og, &oa, 0) != 0)
        return 5;
    const int same = memcmp(q, oq, (size_t)n / 2) == 0 && memcmp(s, os, (size_t)n / 16) == 0 &&
                     memcmp(&g, &og, 4) == 0 && memcmp(&a, &oa, 4) == 0;
    printf("%lldx%lld codes/scales/g/amax %s (g %.9g, amax %.9g)\n", (long long)rows,
           (long long)cols, same ? "identical" : "DIFFER", g, a);
    hipFree(dx);
    hipFree(dq);
    hipFree(ds);
    hipFree(dg);
    hipFree(da);
    free(x);
    free(q);
    free(s);
    free(oq);
    free(os);
    return same ? 0 : 1;
}
