/* A plain C client of librankred: the only headers it needs are rc.h and the
 * HIP runtime API for device memory.  Reads R rank inputs of N float32 from a
 * file, runs all_reduce (Sum) and reduce_scatter (Max) through the C ABI on
 * the null stream, and writes rank 0's all_reduce output followed by every
 * rank's reduce_scatter shard to another file.  Also checks that a shape
 * mismatch comes back as RC_ERR_SHAPE_MISMATCH with a message.
 *
 *   c_client <R> <N> <inputs.bin> <outputs.bin>      (N divisible by R) */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "rc.h"

#define CHECK_HIP(x)                                                       \
    do {                                                                   \
        hipError_t e_ = (x);                                               \
        if (e_ != hipSuccess) {                                            \
            fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));        \
            return 10;                                                     \
        }                                                                  \
    } while (0)

static void describe(rc_buf* b, const void* send, void* recv, long long n, int op) {
    memset(b, 0, sizeof *b);
    b->send = send;
    b->recv = recv;
    b->dtype = RC_F32;
    b->op = op;
    b->ndim = 1;
    b->dims[0] = n;
}

int main(int argc, char** argv) {
    if (argc != 5) return 2;
    const int R = atoi(argv[1]);
    const long long N = atoll(argv[2]);
    if (R < 1 || R > RC_MAX_RANKS || N < 1 || N % R) return 2;
    const size_t bytes = (size_t)N * sizeof(float);
    float* host = (float*)malloc(bytes * R);
    FILE* f = fopen(argv[3], "rb");
    if (!host || !f || fread(host, bytes, R, f) != (size_t)R) return 3;
    fclose(f);

    void *send[RC_MAX_RANKS], *recv[RC_MAX_RANKS], *shard[RC_MAX_RANKS];
    for (int r = 0; r < R; ++r) {
        CHECK_HIP(hipMalloc(&send[r], bytes));
        CHECK_HIP(hipMalloc(&recv[r], bytes));
        CHECK_HIP(hipMalloc(&shard[r], bytes / R));
        CHECK_HIP(hipMemcpy(send[r], host + (size_t)r * N, bytes, hipMemcpyHostToDevice));
    }
    if (rc_abi_version() != RC_ABI_VERSION) return 4;
    if (rc_register(R, NULL) != RC_OK) {
        fprintf(stderr, "register: %s\n", rc_last_error());
        return 5;
    }
    rc_buf bufs[RC_MAX_RANKS];
    for (int r = 0; r < R; ++r) describe(&bufs[r], send[r], recv[r], N, RC_SUM);
    if (rc_all_reduce(bufs, NULL) != RC_OK) {
        fprintf(stderr, "all_reduce: %s\n", rc_last_error());
        return 6;
    }
    for (int r = 0; r < R; ++r) describe(&bufs[r], send[r], shard[r], N, RC_MAX);
    if (rc_reduce_scatter(bufs, NULL) != RC_OK) {
        fprintf(stderr, "reduce_scatter: %s\n", rc_last_error());
        return 7;
    }
    /* a mismatch is reported before anything is enqueued */
    bufs[R - 1].dims[0] = N - 1;
    if (R > 1 && (rc_reduce_scatter(bufs, NULL) != RC_ERR_SHAPE_MISMATCH || rc_last_error()[0] == '\0')) return 8;
    CHECK_HIP(hipDeviceSynchronize());

    f = fopen(argv[4], "wb");
    if (!f) return 9;
    CHECK_HIP(hipMemcpy(host, recv[0], bytes, hipMemcpyDeviceToHost));
    fwrite(host, bytes, 1, f);
    for (int r = 0; r < R; ++r) {
        CHECK_HIP(hipMemcpy(host, shard[r], bytes / R, hipMemcpyDeviceToHost));
        fwrite(host, bytes / R, 1, f);
    }
    fclose(f);
    if (rc_finish() != RC_OK) return 11;
    for (int r = 0; r < R; ++r) {
        hipFree(send[r]);
        hipFree(recv[r]);
        hipFree(shard[r]);
    }
    free(host);
    printf("c_client: ok\n");
    return 0;
}
