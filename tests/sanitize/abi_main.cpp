// Host sanitizer driver for the C ABI (test infrastructure): calls every entry point of include/kda.h
// with rejected arguments of every kind and checks the documented status; on a host without a GPU it
// also calls them with valid arguments and expects KDA_ERROR_NO_DEVICE (with a GPU it skips those: the
// fake pointers would be launched on). Built by tests/test_sanitizers_cpu.py with the library sources
// and AddressSanitizer on the host code only, so an out-of-bounds or invalid access in the validation,
// the workspace sizing or the status strings ends the run with a report.
#include "../../include/kda.h"

#include <hip/hip_runtime.h>
#include <stdio.h>
#include <string.h>

static int fails = 0;
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); ++fails; } } while (0)

static char *const A = reinterpret_cast<char *>(1 << 20);  // 16-byte aligned, never dereferenced

static kda_status_t fwd(const void *q, const void *o, void *ws, size_t wsb, int64_t T, int32_t K, int32_t chunk,
                        kda_dtype_t io, kda_operands_t ops, const int32_t *cu, int32_t N) {
    return kda_chunk_fwd(q, A, A, A, A, nullptr, nullptr, cu, 1, T, 2, K, 32, N, chunk, io, KDA_GATE_LOG_DECAY,
                         KDA_QK_AS_GIVEN, KDA_CONV_NONE, nullptr, ops, io, const_cast<void *>(o), (float *)A, ws, wsb,
                         nullptr);
}

int main() {
    int ndev = 0;
    const bool device = hipGetDeviceCount(&ndev) == hipSuccess && ndev > 0;
    (void)hipGetLastError();
    CHECK(kda_abi_version() == 11);
    for (int s = -1; s < 8; ++s) CHECK(strlen(kda_status_string((kda_status_t)s)) > 0);
    // workspace queries over a sweep of sizes and options (valid and not)
    const int64_t Ts[] = {0, 1, 15, 16, 17, 4096, (int64_t)1 << 40};
    const int32_t dims[] = {16, 32, 64, 96, 128};
    for (int64_t T : Ts)
        for (int32_t K : dims)
            for (int32_t V : dims)
                for (int chunk : {16, 32, 64})
                    for (int io = 0; io < 3; ++io)
                        for (int ops = 0; ops < 3; ++ops) {
                            const size_t a = kda_chunk_fwd_workspace_bytes(1, T, 3, K, V, 2, chunk, (kda_dtype_t)io,
                                                                           KDA_CONV_NONE, (kda_operands_t)ops);
                            const size_t b = kda_chunk_prep_workspace_bytes(1, T, 3, K, V, 2, chunk, (kda_dtype_t)io,
                                                                            KDA_CONV_SHORT4, (kda_operands_t)ops);
                            CHECK(a < ((size_t)1 << 62) && b < ((size_t)1 << 62));
                        }
    CHECK(kda_chunk_bwd_workspace_bytes(1, 64, 2, 32, 32, 1, KDA_QK_AS_GIVEN, KDA_CONV_NONE) > 0);
    CHECK(kda_chunk_bwd_workspace_bytes(1, 64, 2, 32, 32, 1, KDA_QK_L2NORM, KDA_CONV_SHORT4_SILU) >
          kda_chunk_bwd_workspace_bytes(1, 64, 2, 32, 32, 1, KDA_QK_AS_GIVEN, KDA_CONV_NONE));
    CHECK(kda_chunk_bwd_workspace_bytes(2, 64, 2, 48, 32, 2, KDA_QK_AS_GIVEN, KDA_CONV_NONE) == 0);
    CHECK(kda_chunk_bwd_workspace_bytes(1, 64, 2, 32, 32, 1, KDA_QK_AS_GIVEN, (kda_conv_t)3) == 0);
    // the backward in segments: a multiple of 32 tokens, no convolution, below one call's workspace
    CHECK(kda_chunk_bwd_segmented_workspace_bytes(1, 4096, 2, 32, 32, 1, KDA_QK_AS_GIVEN, KDA_CONV_NONE, 256) > 0);
    CHECK(kda_chunk_bwd_segmented_workspace_bytes(1, 4096, 2, 32, 32, 1, KDA_QK_AS_GIVEN, KDA_CONV_NONE, 256) <
          kda_chunk_bwd_workspace_bytes(1, 4096, 2, 32, 32, 1, KDA_QK_AS_GIVEN, KDA_CONV_NONE));
    CHECK(kda_chunk_bwd_segmented_workspace_bytes(1, 4096, 2, 32, 32, 1, KDA_QK_AS_GIVEN, KDA_CONV_NONE, 48) == 0);
    CHECK(kda_chunk_bwd_segmented_workspace_bytes(1, 4096, 2, 32, 32, 1, KDA_QK_AS_GIVEN, KDA_CONV_SHORT4, 256) == 0);
    // prefill: rejected arguments
    CHECK(fwd(nullptr, A, A, 1 << 30, 64, 32, 16, KDA_DTYPE_BF16, KDA_OPERANDS_BF16, nullptr, 1) == KDA_ERROR_INVALID_VALUE);
    CHECK(fwd(A + 8, A, A, 1 << 30, 64, 32, 16, KDA_DTYPE_BF16, KDA_OPERANDS_BF16, nullptr, 1) == KDA_ERROR_INVALID_VALUE);
    CHECK(fwd(A, A, A, 1 << 30, 64, 48, 16, KDA_DTYPE_BF16, KDA_OPERANDS_BF16, nullptr, 1) == KDA_ERROR_NOT_SUPPORTED);
    CHECK(fwd(A, A, A, 1 << 30, 64, 32, 64, KDA_DTYPE_BF16, KDA_OPERANDS_FP16, nullptr, 1) == KDA_ERROR_NOT_SUPPORTED);
    CHECK(fwd(A, A, A, 1 << 30, 64, 32, 16, KDA_DTYPE_BF16, (kda_operands_t)7, nullptr, 1) == KDA_ERROR_INVALID_VALUE);
    CHECK(fwd(A, A, A, 10, 64, 32, 64, KDA_DTYPE_BF16, KDA_OPERANDS_BF16, nullptr, 1) == KDA_ERROR_WORKSPACE_TOO_SMALL);
    CHECK(fwd(A, A, nullptr, 1 << 30, 64, 32, 16, KDA_DTYPE_BF16, KDA_OPERANDS_BF16, nullptr, 1) ==
          KDA_ERROR_WORKSPACE_TOO_SMALL);
    CHECK(fwd(A, A, A, 1 << 30, (int64_t)1 << 60, 32, 16, KDA_DTYPE_BF16, KDA_OPERANDS_BF16, nullptr, 1) ==
          KDA_ERROR_INVALID_VALUE);
    CHECK(fwd(A, A, A, 1 << 30, 64, 32, 16, KDA_DTYPE_BF16, KDA_OPERANDS_BF16, (const int32_t *)(A + 2), 3) ==
          KDA_ERROR_INVALID_VALUE);
    CHECK(kda_chunk_prep(A, A, A, A, nullptr, 1, 64, 2, 32, 32, 1, 16, KDA_DTYPE_FP32, KDA_GATE_LOG_DECAY,
                         KDA_QK_AS_GIVEN, KDA_CONV_NONE, nullptr, KDA_OPERANDS_FP16, A, 1 << 30, nullptr) ==
          KDA_ERROR_NOT_SUPPORTED);
    CHECK(kda_chunk_state(A, nullptr, (float *)A, nullptr, 1, 64, 2, 32, 32, 1, 16, KDA_DTYPE_BF16, KDA_CONV_NONE,
                          nullptr, KDA_DTYPE_BF16, A, (float *)A, A, 1 << 30, nullptr) == KDA_ERROR_INVALID_VALUE);
    CHECK(kda_decode_step(A, A, A, A, A, nullptr, (float *)A, A, 4, 2, 32, 96, KDA_DTYPE_BF16, KDA_GATE_LOG_DECAY,
                          KDA_QK_AS_GIVEN, KDA_CONV_NONE, nullptr, nullptr, KDA_DTYPE_BF16, nullptr) ==
          KDA_ERROR_NOT_SUPPORTED);
    CHECK(kda_decode_step(A, A, A, A, A, nullptr, nullptr, A, 4, 2, 32, 32, KDA_DTYPE_BF16, KDA_GATE_LOG_DECAY,
                          KDA_QK_AS_GIVEN, KDA_CONV_NONE, nullptr, nullptr, KDA_DTYPE_BF16, nullptr) ==
          KDA_ERROR_INVALID_VALUE);
    float *f = (float *)A;
    CHECK(kda_chunk_bwd(A, A, A, A, A, nullptr, nullptr, nullptr, nullptr, nullptr, 1, 64, 2, 32, 32, 1,
                        KDA_DTYPE_BF16, KDA_GATE_LOG_DECAY, KDA_QK_AS_GIVEN, KDA_CONV_NONE, nullptr, f + 4096,
                        f + 8192, f + 12288, f + 16384, f + 20480, nullptr, nullptr, nullptr, A, 1 << 30,
                        nullptr) == KDA_ERROR_INVALID_VALUE);  // d_o missing
    int32_t err = 0;
    CHECK(kda_workspace_status(nullptr, 1024, &err, nullptr) == KDA_ERROR_INVALID_VALUE);
    CHECK(kda_workspace_status(A, 100, &err, nullptr) == KDA_ERROR_WORKSPACE_TOO_SMALL);
    if (!device) {  // valid arguments reach the device check
        CHECK(fwd(A, A, A, 1 << 30, 64, 32, 16, KDA_DTYPE_BF16, KDA_OPERANDS_BF16, nullptr, 1) == KDA_ERROR_NO_DEVICE);
        CHECK(fwd(A, A, A, 1 << 30, 64, 32, 16, KDA_DTYPE_BF16, KDA_OPERANDS_FP16, nullptr, 1) == KDA_ERROR_NO_DEVICE);
        CHECK(fwd(A, A, A, 1 << 30, 64, 32, 64, KDA_DTYPE_FP32, KDA_OPERANDS_BF16, (const int32_t *)A, 1) ==
              KDA_ERROR_NO_DEVICE);
        CHECK(kda_workspace_status(A, 1024, &err, nullptr) == KDA_ERROR_NO_DEVICE);
    }
    if (fails) {
        fprintf(stderr, "%d checks failed\n", fails);
        return 1;
    }
    printf("abi sanitizer driver: all checks passed (%s)\n", device ? "device present: valid calls skipped" : "no device");
    return 0;
}
