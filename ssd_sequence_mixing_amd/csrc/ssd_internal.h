// Internal interfaces between the C ABI host code and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssd.h"

namespace ssd {

// Everything the forward launch sequence needs, validated by the caller.
struct FwdArgs {
    const void *X, *dt, *B, *C;
    const float *A, *D;
    void *Y;
    float *final_state;        // may be null
    const float *init;         // (batch, H, P, N) initial state, or null for zero
    int64_t batch, T, H, P, N, G, Q, nC, Tpad;
    ssd_dtype dtype;
    float *cs2, *dtf;          // workspace: (batch, H, Tpad) each
    void *Gbuf;                // workspace: (batch, G, tiles, 64, 64) in the storage type
    int64_t g_bytes;
};

// Kernel arguments of the chunk walk (passed by value).
struct PrepArgs {
    const void *dt, *B, *C;
    const float *A;
    void *Gbuf;
    float *cs2, *dtf;
    int T, H, G, nC, Tpad, ntiles, cb_blocks;
    uint32_t g_bytes;
};

struct WalkArgs {
    const void *X, *B, *C;
    void *Y;
    const void *Gbuf;
    const float *cs2, *dtf, *D;
    const float *init;         // (batch, H, P, N) or null for a zero state
    float *final_state;        // may be null
    int batch, T, H, G, nC, Tpad;
    int P, NS;                 // head dimension, and the work-groups sharing each head's P columns
    uint32_t g_bytes;
};

struct StepArgs {
    float *state;
    const void *x, *dt, *B, *C;
    const float *A, *D;
    void *y;
    int64_t batch, H, P, N, G;
    ssd_dtype dtype;
};

// Phase 1: chunk-local log-decay prefix sums and C B^T tiles into the workspace.
ssd_status launch_prepare(const FwdArgs &f, hipStream_t s);
// Phase 2: the chunk walk (reads the prepared workspace).
ssd_status launch_walk(const FwdArgs &f, hipStream_t s);
// LDS bytes one chunk-walk work-group needs, or -1 if there is no kernel.
int fwd_lds_bytes(ssd_dtype dt, int64_t Q, int64_t P, int64_t N);
ssd_status launch_step(const StepArgs &a, hipStream_t s);

constexpr int kMaxLds = 160 * 1024;

// Launches a kernel and returns the status of that launch itself (not an
// error some earlier, unrelated runtime call may have left pending).
template <typename T> struct ident { using type = T; };
template <typename... Args>
inline hipError_t launch(void (*kernel)(Args...), dim3 grid, dim3 block, hipStream_t s,
                         typename ident<Args>::type... args) {
    void *argv[] = {(void *)&args..., nullptr};
    return hipLaunchKernel((const void *)kernel, grid, block, argv, 0, s);
}

}  // namespace ssd
