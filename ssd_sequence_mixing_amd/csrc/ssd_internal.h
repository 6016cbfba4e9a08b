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
    const int *cu;             // packed variable-length batch: (batch + 1) cumulative lengths, or null
    int64_t total;             // tokens in the packed batch (cu != null)
    const float *dt_bias;      // fused prologue: dt = [softplus](dt + dt_bias[h]); null = no bias
    int softplus;
    const void *z;             // fused epilogue: Y *= silu(z), z shaped like X; null = no gate
    const float *conv_w;       // fused input activation: X <- silu(causal conv of X), taps (H P, 4); null = none
    const float *conv_b;       // its bias (H P), or null (zero)
    ssd_dtype dtype;
    float *cs2, *dtf;          // workspace: (batch, H, Tpad) each
    void *Gbuf;                // workspace: (batch, G, Tpad / tt, tt, tt) in the storage type
    int64_t g_bytes;
    int ns, tt;                // walk plan: work-groups per head, tile tokens
    int S, cps;                // walk plan: sequence segments, chunks per segment
    int segk;                  // walk plan: pre-pass sub-segments per segment (1 or 2)
    float *seg;                // workspace: (batch, H, (S - 1) segk, P, N) fp32 (sub-)segment states
    bool no_g;                 // the caller reads no C B^T tiles (the backward): prepare skips them
};

// How the walk covers a shape: ns work-groups per head (P / ns columns each)
// and tiles of tt tokens.
struct WalkPlan {
    int ns, tt;   // work-groups per head (P / ns columns each), tile tokens
    int S, cps;   // sequence segments walked in parallel, chunks per segment
    int segk;     // sub-segments per segment in the end-state pre-pass (1 or 2)
};
// Fills the plan; -1 if no kernel covers the shape.
// segments: whether the sequence may be split (not for packed batches).
int fwd_plan(ssd_dtype dt, int64_t batch, int64_t H, int64_t P, int64_t N, int64_t Q, int64_t nC,
             bool segments, WalkPlan *plan);

// Kernel arguments of the chunk walk (passed by value).
struct PrepArgs {
    const void *dt, *B, *C;
    const float *A;
    void *Gbuf;
    float *cs2, *dtf;
    int T, H, G, nC, Tpad, ntiles, cb_blocks;
    const int *cu;             // see FwdArgs
    int total;
    const float *dt_bias;      // see FwdArgs
    int softplus;
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
    int S, SL, cps;            // sequence segments, segments in this launch, chunks per segment
    int segk;                  // seg holds (S - 1) segk sub-segment states per (batch, head); segment
                               // s > 0 enters with the one in slot s segk - 1
    float *seg;                // (batch, H, (S - 1) segk, P, N) segment states (S > 1)
    const int *cu;             // see FwdArgs
    int total;
    const void *z;             // see FwdArgs
    const float *conv_w, *conv_b;  // see FwdArgs
    uint32_t g_bytes;
};

struct StepArgs {
    float *state;
    const void *x, *dt, *B, *C;
    const float *A, *D;
    void *y;
    const float *dt_bias;      // see FwdArgs
    int softplus;
    const void *z;             // (batch, H, P) like x, or null
    void *conv_state;          // input convolution: (batch, H P, 3) raw inputs, oldest first, storage type
    const float *conv_w;       // its taps (H P, 4), or null for no convolution
    const float *conv_b;       // its bias (H P), or null (zero)
    int64_t batch, H, P, N, G;
    ssd_dtype dtype;
};

// Backward pass (ssd_bwd.hip).
struct StatePassArgs {          // k_state_pass
    const void *U, *V;          // X / dY (batch, T, H, P) and B / C (batch, T, G, N)
    const float *cs2, *dtf;     // log-decay workspace (batch, H, Tpad)
    const float *init;          // state before the first tile walked (fp32), or null
    void *Sst;                  // (batch, H, ntiles, P, N) storage type: the state entering each tile
    float *out;                 // state after the last tile walked (fp32), or null
    int H, G, T, Tpad, ntiles, tpc;  // tpc: 64-token tiles per chunk
};

struct BwdTileArgs {            // k_bwd_tile
    const void *X, *dY, *B, *C, *dt;
    const float *D;
    const void *Hst, *Est;      // entering states / arriving adjoints per tile
    const float *cs2, *dtf;
    void *dX;
    float *rbuf, *qbuf, *xybuf; // per (batch, head, token): x.v, dy.y' - dt x.v, dy.x
    float *dBp, *dCp;           // (batch, Tpad, nblk, G, N) partial sums over head blocks
    void *dB, *dC;              // one head block per group: dB, dC (storage type) written directly
    float *lamb;                // (batch, H, ntiles, NS, 8) per-wavefront shares of
                                // <E_tile, state after the tile>
    float *dXp;                 // NS > 1: (NS, batch, T, H, P) fp32 parts of dX
    size_t tok_stride;          // elements between the n slices' rbuf / qbuf parts
    size_t dx_stride;           // elements between the n slices' dXp parts
    int H, G, T, Tpad, ntiles, tpc, nblk;
};

struct BwdFinArgs {             // k_bwd_fin
    const float *qbuf, *rbuf, *xybuf, *lamb;
    size_t tok_stride;          // elements between the n slices' rbuf / qbuf parts
    int ns;                     // n slices of k_bwd_tile
    const void *dt;
    const float *A;
    void *ddt;
    float *dApart, *dDpart;     // (batch, H, ntiles) shares of dA, dD
    int batch, T, Tpad, H, ntiles;
};

struct BwdArgs {
    FwdArgs f;                  // forward inputs and the prepared log-decays
    const void *dY;
    const float *dF;            // gradient of the final state, or null
    void *dX, *ddt, *dB, *dC;
    float *dA, *dD, *dinit;     // dinit may be null
    void *Hst, *Est;            // workspace, storage type
    float *lamb, *dApart, *dDpart;                  // workspace, fp32, (batch, H, ntiles) each
    float *rbuf, *qbuf, *xybuf, *dBp, *dCp;          // workspace, fp32 (rbuf, qbuf: one part per n slice)
    float *dXp;                 // workspace, fp32, n slices > 1 only
    int nblk;                   // head blocks per group
};

// Whether a backward kernel covers (dtype, P, N).
bool bwd_supported(ssd_dtype dt, int64_t P, int64_t N);
// Work-groups k_bwd_tile splits the n axis over (1 where it fits one CU's LDS).
int bwd_nslices(ssd_dtype dt, int64_t P, int64_t N);
// The backward launches (after launch_prepare on the same FwdArgs).
ssd_status launch_bwd(const BwdArgs &w, hipStream_t s);

// Phase 1: chunk-local log-decay prefix sums and (unless f.no_g) C B^T tiles
// into the workspace.
ssd_status launch_prepare(const FwdArgs &f, hipStream_t s);
// Whether the walk with the fused input convolution fits LDS for a column slice.
bool walk_conv_fits(ssd_dtype dt, int64_t Q, int64_t PW, int64_t N);
// Phase 2: the chunk walk (reads the prepared workspace).
ssd_status launch_walk(const FwdArgs &f, hipStream_t s);
// The walk with the fused input convolution (f.conv_w set; ssd_walk_conv.hip).
ssd_status launch_walk_conv(const FwdArgs &f, hipStream_t s);
// The walk with the state kept in the wavefronts that update it
// (ssd_walk_rs.hip): bf16 storage, 64-token tiles, column slices of 32 or 64
// and N of 64 or 128, with or without the gate and the input convolution.
bool walk_rs_supported(const FwdArgs &f);
ssd_status launch_walk_rs(const FwdArgs &f, hipStream_t s);
// The end states of a split sequence's segments 0 .. S - 2 (each entered with
// zero, the first with f.init) into f.seg (ssd_seg_states.hip).
ssd_status launch_seg_states(const FwdArgs &f, hipStream_t s);
// One recurrent decode step.
ssd_status launch_step(const StepArgs &a, hipStream_t s);

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
