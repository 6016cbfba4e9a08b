// C ABI of libssd: argument checks, workspace layout and launch order.
// Every check runs on the host before anything is enqueued.
#include <stddef.h>
#include <stdint.h>

#include <initializer_list>
#include <mutex>

#include "ssd_common.h"
#include "ssd_internal.h"

namespace {

using ssd::FwdArgs;

constexpr int64_t kTwoGiB = (int64_t)1 << 31;

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int64_t esize(ssd_dtype d) { return d == SSD_BF16 ? 2 : 4; }

bool valid_dtype(int d) { return d == SSD_F32 || d == SSD_BF16; }

bool in_set(int64_t v, std::initializer_list<int64_t> s) {
    for (int64_t x : s)
        if (v == x) return true;
    return false;
}

int64_t align256(int64_t v) { return (v + 255) & ~(int64_t)255; }

struct FwdLayout {
    int64_t nC, Tpad, cs_bytes, g_bytes, seg_bytes, total;
    ssd::WalkPlan plan;
};

// Shape checks shared by the workspace query and the forward entry points.
// For a packed variable-length batch, batch is the number of sequences,
// seqlen the longest one, and total the tokens in the packed tensors.
ssd_status check_fwd_shape(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                           int64_t dstate, int64_t ngroups, int64_t chunk, int dtype,
                           FwdLayout *lay, bool varlen = false, int64_t total = 0) {
    if (!valid_dtype(dtype)) return SSD_ERR_UNSUPPORTED;
    if (batch < 0 || seqlen < 0 || nheads <= 0 || headdim <= 0 || dstate <= 0 || ngroups <= 0)
        return SSD_ERR_SHAPE;
    if (nheads % ngroups != 0) return SSD_ERR_SHAPE;
    if (!in_set(chunk, {64, 128, 256})) return SSD_ERR_UNSUPPORTED;
    if (!in_set(headdim, {16, 32, 64, 128}) || !in_set(dstate, {16, 32, 64, 128, 256}))
        return SSD_ERR_UNSUPPORTED;
    if (seqlen > kTwoGiB || nheads > 65536) return SSD_ERR_UNSUPPORTED;
    if (total < 0 || total > kTwoGiB) return SSD_ERR_SHAPE;
    // grid: batch x heads x column slices (<= 4) x segments (<= 4) work-groups.
    // Checked before any size product, which this bound keeps inside int64.
    if (batch > (int64_t)INT32_MAX / 16 || batch * nheads > (int64_t)INT32_MAX / 16) return SSD_ERR_UNSUPPORTED;
    if (ssd::fwd_plan((ssd_dtype)dtype, batch, nheads, headdim, dstate, chunk, (seqlen + chunk - 1) / chunk,
                      !varlen, &lay->plan) != 0)
        return SSD_ERR_UNSUPPORTED;
    const int64_t es = esize((ssd_dtype)dtype);
    // 32-bit buffer offsets: every per-batch slab, padded to whole chunks, and
    // the C B^T buffer stay under 2 GiB, so an offset past the end of a slab
    // (a token past T) can never wrap back into range
    const int64_t nC = (seqlen + chunk - 1) / chunk;
    const int64_t Tpad = nC * chunk;
    if (Tpad * nheads * headdim * es >= kTwoGiB) return SSD_ERR_UNSUPPORTED;
    if (Tpad * ngroups * dstate * es >= kTwoGiB) return SSD_ERR_UNSUPPORTED;
    if (Tpad * nheads * es >= kTwoGiB) return SSD_ERR_UNSUPPORTED;
    if (total * nheads * headdim * es >= kTwoGiB || total * ngroups * dstate * es >= kTwoGiB)
        return SSD_ERR_UNSUPPORTED;
    lay->nC = nC;
    lay->Tpad = Tpad;
    lay->cs_bytes = align256(batch * nheads * Tpad * 4);
    lay->g_bytes = align256(batch * ngroups * Tpad * lay->plan.tt * es);  // one tt x tt tile per tt tokens
    if (lay->g_bytes >= kTwoGiB) return SSD_ERR_UNSUPPORTED;
    lay->seg_bytes = align256(batch * nheads * (lay->plan.S - 1) * lay->plan.segk * headdim * dstate * 4);
    lay->total = (batch == 0 || seqlen == 0) ? 0 : 2 * lay->cs_bytes + lay->g_bytes + lay->seg_bytes;
    return SSD_OK;
}

ssd_status check_workspace(const FwdLayout &lay, const void *workspace, size_t workspace_bytes) {
    if (lay.total > 0) {
        if (!workspace || workspace_bytes < (size_t)lay.total) return SSD_ERR_WORKSPACE;
        if (((uintptr_t)workspace & 255u) != 0) return SSD_ERR_ALIGN;
    }
    return SSD_OK;
}

FwdArgs make_args(const FwdLayout &lay, int64_t batch, int64_t seqlen, int64_t nheads,
                  int64_t headdim, int64_t dstate, int64_t ngroups, int64_t chunk, ssd_dtype dtype,
                  const void *workspace) {
    FwdArgs f = {};
    f.batch = batch; f.T = seqlen; f.H = nheads; f.P = headdim; f.N = dstate; f.G = ngroups;
    f.Q = chunk; f.nC = lay.nC; f.Tpad = lay.Tpad; f.dtype = dtype;
    char *ws = static_cast<char *>(const_cast<void *>(workspace));
    f.cs2 = reinterpret_cast<float *>(ws);
    f.dtf = reinterpret_cast<float *>(ws + lay.cs_bytes);
    f.Gbuf = ws + 2 * lay.cs_bytes;
    f.g_bytes = lay.g_bytes;
    f.ns = lay.plan.ns;
    f.tt = lay.plan.tt;
    f.S = lay.plan.S;
    f.cps = lay.plan.cps;
    f.segk = lay.plan.segk;
    f.seg = reinterpret_cast<float *>(ws + 2 * lay.cs_bytes + lay.g_bytes);
    return f;
}

__global__ void k_fill_state(float *dst, const float *src, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.f;
}

// Empty sequence: the final state is the initial state (zero when none).
ssd_status empty_final_state(float *final_state, const float *init, int64_t n, hipStream_t s) {
    if (!final_state || n == 0) return SSD_OK;
    return ssd::launch(k_fill_state, dim3((unsigned)((n + 255) / 256)), dim3(256), s, final_state,
                       init, n) == hipSuccess
               ? SSD_OK
               : SSD_ERR_HIP;
}

// Backward workspace: the forward's (log-decays, C B^T tiles) followed by the
// per-tile states and adjoints, Lambda at every tile end and each tile's
// shares of dA and dD, three per-token scalars and the head blocks' partial
// dB / dC.
struct BwdLayout {
    FwdLayout fl;
    int nblk, ns;  // head blocks per group, n slices of k_bwd_tile
    int64_t ntiles, st_bytes, lamb_bytes, share_bytes, tok_bytes, rq_bytes, part_bytes, dxp_bytes, total;
};

// Head blocks per group: the fewest (a divisor of the group's head count)
// that give one work-group per CU (256 on this part; k_bwd_tile takes a CU's
// LDS). Fewer blocks mean fewer dB / dC partials and less per-block staging
// (at the 1.3B shape two blocks of 32 heads beat four of 16 by ~10 us).
int bwd_blocks(int64_t batch, int64_t ntiles, int64_t G, int64_t HG) {
    for (int64_t k = 1; k <= HG; ++k)
        if (HG % k == 0 && batch * ntiles * G * k >= 256) return (int)k;
    return (int)HG;
}

ssd_status check_bwd_shape(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate,
                           int64_t ngroups, int64_t chunk, int dtype, BwdLayout *lay) {
    ssd_status st = check_fwd_shape(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype, &lay->fl);
    if (st != SSD_OK) return st;
    if (!ssd::bwd_supported((ssd_dtype)dtype, headdim, dstate)) return SSD_ERR_UNSUPPORTED;
    const int64_t es = esize((ssd_dtype)dtype);
    const int64_t Tpad = lay->fl.Tpad;
    lay->ntiles = Tpad / 64;
    // (batch x heads is bounded by the forward check, so this product fits)
    lay->ns = ssd::bwd_nslices((ssd_dtype)dtype, headdim, dstate);
    // k_bwd_tile's grid (batch x tiles x groups x head blocks x n slices) is at most this
    if (batch * nheads * lay->ntiles * lay->ns > (int64_t)INT32_MAX) return SSD_ERR_UNSUPPORTED;
    lay->nblk = bwd_blocks(batch, lay->ntiles, ngroups, nheads / ngroups);
    const int64_t ns = lay->ns;
    lay->st_bytes = align256(batch * nheads * lay->ntiles * headdim * dstate * es);
    lay->lamb_bytes = align256(batch * nheads * lay->ntiles * 4);
    lay->share_bytes = align256(batch * nheads * lay->ntiles * ns * 8 * 4);  // Lambda shares, 8 per tile and slice
    lay->tok_bytes = align256(batch * nheads * Tpad * 4);
    lay->rq_bytes = align256(ns * batch * nheads * Tpad * 4);  // x.v and the dy.y' scalar, one part per slice
    lay->part_bytes = align256(batch * Tpad * lay->nblk * ngroups * dstate * 4);
    lay->dxp_bytes = ns > 1 ? align256(ns * batch * seqlen * nheads * headdim * 4) : 0;
    const int64_t fwd = 2 * lay->fl.cs_bytes + lay->fl.g_bytes + lay->fl.seg_bytes;
    lay->total = (batch == 0 || seqlen == 0)
                     ? 0
                     : fwd + 2 * lay->st_bytes + lay->share_bytes + 2 * lay->lamb_bytes + 2 * lay->rq_bytes +
                           lay->tok_bytes + 2 * lay->part_bytes + lay->dxp_bytes;
    return SSD_OK;
}

__global__ void k_zero(float *p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0.f;
}

// The forward's workspace for callers that cannot allocate
// (ssd_chunk_scan_fwd_noalloc): one array per GPU, loaded with the library's
// code and held until the process ends. Host code never passes the array's
// name to a kernel (on the host it is only a stand-in for the symbol); it
// passes the device address hipGetSymbolAddress returns for the current GPU.
static __device__ __align__(256) unsigned char scratch[SSD_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each GPU, once looked up

// The address of the current GPU's copy of `scratch`, looked up once per GPU.
ssd_status scratch_of_current_device(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SSD_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SSD_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SSD_OK;
}

// The forward with every option (ssd_chunk_scan_fwd_fused's arguments). With
// use_scratch the workspace arguments are ignored and the current GPU's
// `scratch` serves instead; problems needing more return SSD_ERR_TOO_LARGE.
ssd_status fwd_impl(const void *X, const float *conv_w, const float *conv_b, const void *dt,
                    const float *dt_bias, int dt_softplus, const float *A, const void *B, const void *C,
                    const float *D, const void *z, int64_t chunk, void *Y, float *final_state, int64_t batch,
                    int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate, int64_t ngroups,
                    ssd_dtype dtype, void *workspace, size_t workspace_bytes, bool use_scratch, void *stream) {
    if (dt_softplus < 0 || dt_softplus > 2) return SSD_ERR_UNSUPPORTED;
    if (!conv_w && conv_b) return SSD_ERR_NULL;
    if (!aligned16(conv_w) || ((uintptr_t)conv_b & 3u) != 0) return SSD_ERR_ALIGN;
    const bool empty = (batch == 0 || seqlen == 0);
    // an empty problem reads no input, so its input pointers may be NULL
    if (!empty && (!X || !dt || !A || !B || !C || !D || !Y)) return SSD_ERR_NULL;
    FwdLayout lay;
    ssd_status st =
        check_fwd_shape(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, (int)dtype, &lay);
    if (st != SSD_OK) return st;
    if (conv_w && !ssd::walk_conv_fits(dtype, chunk, headdim / lay.plan.ns, dstate)) return SSD_ERR_UNSUPPORTED;
    if (!aligned16(X) || !aligned16(dt) || !aligned16(A) || !aligned16(B) || !aligned16(C) ||
        !aligned16(D) || !aligned16(Y) || !aligned16(final_state) || !aligned16(dt_bias) || !aligned16(z))
        return SSD_ERR_ALIGN;
    if (use_scratch) {
        if ((size_t)lay.total > (size_t)SSD_NOALLOC_SCRATCH_BYTES) return SSD_ERR_TOO_LARGE;
        workspace = nullptr;
        workspace_bytes = SSD_NOALLOC_SCRATCH_BYTES;
        if (lay.total > 0 && (st = scratch_of_current_device(&workspace)) != SSD_OK) return st;
    }
    if ((st = check_workspace(lay, workspace, workspace_bytes)) != SSD_OK) return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (batch == 0) return SSD_OK;
    if (seqlen == 0)
        return empty_final_state(final_state, nullptr, batch * nheads * headdim * dstate, s);
    FwdArgs f = make_args(lay, batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype,
                          workspace);
    f.X = X; f.dt = dt; f.A = A; f.B = B; f.C = C; f.D = D; f.Y = Y; f.final_state = final_state;
    f.dt_bias = dt_bias; f.softplus = dt_softplus; f.z = z;
    f.conv_w = conv_w; f.conv_b = conv_b;
    if ((st = ssd::launch_prepare(f, s)) != SSD_OK) return st;
    return ssd::launch_walk(f, s);
}

// The decode step with every option (defined after the entry points).
ssd_status step_impl(float *state, void *conv_state, const void *x, const float *conv_w, const float *conv_b,
                     const void *dt, const float *dt_bias, int dt_softplus, const float *A, const void *B,
                     const void *C, const float *D, const void *z, void *y, int64_t batch, int64_t nheads,
                     int64_t headdim, int64_t dstate, int64_t ngroups, ssd_dtype dtype, void *stream);

}  // namespace

extern "C" {

const char *ssd_status_string(int status) {
    switch (status) {
        case SSD_OK: return "SSD_OK";
        case SSD_ERR_NULL: return "SSD_ERR_NULL: a required pointer is NULL";
        case SSD_ERR_SHAPE: return "SSD_ERR_SHAPE: invalid dimensions";
        case SSD_ERR_UNSUPPORTED: return "SSD_ERR_UNSUPPORTED: no kernel for this configuration";
        case SSD_ERR_WORKSPACE: return "SSD_ERR_WORKSPACE: workspace missing or too small";
        case SSD_ERR_ALIGN: return "SSD_ERR_ALIGN: pointer not 16-byte aligned";
        case SSD_ERR_HIP: return "SSD_ERR_HIP: HIP runtime error at launch";
        case SSD_ERR_TOO_LARGE:
            return "SSD_ERR_TOO_LARGE: the problem needs more workspace than the library's static scratch holds";
    }
    return "SSD_ERR_UNKNOWN";
}

size_t ssd_chunk_scan_fwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t nheads,
                                          int64_t headdim, int64_t dstate, int64_t ngroups,
                                          int64_t chunk, ssd_dtype dtype) {
    FwdLayout lay;
    if (check_fwd_shape(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, (int)dtype, &lay) !=
        SSD_OK)
        return (size_t)-1;
    return (size_t)lay.total;
}

ssd_status ssd_chunk_scan_prepare(const void *dt, const float *A, const void *B, const void *C,
                                  int64_t chunk, int64_t batch, int64_t seqlen, int64_t nheads,
                                  int64_t headdim, int64_t dstate, int64_t ngroups, ssd_dtype dtype,
                                  void *workspace, size_t workspace_bytes, void *stream) {
    const bool empty = (batch == 0 || seqlen == 0);
    if (!empty && (!dt || !A || !B || !C)) return SSD_ERR_NULL;
    FwdLayout lay;
    ssd_status st =
        check_fwd_shape(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, (int)dtype, &lay);
    if (st != SSD_OK) return st;
    if (!aligned16(dt) || !aligned16(A) || !aligned16(B) || !aligned16(C)) return SSD_ERR_ALIGN;
    if ((st = check_workspace(lay, workspace, workspace_bytes)) != SSD_OK) return st;
    if (empty) return SSD_OK;
    FwdArgs f = make_args(lay, batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype,
                          workspace);
    f.dt = dt; f.A = A; f.B = B; f.C = C;
    return ssd::launch_prepare(f, reinterpret_cast<hipStream_t>(stream));
}

ssd_status ssd_chunk_scan_walk(const void *X, const void *B, const void *C, const float *D,
                               const float *initial_state, int64_t chunk, void *Y,
                               float *final_state, int64_t batch, int64_t seqlen, int64_t nheads,
                               int64_t headdim, int64_t dstate, int64_t ngroups, ssd_dtype dtype,
                               const void *workspace, size_t workspace_bytes, void *stream) {
    const bool empty = (batch == 0 || seqlen == 0);
    if (!empty && (!X || !B || !C || !D || !Y)) return SSD_ERR_NULL;
    FwdLayout lay;
    ssd_status st =
        check_fwd_shape(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, (int)dtype, &lay);
    if (st != SSD_OK) return st;
    if (!aligned16(X) || !aligned16(B) || !aligned16(C) || !aligned16(D) || !aligned16(Y) ||
        !aligned16(initial_state) || !aligned16(final_state))
        return SSD_ERR_ALIGN;
    if ((st = check_workspace(lay, workspace, workspace_bytes)) != SSD_OK) return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (batch == 0) return SSD_OK;
    if (seqlen == 0)
        return empty_final_state(final_state, initial_state, batch * nheads * headdim * dstate, s);
    FwdArgs f = make_args(lay, batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype,
                          workspace);
    f.X = X; f.B = B; f.C = C; f.D = D; f.Y = Y; f.init = initial_state; f.final_state = final_state;
    return ssd::launch_walk(f, s);
}

ssd_status ssd_chunk_scan_fwd(const void *X, const void *dt, const float *A, const void *B,
                              const void *C, const float *D, int64_t chunk, void *Y,
                              float *final_state, int64_t batch, int64_t seqlen, int64_t nheads,
                              int64_t headdim, int64_t dstate, int64_t ngroups, ssd_dtype dtype,
                              void *workspace, size_t workspace_bytes, void *stream) {
    return ssd_chunk_scan_fwd_gated(X, dt, nullptr, 0, A, B, C, D, nullptr, chunk, Y, final_state, batch,
                                    seqlen, nheads, headdim, dstate, ngroups, dtype, workspace,
                                    workspace_bytes, stream);
}

ssd_status ssd_chunk_scan_fwd_gated(const void *X, const void *dt, const float *dt_bias, int dt_softplus,
                                    const float *A, const void *B, const void *C, const float *D,
                                    const void *z, int64_t chunk, void *Y, float *final_state,
                                    int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                                    int64_t dstate, int64_t ngroups, ssd_dtype dtype, void *workspace,
                                    size_t workspace_bytes, void *stream) {
    return ssd_chunk_scan_fwd_fused(X, nullptr, nullptr, dt, dt_bias, dt_softplus, A, B, C, D, z, chunk, Y,
                                    final_state, batch, seqlen, nheads, headdim, dstate, ngroups, dtype, workspace,
                                    workspace_bytes, stream);
}

ssd_status ssd_chunk_scan_fwd_fused(const void *X, const float *conv_w, const float *conv_b, const void *dt,
                                    const float *dt_bias, int dt_softplus, const float *A, const void *B,
                                    const void *C, const float *D, const void *z, int64_t chunk, void *Y,
                                    float *final_state, int64_t batch, int64_t seqlen, int64_t nheads,
                                    int64_t headdim, int64_t dstate, int64_t ngroups, ssd_dtype dtype,
                                    void *workspace, size_t workspace_bytes, void *stream) {
    return fwd_impl(X, conv_w, conv_b, dt, dt_bias, dt_softplus, A, B, C, D, z, chunk, Y, final_state, batch,
                    seqlen, nheads, headdim, dstate, ngroups, dtype, workspace, workspace_bytes, false, stream);
}

ssd_status ssd_chunk_scan_fwd_noalloc(const void *X, const void *dt, const float *A, const void *B,
                                      const void *C, const float *D, int64_t chunk, void *Y,
                                      float *final_state, int64_t batch, int64_t seqlen, int64_t nheads,
                                      int64_t headdim, int64_t dstate, int64_t ngroups, ssd_dtype dtype,
                                      void *stream) {
    return fwd_impl(X, nullptr, nullptr, dt, nullptr, 0, A, B, C, D, nullptr, chunk, Y, final_state, batch,
                    seqlen, nheads, headdim, dstate, ngroups, dtype, nullptr, 0, true, stream);
}

size_t ssd_chunk_scan_varlen_workspace_bytes(int64_t num_seqs, int64_t max_seqlen, int64_t nheads,
                                             int64_t headdim, int64_t dstate, int64_t ngroups,
                                             int64_t chunk, ssd_dtype dtype) {
    FwdLayout lay;
    if (check_fwd_shape(num_seqs, max_seqlen, nheads, headdim, dstate, ngroups, chunk, (int)dtype, &lay,
                        true) != SSD_OK)
        return (size_t)-1;
    return (size_t)lay.total;
}

ssd_status ssd_chunk_scan_fwd_varlen(const void *X, const void *dt, const float *A, const void *B,
                                     const void *C, const float *D, int64_t chunk,
                                     const int32_t *cu_seqlens, int64_t num_seqs, int64_t max_seqlen,
                                     int64_t total_tokens, const float *initial_state, void *Y,
                                     float *final_state, int64_t nheads, int64_t headdim,
                                     int64_t dstate, int64_t ngroups, ssd_dtype dtype, void *workspace,
                                     size_t workspace_bytes, void *stream) {
    const bool empty = (num_seqs == 0 || max_seqlen == 0 || total_tokens == 0);
    if (num_seqs > 0 && !cu_seqlens) return SSD_ERR_NULL;
    if (!empty && (!X || !dt || !A || !B || !C || !D || !Y)) return SSD_ERR_NULL;
    FwdLayout lay;
    ssd_status st = check_fwd_shape(num_seqs, max_seqlen, nheads, headdim, dstate, ngroups, chunk, (int)dtype,
                                    &lay, true, total_tokens);
    if (st != SSD_OK) return st;
    if (!aligned16(X) || !aligned16(dt) || !aligned16(A) || !aligned16(B) || !aligned16(C) ||
        !aligned16(D) || !aligned16(Y) || !aligned16(initial_state) || !aligned16(final_state))
        return SSD_ERR_ALIGN;
    if ((st = check_workspace(lay, workspace, workspace_bytes)) != SSD_OK) return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (num_seqs == 0) return SSD_OK;
    if (empty)
        return empty_final_state(final_state, initial_state, num_seqs * nheads * headdim * dstate, s);
    FwdArgs f = make_args(lay, num_seqs, max_seqlen, nheads, headdim, dstate, ngroups, chunk, dtype,
                          workspace);
    f.X = X; f.dt = dt; f.A = A; f.B = B; f.C = C; f.D = D; f.Y = Y;
    f.init = initial_state; f.final_state = final_state;
    f.cu = cu_seqlens; f.total = total_tokens;
    if ((st = ssd::launch_prepare(f, s)) != SSD_OK) return st;
    return ssd::launch_walk(f, s);
}

ssd_status ssd_step(float *state, const void *x, const void *dt, const float *A, const void *B,
                    const void *C, const float *D, void *y, int64_t batch, int64_t nheads,
                    int64_t headdim, int64_t dstate, int64_t ngroups, ssd_dtype dtype,
                    void *stream) {
    return ssd_step_gated(state, x, dt, nullptr, 0, A, B, C, D, nullptr, y, batch, nheads, headdim, dstate,
                          ngroups, dtype, stream);
}

ssd_status ssd_step_gated(float *state, const void *x, const void *dt, const float *dt_bias, int dt_softplus,
                          const float *A, const void *B, const void *C, const float *D, const void *z,
                          void *y, int64_t batch, int64_t nheads, int64_t headdim, int64_t dstate,
                          int64_t ngroups, ssd_dtype dtype, void *stream) {
    return step_impl(state, nullptr, x, nullptr, nullptr, dt, dt_bias, dt_softplus, A, B, C, D, z, y, batch,
                     nheads, headdim, dstate, ngroups, dtype, stream);
}

ssd_status ssd_step_fused(float *state, void *conv_state, const void *x, const float *conv_w, const float *conv_b,
                          const void *dt, const float *dt_bias, int dt_softplus, const float *A, const void *B,
                          const void *C, const float *D, const void *z, void *y, int64_t batch, int64_t nheads,
                          int64_t headdim, int64_t dstate, int64_t ngroups, ssd_dtype dtype, void *stream) {
    if (batch != 0 && (!conv_state || !conv_w)) return SSD_ERR_NULL;
    return step_impl(state, conv_state, x, conv_w, conv_b, dt, dt_bias, dt_softplus, A, B, C, D, z, y, batch,
                     nheads, headdim, dstate, ngroups, dtype, stream);
}

}  // extern "C"

namespace {

ssd_status step_impl(float *state, void *conv_state, const void *x, const float *conv_w, const float *conv_b,
                     const void *dt, const float *dt_bias, int dt_softplus, const float *A, const void *B,
                     const void *C, const float *D, const void *z, void *y, int64_t batch, int64_t nheads,
                     int64_t headdim, int64_t dstate, int64_t ngroups, ssd_dtype dtype, void *stream) {
    if (dt_softplus < 0 || dt_softplus > 2) return SSD_ERR_UNSUPPORTED;
    if (batch != 0 && (!state || !x || !dt || !A || !B || !C || !D || !y)) return SSD_ERR_NULL;
    if (!valid_dtype((int)dtype)) return SSD_ERR_UNSUPPORTED;
    if (batch < 0 || nheads <= 0 || headdim <= 0 || dstate <= 0 || ngroups <= 0) return SSD_ERR_SHAPE;
    if (nheads % ngroups != 0) return SSD_ERR_SHAPE;
    if (!in_set(dstate, {4, 8, 16, 32, 64, 128, 256})) return SSD_ERR_UNSUPPORTED;
    if (!aligned16(state) || !aligned16(x) || !aligned16(dt) || !aligned16(A) || !aligned16(B) ||
        !aligned16(C) || !aligned16(D) || !aligned16(y) || !aligned16(dt_bias) || !aligned16(z) ||
        !aligned16(conv_state) || !aligned16(conv_w) || ((uintptr_t)conv_b & 3u) != 0)
        return SSD_ERR_ALIGN;
    if (batch == 0) return SSD_OK;
    // grid size bound (each factor first, so that the product stays inside int64)
    if (batch > (int64_t)UINT32_MAX || nheads > 65536 || headdim > 4096) return SSD_ERR_UNSUPPORTED;
    const int64_t rows = batch * nheads * headdim;
    if (rows > (int64_t)UINT32_MAX) return SSD_ERR_UNSUPPORTED;
    ssd::StepArgs a;
    a.state = state; a.x = x; a.dt = dt; a.B = B; a.C = C; a.A = A; a.D = D; a.y = y;
    a.batch = batch; a.H = nheads; a.P = headdim; a.N = dstate; a.G = ngroups; a.dtype = dtype;
    a.dt_bias = dt_bias; a.softplus = dt_softplus; a.z = z;
    a.conv_state = conv_state; a.conv_w = conv_w; a.conv_b = conv_b;
    return ssd::launch_step(a, reinterpret_cast<hipStream_t>(stream));
}

}  // namespace

extern "C" {

size_t ssd_chunk_scan_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                                          int64_t dstate, int64_t ngroups, int64_t chunk, ssd_dtype dtype) {
    BwdLayout lay;
    if (check_bwd_shape(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, (int)dtype, &lay) != SSD_OK)
        return (size_t)-1;
    return (size_t)lay.total;
}

ssd_status ssd_chunk_scan_bwd(const void *X, const void *dt, const float *A, const void *B, const void *C,
                              const float *D, int64_t chunk, const float *initial_state, const void *dY,
                              const float *d_final_state, void *dX, void *ddt, float *dA, void *dB, void *dC,
                              float *dD, float *d_initial_state, int64_t batch, int64_t seqlen, int64_t nheads,
                              int64_t headdim, int64_t dstate, int64_t ngroups, ssd_dtype dtype, void *workspace,
                              size_t workspace_bytes, void *stream) {
    if (batch > 0 && (!A || !D || !dA || !dD)) return SSD_ERR_NULL;
    const bool empty = (batch == 0 || seqlen == 0);
    if (!empty && (!X || !dt || !B || !C || !dY || !dX || !ddt || !dB || !dC)) return SSD_ERR_NULL;
    BwdLayout lay;
    ssd_status st = check_bwd_shape(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, (int)dtype, &lay);
    if (st != SSD_OK) return st;
    if (!aligned16(X) || !aligned16(dt) || !aligned16(A) || !aligned16(B) || !aligned16(C) || !aligned16(D) ||
        !aligned16(initial_state) || !aligned16(dY) || !aligned16(d_final_state) || !aligned16(dX) ||
        !aligned16(ddt) || !aligned16(dA) || !aligned16(dB) || !aligned16(dC) || !aligned16(dD) ||
        !aligned16(d_initial_state))
        return SSD_ERR_ALIGN;
    if (lay.total > 0) {
        if (!workspace || workspace_bytes < (size_t)lay.total) return SSD_ERR_WORKSPACE;
        if (((uintptr_t)workspace & 255u) != 0) return SSD_ERR_ALIGN;
    }
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (batch == 0) return SSD_OK;
    if (seqlen == 0) {
        // nothing flows through: dA = dD = 0, and the initial state's gradient is dF
        if (ssd::launch(k_zero, dim3((unsigned)((nheads + 255) / 256)), dim3(256), s, dA, nheads) != hipSuccess ||
            ssd::launch(k_zero, dim3((unsigned)((nheads + 255) / 256)), dim3(256), s, dD, nheads) != hipSuccess)
            return SSD_ERR_HIP;
        return empty_final_state(d_initial_state, d_final_state, batch * nheads * headdim * dstate, s);
    }
    ssd::BwdArgs w = {};
    w.f = make_args(lay.fl, batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype, workspace);
    w.f.X = X; w.f.dt = dt; w.f.A = A; w.f.B = B; w.f.C = C; w.f.D = D; w.f.init = initial_state;
    w.f.no_g = true;
    char *ws = static_cast<char *>(workspace) + 2 * lay.fl.cs_bytes + lay.fl.g_bytes + lay.fl.seg_bytes;
    w.Hst = ws; ws += lay.st_bytes;
    w.Est = ws; ws += lay.st_bytes;
    w.lamb = reinterpret_cast<float *>(ws); ws += lay.share_bytes;
    w.dApart = reinterpret_cast<float *>(ws); ws += lay.lamb_bytes;
    w.dDpart = reinterpret_cast<float *>(ws); ws += lay.lamb_bytes;
    w.rbuf = reinterpret_cast<float *>(ws); ws += lay.rq_bytes;
    w.qbuf = reinterpret_cast<float *>(ws); ws += lay.rq_bytes;
    w.xybuf = reinterpret_cast<float *>(ws); ws += lay.tok_bytes;
    w.dBp = reinterpret_cast<float *>(ws); ws += lay.part_bytes;
    w.dCp = reinterpret_cast<float *>(ws); ws += lay.part_bytes;
    w.dXp = lay.dxp_bytes ? reinterpret_cast<float *>(ws) : nullptr;
    w.nblk = lay.nblk;
    w.dY = dY; w.dF = d_final_state; w.dX = dX; w.ddt = ddt; w.dB = dB; w.dC = dC;
    w.dA = dA; w.dD = dD; w.dinit = d_initial_state;
    if ((st = ssd::launch_prepare(w.f, s)) != SSD_OK) return st;
    return ssd::launch_bwd(w, s);
}

}  // extern "C"
