// Backward pass of the SSD core: the gradients of <dY, Y> + <dF, final_state>
// with respect to X, dt, A, B, C, D and the initial state.
//
// Per (batch, head), with a_t = exp(dt_t A), states s_t and the adjoint
// ds_t = dy_t C_t^T + a_{t+1} ds_{t+1}:
//   dx_t = dt_t ds_t B_t + D dy_t          dB_t += dt_t ds_t^T x_t
//   dC_t += s_t^T dy_t                     dD   += <dy_t, x_t>
//   ddt_t = x_t^T ds_t B_t + A Lambda_t    dA   += dt_t Lambda_t
// with Lambda_t = <ds_t, a_t s_{t-1}>. Writing y_t' = s_t C_t (the scan's
// part of y_t) and v_t = ds_t B_t, the recurrences give
//   Lambda_t = (dy_t . y_t' - dt_t x_t . v_t) + Lambda_{t+1},
// a reverse running sum of per-token scalars. At a tile boundary Lambda is
// also <E, s> of the adjoint arriving from the next tile and the state
// leaving this one, s = 2^{cs_e - cs_r} h + sum_j 2^{cs_e - cs'_j} x_j B_j^T
// with h the state entering the tile; k_bwd_tile forms it as
// 2^{cs_e - cs_r} <E, h> + sum_j 2^{cs_e - cs'_j} x_j . (E B_j) from the
// operands it already holds, and the running sum restarts from it at every
// tile. dA sums dt_t Lambda_t, which cancels heavily; a running sum over the
// whole sequence would carry every rounding error of the per-token scalars
// (bf16 operands) into all earlier tokens.
//
// The work follows the chunked form of the forward (the reading report's
// section 3.1: quadratic diagonal blocks, rank-N blocks through states handed
// across block boundaries), in 64-token tiles:
//   k_state_passes, reverse work-groups
//                      per (batch, head, slice of the state's columns;
//                      one slice unless the pairs are too few to fill the
//                      CUs), tiles in reverse: the adjoint
//                      arriving at every tile from the tokens after it,
//                      E = a ds of the next token (stored in the storage
//                      type), and finally a_0 ds_0, the initial state's
//                      gradient;
//   k_state_passes, forward work-groups (the same launch)
//                      per (batch, head, column slice): the state entering every tile
//                      (stored in the storage type);
//   k_bwd_tile         per (batch, tile, group, block of heads, slice of the
//                      state's columns): everything inside the tile from h
//                      (entering state) and E (arriving adjoint): y', v, dx,
//                      the per-token scalars of Lambda, Lambda at the tile's
//                      end, and dB, dC summed over the block's heads;
//   k_bwd_dx           (more than one slice) dx from the slices' fp32 parts;
//   k_bwd_fin          per (batch, head, tile): Lambda down the tile, ddt, and
//                      the tile's shares of dA, dD (k_bwd_heads adds them up);
//   k_bwd_sum_bc       dB and dC summed over head blocks, in the storage type
//                      (with one block per group k_bwd_tile writes them).
// Within a tile (t the row token, j <= t and u >= t other tokens of the
// tile, cs the chunk-local base-2 log-decays, cs' = cs - log2 dt, r / e the
// tile's reference (token before it) and end):
//   y'  = 2^{cs_t - cs_r} C_t h^T + sum_{j<=t} (C_t.B_j) 2^{cs_t - cs'_j} x_j
//   v   = 2^{cs_e - cs_t} E B_t   + sum_{u>=t} (C_u.B_t) 2^{cs_u - cs_t} dy_u
//   dC_t += 2^{cs_t - cs_r} h^T dy_t + sum_{j<=t} (x_j.dy_t) 2^{cs_t - cs'_j} B_j
//   dB_t += dt_t [2^{cs_e - cs_t} E^T x_t + sum_{u>=t} (dy_u.x_t) 2^{cs_u - cs_t} C_u]
// Every exponent is <= 0 where it is used (or equals log2 dt_j), so nothing
// overflows; masked positions are selected to zero before use.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "ssd_common.h"
#include "ssd_internal.h"

namespace ssd {

constexpr int kBT = 64;  // tile tokens

template <typename TI>
__device__ __forceinline__ void store4(TI *p, f32x4 v) {
    if constexpr (sizeof(TI) == 2) {
        const bf16x4 b = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
        *reinterpret_cast<bf16x4 *>(p) = b;
    } else {
        *reinterpret_cast<f32x4 *>(p) = v;
    }
}

template <typename TI>
__device__ __forceinline__ void lds_st4(TI *p, float a, float b, float c, float d) {
    store4<TI>(p, f32x4{a, b, c, d});
}

// A fragment from two runs of 4 consecutive elements (k slots 0-3 and 4-7).
template <typename TI>
__device__ __forceinline__ typename Traits<TI>::frag lds_frag_split(const TI *p0, const TI *p1) {
    typename Traits<TI>::frag f;
    if constexpr (sizeof(TI) == 2) {
        const bf16x4 a = *reinterpret_cast<const bf16x4 *>(p0);
        const bf16x4 b = *reinterpret_cast<const bf16x4 *>(p1);
        f[0] = a[0]; f[1] = a[1]; f[2] = a[2]; f[3] = a[3];
        f[4] = b[0]; f[5] = b[1]; f[6] = b[2]; f[7] = b[3];
    } else {
        const f32x4 a = *reinterpret_cast<const f32x4 *>(p0);
        const f32x4 b = *reinterpret_cast<const f32x4 *>(p1);
        f[0] = a[0]; f[1] = a[1]; f[2] = a[2]; f[3] = a[3];
        f[4] = b[0]; f[5] = b[1]; f[6] = b[2]; f[7] = b[3];
    }
    return f;
}

// Transposing stage: an R x Cc tile of global rows (row q at byte offset
// off0 + q * rstride, Cc contiguous elements) into LDS as dst[c * LD + q],
// row q scaled by wt(q) when kW. Units of 4 rows x 8 columns; every thread
// issues its loads unconditionally (spare units at an out-of-range offset).
template <typename TI, int R, int Cc, int NTH, bool kW, typename WF>
__device__ __forceinline__ void stage_T(rsrc_t rs, uint32_t off0, uint32_t rstride, TI *dst, int LD,
                                        int tid, WF wt) {
    using Tr = Traits<TI>;
    constexpr int ES = Tr::kBytes;
    constexpr int UR = R / 4, U = UR * (Cc / 8), K = (U + NTH - 1) / NTH;
    typename Tr::frag v[K][4];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int u = tid + k * NTH;
        const int rq = u % UR, co = (u / UR) % (Cc / 8);
        const uint32_t o = off0 + (uint32_t)(4 * rq) * rstride + (uint32_t)(8 * co * ES);
#pragma unroll
        for (int i = 0; i < 4; ++i) v[k][i] = Tr::load_frag(rs, oob_if(u >= U, o + (uint32_t)i * rstride));
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int u = tid + k * NTH;
        if (u >= U) continue;
        const int rq = u % UR, co = u / UR;
        float w[4] = {1.f, 1.f, 1.f, 1.f};
        if constexpr (kW) {
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = wt(4 * rq + i);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e)
            lds_st4<TI>(dst + (8 * co + e) * LD + 4 * rq, Tr::frag_get(v[k][0], e) * w[0],
                        Tr::frag_get(v[k][1], e) * w[1], Tr::frag_get(v[k][2], e) * w[2],
                        Tr::frag_get(v[k][3], e) * w[3]);
    }
}

// Plain stage: R rows of Cc elements into dst[q * LD + c], 16 bytes at a time.
template <typename TI, int R, int Cc, int NTH>
__device__ __forceinline__ void stage_N(rsrc_t rs, uint32_t off0, uint32_t rstride, TI *dst, int LD, int tid) {
    constexpr int ES = sizeof(TI);
    constexpr int VPR = Cc * ES / 16, U = R * VPR, K = (U + NTH - 1) / NTH;
    u32x4 v[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int u = tid + k * NTH;
        v[k] = buf_ld128(rs, oob_if(u >= U, off0 + (uint32_t)(u / VPR) * rstride + (uint32_t)((u % VPR) * 16)));
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int u = tid + k * NTH;
        if (u >= U) continue;
        *reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(dst + (u / VPR) * LD) + (u % VPR) * 16) = v[k];
    }
}

// Two-phase staging, so that a tile's global loads can be issued while the
// previous one is computed: load() fills registers with an R x Cc tile in
// units of 4 rows x 8 columns; store_T() / store_N() write them to LDS
// transposed (dst[c * LD + q], rows optionally weighted) or as they are
// (dst[q * LD + c]).
template <typename TI, int R, int Cc, int NTH>
struct TileRegs {
    using Tr = Traits<TI>;
    static constexpr int ES = Tr::kBytes, UR = R / 4, U = UR * (Cc / 8), K = (U + NTH - 1) / NTH;
    typename Tr::frag v[K][4];
    __device__ __forceinline__ void load(rsrc_t rs, uint32_t off0, uint32_t rstride, int tid) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int u = tid + k * NTH;
            const int rq = u % UR, co = (u / UR) % (Cc / 8);
            const uint32_t o = off0 + (uint32_t)(4 * rq) * rstride + (uint32_t)(8 * co * ES);
#pragma unroll
            for (int i = 0; i < 4; ++i) v[k][i] = Tr::load_frag(rs, oob_if(u >= U, o + (uint32_t)i * rstride));
        }
    }
    template <bool kW, typename WF>
    __device__ __forceinline__ void store_T(TI *dst, int LD, int tid, WF wt) const {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int u = tid + k * NTH;
            if (u >= U) continue;
            const int rq = u % UR, co = u / UR;
            if constexpr (kW) {
                float w[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = wt(4 * rq + i);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    lds_st4<TI>(dst + (8 * co + e) * LD + 4 * rq, Tr::frag_get(v[k][0], e) * w[0],
                                Tr::frag_get(v[k][1], e) * w[1], Tr::frag_get(v[k][2], e) * w[2],
                                Tr::frag_get(v[k][3], e) * w[3]);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    TI *d = dst + (8 * co + e) * LD + 4 * rq;
                    if constexpr (ES == 2) {
                        const bf16x4 q = {v[k][0][e], v[k][1][e], v[k][2][e], v[k][3][e]};
                        *reinterpret_cast<bf16x4 *>(d) = q;
                    } else {
                        const f32x4 q = {v[k][0][e], v[k][1][e], v[k][2][e], v[k][3][e]};
                        *reinterpret_cast<f32x4 *>(d) = q;
                    }
                }
            }
        }
    }
    __device__ __forceinline__ void store_N(TI *dst, int LD, int tid) const {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int u = tid + k * NTH;
            if (u >= U) continue;
            const int rq = u % UR, co = u / UR;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<typename Tr::frag *>(dst + (4 * rq + i) * LD + 8 * co) = v[k][i];
        }
    }
};

// ---------------------------------------------------------------------------
// The state passes: one work-group of SP_NW wavefronts per (batch, head) walks
// the tiles (backwards when kRev) with the P x N state in matrix-core
// accumulators, wave w owning the state's columns n in blocks w, w + SP_NW, ...
// Before each tile it stores the state it carries into Sst[tile] ([p][n],
// storage type); after the last one it writes the state (fp32) to `out`.
//   forward: S <- 2^{cs_e - cs_r} S + sum_t 2^{cs_e - cs'_t} x_t B_t^T
//   reverse: S <- 2^{cs_e - cs_r} S + sum_t 2^{cs_t - cs_r} dy_t C_t^T
// (U = X or dY, V = B or C). The two passes share nothing, so k_state_passes
// runs both in one launch (reverse work-groups first), two work-groups per CU.
// Columns n of the state evolve independently (V's column n feeds only the
// state's column n), so where (batch, head) pairs are too few to fill the
// CUs, each pass splits the state's N columns into slices of NL, one
// work-group per slice, each staging the whole U tile and its slice of V.
// ---------------------------------------------------------------------------
constexpr int SP_NW = 4;  // wavefronts per state-pass work-group

template <typename TI, int P, int N>  // N: the work-group's slice of the state's columns
struct SpLds {
    static constexpr int ES = sizeof(TI), PAD = 16 / ES, T_LD = kBT + PAD, S_LD = N + PAD;
    TI UT[P * T_LD];
    TI VT[N * T_LD];
    // the state each tile stores goes through LDS ([p][n], padded rows) so that
    // it leaves as whole 16-byte row pieces: written straight from the
    // accumulators each store instruction would cover 16 rows x 32 bytes
    TI SS[P * S_LD];
    float WT[kBT];
};

// One pass over the state columns n0 .. n0 + NL - 1 (of N) of (batch, head) bh.
template <typename TI, int P, int N, int NL, bool kRev>
__device__ __forceinline__ void state_pass(const StatePassArgs &a, SpLds<TI, P, NL> &sm, const int bh,
                                           const int n0) {
    using Tr = Traits<TI>;
    using frag = typename Tr::frag;
    using L = SpLds<TI, P, NL>;
    constexpr int ES = Tr::kBytes, T_LD = L::T_LD, S_LD = L::S_LD;
    constexpr int NW = SP_NW, NTH = 64 * NW;  // wave w owns n-blocks w, w + NW, ... of the slice
    constexpr int PB = P / 16, NB = NL / 16, NBW = (NB + NW - 1) / NW;
    TI *const UT = sm.UT, *const VT = sm.VT, *const SS = sm.SS;
    float *const WT = sm.WT;

    const int H = a.H, G = a.G, T = a.T;
    const int b = bh / H, h = bh - b * H, g = (h * G) / H;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, kg = lane >> 4;
    const rsrc_t ru = make_rsrc(reinterpret_cast<const char *>(a.U) + (size_t)b * T * H * P * ES,
                                (uint32_t)((size_t)T * H * P * ES));
    const rsrc_t rv = make_rsrc(reinterpret_cast<const char *>(a.V) + (size_t)b * T * G * N * ES,
                                (uint32_t)((size_t)T * G * N * ES));
    const float *cs = a.cs2 + (size_t)bh * a.Tpad;
    const float *cp = a.dtf + (size_t)bh * a.Tpad;

    f32x4 acc[PB][NBW];
#pragma unroll
    for (int pb = 0; pb < PB; ++pb)
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
            const int nb = w + NW * j;
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            if (a.init && nb < NB)
                v = *reinterpret_cast<const f32x4 *>(a.init + ((size_t)bh * P + 16 * pb + r) * N + n0 + 16 * nb +
                                                     4 * kg);
            acc[pb][j] = v;
        }
    const int ntiles = a.ntiles;
    // a tile's U, V and per-token exponent terms, loaded two tiles ahead into
    // one of two register sets.
    // Every slot is consumed before it is loaded again (a value still live
    // across the next load into its slot becomes a register copy at the loop's
    // back edge, and the copy waits for every load in flight).
    TileRegs<TI, kBT, P, NTH> ur[2];
    TileRegs<TI, kBT, NL, NTH> vr[2];
    float wcs[2] = {0.f, 0.f};                   // this thread's token term
    float pcs_r[2] = {0.f, 0.f}, pcs_e[2] = {0.f, 0.f};
    auto issue = [&](int tau, auto Sc) {
        constexpr int S = decltype(Sc)::value;
        const int t0 = tau * kBT;
        ur[S].load(ru, (uint32_t)(((size_t)t0 * H + h) * P * ES), (uint32_t)(H * P * ES), tid);
        vr[S].load(rv, (uint32_t)((((size_t)t0 * G + g) * N + n0) * ES), (uint32_t)(G * N * ES), tid);
        // unconditional: a chunk's first tile takes 0 where the value is used
        pcs_r[S] = cs[max(t0 - 1, 0)];
        pcs_e[S] = cs[t0 + kBT - 1];
        wcs[S] = kRev ? cs[t0 + (tid & 63)] : cp[t0 + (tid & 63)];
    };
    auto tile_of = [&](int it) { return kRev ? max(ntiles - 1 - it, 0) : min(it, ntiles - 1); };
    issue(tile_of(0), std::integral_constant<int, 0>{});
    issue(tile_of(1), std::integral_constant<int, 1>{});
    auto step = [&](int it, auto Sc) {
        constexpr int S = decltype(Sc)::value;
        const int tau = tile_of(it);
        TI *dst = reinterpret_cast<TI *>(a.Sst) + ((size_t)bh * ntiles + tau) * P * N + n0;
#pragma unroll
        for (int pb = 0; pb < PB; ++pb)
#pragma unroll
            for (int j = 0; j < NBW; ++j) {
                const int nb = w + NW * j;
                if (nb < NB) store4<TI>(SS + (16 * pb + r) * S_LD + 16 * nb + 4 * kg, acc[pb][j]);
            }
        const float cs_r = (tau % a.tpc == 0) ? 0.f : pcs_r[S], cs_e = pcs_e[S];
        const float dec = fast_exp2(cs_e - cs_r);
        // every wavefront writes the same 64 weights: no load result is consumed under a
        // branch (that made the compiler wait for every load in flight, the prefetch included)
        WT[tid & (kBT - 1)] = kRev ? fast_exp2(wcs[S] - cs_r) : fast_exp2(cs_e - wcs[S]);
        __syncthreads();  // SS and WT visible; the previous tile's reads of UT / VT are done
        {
            constexpr int VPRS = NL * ES / 16;  // 16-byte pieces per row of the slice
#pragma unroll
            for (int v = tid; v < P * VPRS; v += NTH) {
                const int p = v / VPRS, c = v % VPRS;
                *reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(dst) + (size_t)p * N * ES + c * 16) =
                    *reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(SS) + p * S_LD * ES + c * 16);
            }
        }
        ur[S].template store_T<false>(UT, T_LD, tid, [](int) { return 1.f; });
        vr[S].template store_T<true>(VT, T_LD, tid, [&](int q) { return WT[q]; });
        __syncthreads();
        // the tile after next is loaded while this one is computed (past the end: a reload)
        issue(tile_of(it + 2), Sc);
#pragma unroll
        for (int pb = 0; pb < PB; ++pb)
#pragma unroll
            for (int j = 0; j < NBW; ++j) acc[pb][j] *= dec;
#pragma unroll
        for (int k2 = 0; k2 < kBT / 32; ++k2) {
            frag ua[PB];
#pragma unroll
            for (int pb = 0; pb < PB; ++pb) ua[pb] = Tr::lds_frag(UT + (16 * pb + r) * T_LD + 32 * k2 + 8 * kg);
#pragma unroll
            for (int j = 0; j < NBW; ++j) {
                const int nb = w + NW * j;
                if (nb < NB) {
                    const frag vb = Tr::lds_frag(VT + (16 * nb + r) * T_LD + 32 * k2 + 8 * kg);
#pragma unroll
                    for (int pb = 0; pb < PB; ++pb) acc[pb][j] = Tr::mma(vb, ua[pb], acc[pb][j]);
                }
            }
        }
        __syncthreads();
    };
    // pairs of steps with no condition inside the loop body (a conditional second step made
    // the compiler drain every load in flight at the back edge), then an odd last tile
    int it = 0;
    for (; it + 1 < ntiles; it += 2) {
        step(it, std::integral_constant<int, 0>{});
        step(it + 1, std::integral_constant<int, 1>{});
    }
    if (it < ntiles) step(it, std::integral_constant<int, 0>{});
    if (a.out) {
#pragma unroll
        for (int pb = 0; pb < PB; ++pb)
#pragma unroll
            for (int j = 0; j < NBW; ++j) {
                const int nb = w + NW * j;
                if (nb < NB)
                    *reinterpret_cast<f32x4 *>(a.out + ((size_t)bh * P + 16 * pb + r) * N + n0 + 16 * nb + 4 * kg) =
                        acc[pb][j];
            }
    }
}

// work-groups [0, nbh N / NL): the reverse pass; the rest: the forward pass;
// each (batch, head) pair's N / NL column slices are consecutive
template <typename TI, int P, int N, int NL>
__global__ __launch_bounds__(64 * SP_NW) void k_state_passes(StatePassArgs rev, StatePassArgs fwd, int nbh) {
    constexpr int NSL = N / NL;
    __shared__ __attribute__((aligned(16))) SpLds<TI, P, NL> sm;
    const int per = nbh * NSL;
    const int x = (int)blockIdx.x < per ? (int)blockIdx.x : (int)blockIdx.x - per;
    const int bh = x / NSL, n0 = (x % NSL) * NL;
    if ((int)blockIdx.x < per) state_pass<TI, P, N, NL, true>(rev, sm, bh, n0);
    else state_pass<TI, P, N, NL, false>(fwd, sm, bh, n0);
}

// Column slices of the state passes: halve the slice (down to 64 columns)
// while the two passes together have fewer than two work-groups per CU.
static int state_pass_slices(int64_t nbh, int N) {
    int nsl = 1;
    while (2 * nbh * nsl < 2 * 256 && N / (2 * nsl) >= 64) nsl *= 2;
    return nsl;
}

// ---------------------------------------------------------------------------
// k_bwd_tile: LDS layout and the work of one (batch, tile, group, head block).
// ---------------------------------------------------------------------------
template <typename TI, int P, int N>
struct BwdCfg {
    static constexpr int ES = sizeof(TI), PAD = 16 / ES;
    static constexpr int PB = P / 16, NB = N / 16, NK = N / 32, KP = P / 32;
    static constexpr int T_LD = kBT + PAD, P_LD = P + PAD, N_LD = N + PAD;
    // element offsets (storage type); N is the work-group's slice of the state columns
    static constexpr int BT_OFF = 0;                       // B^T [n][t], per tile
    static constexpr int CT_OFF = BT_OFF + N * T_LD;       // C^T [n][t], per tile
    static constexpr int OS_OFF = CT_OFF + N * T_LD;       // dX staging, 16 rows per wave
    static constexpr int HEAD_OFF = OS_OFF + 4 * 16 * P_LD;
    // two per-head buffers (head k in buffer k % 2), each row-major only: the
    // transposed operands are read from them with the LDS transpose read
    static constexpr int XN = 0;                           // X [t][p]
    static constexpr int DYN = XN + kBT * P_LD;            // dY [t][p]
    static constexpr int HN = DYN + kBT * P_LD;            // h [p][n]
    static constexpr int EN = HN + P * N_LD;               // E [p][n]
    static constexpr int BUF = EN + P * N_LD;
    static constexpr int ELEMS = HEAD_OFF + 2 * BUF;
    // bytes: per buffer the head's cs, cs', dt of the tile's tokens, then cs before the tile
    // (0 at a chunk's start), cs at its end and D
    static constexpr int F_OFF = (ELEMS * ES + 15) / 16 * 16;
    static constexpr int FBUF = 3 * kBT + 4;
    static constexpr int LDS = F_OFF + 2 * FBUF * 4;
    static constexpr bool kFits = LDS <= 160 * 1024 && P % 32 == 0 && N % 32 == 0;
};

// Four consecutive rows kb .. kb + 3 of column c0 + (lane & 15) of a
// row-major matrix M in LDS (row pitch ld elements); kb may differ between the
// wavefront's four 16-lane groups. bf16: one LDS transpose read, in which lane
// j of a group supplies the address of row kb + j / 4, columns c0 + 4 (j % 4)
// .. + 3, and receives the column of its own lane index; fp32: four reads.
__device__ __forceinline__ u32x2 tr4_bits(const bf16 *M, int ld, int kb, int c0, int lane) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
    const int j = lane & 15;
    const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(M + (kb + (j >> 2)) * ld + c0 + 4 * (j & 3)));
    return __builtin_bit_cast(u32x2, v);
}
template <typename TI>
__device__ __forceinline__ void tr4(const TI *M, int ld, int kb, int c0, int lane, TI (&o)[4]) {
    if constexpr (sizeof(TI) == 2) {
        const u32x2 w = tr4_bits(M, ld, kb, c0, lane);
        const uint32_t w0 = w[0], w1 = w[1];
        o[0] = __builtin_bit_cast(bf16, (uint16_t)(w0 & 0xffffu));
        o[1] = __builtin_bit_cast(bf16, (uint16_t)(w0 >> 16));
        o[2] = __builtin_bit_cast(bf16, (uint16_t)(w1 & 0xffffu));
        o[3] = __builtin_bit_cast(bf16, (uint16_t)(w1 >> 16));
    } else {
        const int c = c0 + (lane & 15);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = M[(kb + e) * ld + c];
    }
}
// A matrix-core operand from a row-major matrix read down its columns: slots
// 0-3 rows kb0 .. kb0 + 3, slots 4-7 rows kb1 .. kb1 + 3, column c0 + (lane & 15).
template <typename TI>
__device__ __forceinline__ typename Traits<TI>::frag tr_frag(const TI *M, int ld, int kb0, int kb1, int c0,
                                                               int lane) {
    typename Traits<TI>::frag f;
    if constexpr (sizeof(TI) == 2) {
        const u32x2 a = tr4_bits(M, ld, kb0, c0, lane), b = tr4_bits(M, ld, kb1, c0, lane);
        const uint32_t a0 = a[0], a1 = a[1], b0 = b[0], b1 = b[1];
        f = __builtin_bit_cast(bf16x8, u32x4{a0, a1, b0, b1});
    } else {
        TI x[4], y[4];
        tr4<TI>(M, ld, kb0, c0, lane, x);
        tr4<TI>(M, ld, kb1, c0, lane, y);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            f[e] = x[e];
            f[4 + e] = y[e];
        }
    }
    return f;
}

// Sum over each row of 16 lanes, left in every lane of the row, with DPP moves on the vector
// ALU (no LDS traffic): neighbours, then pairs (quad permutes), then the two quads of each
// half-row (half-row mirror), then the two half-rows (row mirror).
__device__ __forceinline__ float row16_sum(float v) {
    auto mv = [](float x, int ctrl) -> float {
        switch (ctrl) {  // the control word must be a constant
            case 0xB1: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
            case 0x4E: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
            case 0x141: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
            default: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));
        }
    };
    v += mv(v, 0xB1);   // quad_perm [1, 0, 3, 2]: lane ^ 1
    v += mv(v, 0x4E);   // quad_perm [2, 3, 0, 1]: lane ^ 2
    v += mv(v, 0x141);  // row_half_mirror: lane i <- 7 - i within each 8
    v += mv(v, 0x140);  // row_mirror: lane i <- 15 - i
    return v;
}
// Sum over all 64 lanes: the rows' sums, then across rows with two lane shuffles.
__device__ __forceinline__ float wave_sum(float v) {
    v = row16_sum(v);
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}

// 8 wavefronts in two roles over the same staged tile and head: waves 0-3
// (16 token rows each) form y', v, dX and the per-token scalars; waves 4-7
// (same rows) form x.dy products, dC and dB. The roles share no results, so
// the two waves on each SIMD overlap.
// Where the LDS of one work-group cannot hold the whole n axis, NS = N / NL
// work-groups take a slice of NL state columns each. Every sum over n (y', v,
// C B^T, and through them dX, the per-token scalars and Lambda's parts) is
// then a sum of the slices' partial results, which they write separately
// (dX in fp32) for k_bwd_fin and k_bwd_dx to add in a fixed order; dB and dC
// are per n and come out whole.
template <typename TI, int P, int N, int NL>
__global__ __launch_bounds__(512, 1) void k_bwd_tile(BwdTileArgs a) {
    using Tr = Traits<TI>;
    using frag = typename Tr::frag;
    using Cfg = BwdCfg<TI, P, NL>;
    constexpr int NS = N / NL;
    constexpr int ES = Cfg::ES, PB = Cfg::PB, NB = Cfg::NB, NK = Cfg::NK, KP = Cfg::KP;
    constexpr int T_LD = Cfg::T_LD, P_LD = Cfg::P_LD, N_LD = Cfg::N_LD;
    __shared__ __attribute__((aligned(16))) char smem[Cfg::LDS];
    TI *const L = reinterpret_cast<TI *>(smem);
    TI *const BT = L + Cfg::BT_OFF, *const CT = L + Cfg::CT_OFF;
    TI *const HB = L + Cfg::HEAD_OFF;                                  // the two per-head buffers
    float *const FB = reinterpret_cast<float *>(smem + Cfg::F_OFF);    // their cs, cs', dt
    // the current head's buffer (set at the top of each head)
    const TI *XN = nullptr, *DYN = nullptr, *HN = nullptr, *EN = nullptr;
    const float *CS = nullptr, *CP = nullptr, *DT = nullptr, *SC = nullptr;
    auto use_buffer = [&](int sb) __attribute__((always_inline)) {
        const TI *B0 = HB + sb * Cfg::BUF;
        XN = B0 + Cfg::XN; DYN = B0 + Cfg::DYN; HN = B0 + Cfg::HN; EN = B0 + Cfg::EN;
        CS = FB + sb * Cfg::FBUF; CP = CS + kBT; DT = CP + kBT; SC = DT + kBT;
    };

    const int H = a.H, G = a.G, T = a.T, HG = H / G, nblk = a.nblk, hpb = HG / nblk;
    int x = blockIdx.x;
    const int sl = x % NS;
    x /= NS;
    const int blk = x % nblk;
    x /= nblk;
    const int g = x % G;
    x /= G;
    const int tau = x % a.ntiles;
    const int b = x / a.ntiles;
    const int t0 = tau * kBT;
    const int n0 = sl * NL;  // this work-group's state columns n0 .. n0 + NL - 1
    const size_t tsl = (size_t)sl * a.tok_stride;  // its per-token partials
    const size_t tsl_x = (size_t)sl * a.dx_stride;  // and its part of dx (NS > 1)
    constexpr int NTH = 512;
    const int tid = threadIdx.x, lane = tid & 63, r = lane & 15, kg = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool roleA = wv < 4;  // wave-uniform
    const int w = wv & 3;
    TI *OS = L + Cfg::OS_OFF + w * 16 * P_LD;

    const size_t xslab = (size_t)T * H * P * ES, bslab = (size_t)T * G * N * ES;
    const rsrc_t rx = make_rsrc(reinterpret_cast<const char *>(a.X) + b * xslab, (uint32_t)xslab);
    const rsrc_t rdy = make_rsrc(reinterpret_cast<const char *>(a.dY) + b * xslab, (uint32_t)xslab);
    const rsrc_t rdx = make_rsrc(reinterpret_cast<char *>(a.dX) + b * xslab, (uint32_t)xslab);
    const rsrc_t rb = make_rsrc(reinterpret_cast<const char *>(a.B) + b * bslab, (uint32_t)bslab);
    const rsrc_t rc = make_rsrc(reinterpret_cast<const char *>(a.C) + b * bslab, (uint32_t)bslab);
    const uint32_t b_tok = (uint32_t)(G * N * ES), x_tok = (uint32_t)(H * P * ES);

    // ---- per tile, shared by the block's heads ----
    stage_T<TI, kBT, NL, NTH, false>(rb, (uint32_t)((((size_t)t0 * G + g) * N + n0) * ES), b_tok, BT, T_LD, tid,
                                     [](int) { return 1.f; });
    stage_T<TI, kBT, NL, NTH, false>(rc, (uint32_t)((((size_t)t0 * G + g) * N + n0) * ES), b_tok, CT, T_LD, tid,
                                    [](int) { return 1.f; });
    const int trow = 16 * w + r;  // this lane's row token for A operands (tile-local)
    const int kc = w / 2;         // the k step holding the diagonal
    const int rt = tid & 255;     // thread index within the role
    constexpr bool kSplit = ES == 2;  // bf16: y' and v (which feed Lambda) take hi + lo

    // A operand (rows t = 16 w + r) over k slots of step k2 from two
    // 16-column accumulator blocks: slot e < 4 is column 32 k2 + 4 kg + e of
    // src[2 k2], slot e >= 4 column 32 k2 + 16 + 4 kg + e - 4 of src[2 k2 + 1];
    // `causal`: keep columns j <= t weighted 2^{cs_t - cs'_j}, else columns
    // u >= t weighted 2^{cs_u - cs_t}. With `lo`, also the rounding residual
    // of each element in a second fragment (bf16), so hi + lo carries fp32.
    auto make_a = [&](const f32x4 *src, int k2, bool causal, float cs_t, frag *lo) {
        frag f;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int c0 = 32 * k2 + 16 * half + 4 * kg;
            const f32x4 ref = *reinterpret_cast<const f32x4 *>((causal ? CP : CS) + c0);
            const f32x4 sv = src[2 * k2 + half];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = c0 + i;
                float v;
                if (causal) v = (c <= trow) ? sv[i] * fast_exp2(cs_t - ref[i]) : 0.f;
                else v = (c >= trow) ? sv[i] * fast_exp2(ref[i] - cs_t) : 0.f;
                Tr::frag_set(f, 4 * half + i, v);
                if (lo) Tr::frag_set(*lo, 4 * half + i, v - Tr::frag_get(f, 4 * half + i));
            }
        }
        return f;
    };
    // The two roles run separate loops with the same barriers, so that
    // neither role's registers stay live in the other's code.
    if (roleA) {
        // ================= role A: y', v, dX, per-token scalars =================
        // this wave's rows t = 16 w + r of C and B (A operands), and C B^T both ways:
        //   g1[jb][i] = C_t . B_j with j = 16 jb + 4 kg + i   (jb <= w)
        //   g2[ub][i] = C_u . B_t with u = 16 ub + 4 kg + i   (ub >= w)
        frag cw[NK], bw[NK];
        f32x4 g1[4], g2[4];
        const uint32_t grow = (uint32_t)(((t0 * G + g) * N + n0) * ES);
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
            const uint32_t o = grow + (uint32_t)(16 * w + r) * b_tok + (uint32_t)((32 * kk + 8 * kg) * ES);
            cw[kk] = Tr::load_frag(rc, o);
            bw[kk] = Tr::load_frag(rb, o);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            g1[q] = f32x4{0.f, 0.f, 0.f, 0.f};
            g2[q] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (q <= w) {
#pragma unroll
                for (int kk = 0; kk < NK; ++kk) {
                    const uint32_t o = grow + (uint32_t)(16 * q + r) * b_tok + (uint32_t)((32 * kk + 8 * kg) * ES);
                    g1[q] = Tr::mma(Tr::load_frag(rb, o), cw[kk], g1[q]);
                }
            }
            if (q >= w) {
#pragma unroll
                for (int kk = 0; kk < NK; ++kk) {
                    const uint32_t o = grow + (uint32_t)(16 * q + r) * b_tok + (uint32_t)((32 * kk + 8 * kg) * ES);
                    g2[q] = Tr::mma(Tr::load_frag(rc, o), bw[kk], g2[q]);
                }
            }
        }
        // the next head's X, dY and per-token terms load while this head is computed
        TileRegs<TI, kBT, P, 256> xr, dyr;
        // token t0 + (tid & 63) of the prefetched head; dt as its raw bits (0 past the end),
        // converted where it is used, and every load unconditional, so that no wait for it
        // sits under a branch or right after the load
        float pcs = 0.f, pcp = 0.f, pcr = 0.f, pce = 0.f, pd = 0.f;  // pcr, pce, pd: the head's cs_r, cs_e, D
        uint32_t pdt = 0;
        const rsrc_t rdt = make_rsrc(reinterpret_cast<const char *>(a.dt) + (size_t)b * T * H * ES,
                                     (uint32_t)((size_t)T * H * ES));
        auto issue = [&](int k) {
            const int h = g * HG + blk * hpb + k;
            const size_t bh = (size_t)b * H + h;
            const uint32_t xo = (uint32_t)(((size_t)t0 * H + h) * P * ES);
            xr.load(rx, xo, x_tok, rt);
            dyr.load(rdy, xo, x_tok, rt);
            const int t = t0 + (tid & 63);
            pcs = a.cs2[bh * a.Tpad + t];
            pcp = a.dtf[bh * a.Tpad + t];
            pcr = a.cs2[bh * a.Tpad + max(t0 - 1, 0)];
            pce = a.cs2[bh * a.Tpad + t0 + kBT - 1];
            pd = a.D[h];
            const uint32_t od = (uint32_t)(((size_t)t * H + h) * ES);
            if constexpr (ES == 2) pdt = buf_ld16(rdt, od);
            else pdt = buf_ld32(rdt, od);
        };
        // writes the loaded head's X, dY (row-major) and per-token terms into buffer sb
        auto stage = [&](int sb) {
            TI *B0 = HB + sb * Cfg::BUF;
            float *F = FB + sb * Cfg::FBUF;
            // the four role-A wavefronts write the same values
            const uint32_t u = pdt;
            F[tid & 63] = pcs;
            F[kBT + (tid & 63)] = pcp;
            F[2 * kBT + (tid & 63)] = ES == 2 ? __uint_as_float(u << 16) : __uint_as_float(u);
            F[3 * kBT + (tid & 3)] = (tid & 3) == 0 ? (tau % a.tpc == 0 ? 0.f : pcr) : (tid & 3) == 1 ? pce : pd;
            xr.store_N(B0 + Cfg::XN, P_LD, rt);
            dyr.store_N(B0 + Cfg::DYN, P_LD, rt);
        };
        issue(0);
        stage(0);
        issue(min(1, hpb - 1));
        __syncthreads();  // pairs with role B's: head 0 and the tile's B^T, C^T staged
        for (int k = 0; k < hpb; ++k) {
            use_buffer(k & 1);
            const int h = g * HG + blk * hpb + k;
            const size_t bh = (size_t)b * H + h;
            const float cs_r = SC[0], cs_e = SC[1], Dh = SC[2];
            const uint32_t xo = (uint32_t)(((size_t)t0 * H + h) * P * ES);
            const float cs_t = CS[trow];
            float cs_o[4], dt_o[4];  // output rows t = 16 w + 4 kg + i
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                cs_o[i] = CS[16 * w + 4 * kg + i];
                dt_o[i] = DT[16 * w + 4 * kg + i];
            }
            // ---- y' (scan output) and v = ds B, both [t][p] ----
            // Lambda at the tile's end is <E, state after the tile>; the tokens' part of that
            // state, sum_j 2^{cs_e - cs'_j} x_j B_j^T, contributes sum_j 2^{cs_e - cs'_j} x_j.(E B_j),
            // formed here from E B_j before it is scaled into v (role B adds the entering
            // state's part)
            float wl[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) wl[i] = fast_exp2(cs_e - CP[16 * w + 4 * kg + i]);
            float lam = 0.f;
            f32x4 ay[PB], av[PB];
#pragma unroll
            for (int pb = 0; pb < PB; ++pb) {
                ay[pb] = f32x4{0.f, 0.f, 0.f, 0.f};
                av[pb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < NK; ++kk) {
                    ay[pb] = Tr::mma(cw[kk], Tr::lds_frag(HN + (16 * pb + r) * N_LD + 32 * kk + 8 * kg), ay[pb]);
                    av[pb] = Tr::mma(bw[kk], Tr::lds_frag(EN + (16 * pb + r) * N_LD + 32 * kk + 8 * kg), av[pb]);
                }
                TI xl[4];  // x of this lane's 4 rows, column 16 pb + r
                tr4<TI>(XN, P_LD, 16 * w + 4 * kg, 16 * pb, lane, xl);
#pragma unroll
                for (int i = 0; i < 4; ++i) lam += wl[i] * Tr::to_f32(xl[i]) * av[pb][i];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    ay[pb][i] *= fast_exp2(cs_o[i] - cs_r);
                    av[pb][i] *= fast_exp2(cs_e - cs_o[i]);
                }
            }
#pragma unroll
            for (int k2 = 0; k2 < kBT / 32; ++k2) {
                if (k2 <= kc) {
                    frag lo;
                    const frag m = make_a(g1, k2, true, cs_t, kSplit ? &lo : nullptr);
#pragma unroll
                    for (int pb = 0; pb < PB; ++pb) {
                        const frag xb = tr_frag<TI>(XN, P_LD, 32 * k2 + 4 * kg, 32 * k2 + 16 + 4 * kg, 16 * pb, lane);
                        ay[pb] = Tr::mma(m, xb, ay[pb]);
                        if constexpr (kSplit) ay[pb] = Tr::mma(lo, xb, ay[pb]);
                    }
                }
                if (k2 >= kc) {
                    frag lo;
                    const frag m = make_a(g2, k2, false, cs_t, kSplit ? &lo : nullptr);
#pragma unroll
                    for (int pb = 0; pb < PB; ++pb) {
                        const frag db = tr_frag<TI>(DYN, P_LD, 32 * k2 + 4 * kg, 32 * k2 + 16 + 4 * kg, 16 * pb, lane);
                        av[pb] = Tr::mma(m, db, av[pb]);
                        if constexpr (kSplit) av[pb] = Tr::mma(lo, db, av[pb]);
                    }
                }
            }
            // ---- dx, and the per-token scalars x.v, dy.y', dy.x ----
            float sxv[4] = {0.f, 0.f, 0.f, 0.f}, sdy[4] = {0.f, 0.f, 0.f, 0.f}, sxy[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int pb = 0; pb < PB; ++pb) {
                TI xs[4], ds[4];
                tr4<TI>(XN, P_LD, 16 * w + 4 * kg, 16 * pb, lane, xs);
                tr4<TI>(DYN, P_LD, 16 * w + 4 * kg, 16 * pb, lane, ds);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float xv = Tr::to_f32(xs[i]), dv = Tr::to_f32(ds[i]);
                    sxv[i] += xv * av[pb][i];
                    sdy[i] += dv * ay[pb][i];
                    sxy[i] += dv * xv;
                    if constexpr (NS == 1) {
                        OS[(4 * kg + i) * P_LD + 16 * pb + r] = Tr::from_f32(dt_o[i] * av[pb][i] + Dh * dv);
                    } else {
                        // this slice's part of dx in fp32 (the skip term with slice 0's)
                        const int t = t0 + 16 * w + 4 * kg + i;
                        if (t < T)
                            a.dXp[tsl_x + (((size_t)b * T + t) * H + h) * P + 16 * pb + r] =
                                dt_o[i] * av[pb][i] + (sl == 0 ? Dh * dv : 0.f);
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sxv[i] = row16_sum(sxv[i]);
                sdy[i] = row16_sum(sdy[i]);
                sxy[i] = row16_sum(sxy[i]);
            }
            if (r == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const size_t o = bh * a.Tpad + t0 + 16 * w + 4 * kg + i;
                    a.rbuf[tsl + o] = sxv[i];
                    a.qbuf[tsl + o] = sdy[i] - dt_o[i] * sxv[i];
                    if (sl == 0) a.xybuf[o] = sxy[i];
                }
            }
            lam = wave_sum(lam);
            // shares 0-3 of Lambda at the tile's end, one per wavefront (k_bwd_fin adds the 8
            // shares in a fixed order)
            if (lane == 0) a.lamb[((bh * a.ntiles + tau) * NS + sl) * 8 + w] = lam;
            if constexpr (NS == 1) {
                __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
                constexpr int VPR = P * ES / 16;
                for (int v = lane; v < 16 * VPR; v += 64) {
                    const int rl = v / VPR, cv = v % VPR;
                    const u32x4 d =
                        *reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(OS + rl * P_LD) + cv * 16);
                    buf_st128(d, rdx, xo + (uint32_t)(16 * w + rl) * x_tok + (uint32_t)(cv * 16));
                }
            }
            // the next head into the other buffer (its last reads, head k - 1's, ended at the
            // barrier before this head); past the last head a harmless repeat of it
            stage((k + 1) & 1);
            issue(min(k + 2, hpb - 1));
            __syncthreads();
        }
    } else {
        // ================= role B: dC and dB, summed over the heads =================
        f32x4 accb[NB], accc[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            accb[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
            accc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        TileRegs<TI, P, NL, 256> hr, er;
        float pcr = 0.f, pce = 0.f;  // the loaded head's cs before the tile and at its end
        auto issue = [&](int k) {
            const int h = g * HG + blk * hpb + k;
            const size_t so = (((size_t)b * H + h) * a.ntiles + tau) * (size_t)(P * N);
            pcr = a.cs2[((size_t)b * H + h) * a.Tpad + max(t0 - 1, 0)];
            pce = a.cs2[((size_t)b * H + h) * a.Tpad + t0 + kBT - 1];
            hr.load(make_rsrc(reinterpret_cast<const TI *>(a.Hst) + so, (uint32_t)(P * N * ES)),
                    (uint32_t)(n0 * ES), (uint32_t)(N * ES), rt);
            er.load(make_rsrc(reinterpret_cast<const TI *>(a.Est) + so, (uint32_t)(P * N * ES)),
                    (uint32_t)(n0 * ES), (uint32_t)(N * ES), rt);
        };
        // writes the loaded head (head kh)'s h and E (row-major) into buffer sb, and its share of
        // Lambda at the tile's end from the entering state: 2^{cs_e - cs_r} <E, h>, from the loaded
        // pieces (h and E are loaded with the same offsets; spare units read 0)
        auto stage = [&](int kh, int sb) {
            TI *B0 = HB + sb * Cfg::BUF;
            hr.store_N(B0 + Cfg::HN, N_LD, rt);
            er.store_N(B0 + Cfg::EN, N_LD, rt);
            float lam = 0.f;
#pragma unroll
            for (int kq = 0; kq < decltype(hr)::K; ++kq)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const frag hv = hr.v[kq][i], ev = er.v[kq][i];
                    if constexpr (ES == 2) {
                        // pairs straight from the packed registers (v_dot2c_f32_bf16)
#define SSD_DOT2(e)                                                                                \
    lam = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(hv, hv, e, e + 1),                   \
                                          __builtin_shufflevector(ev, ev, e, e + 1), lam, false)
                        SSD_DOT2(0); SSD_DOT2(2); SSD_DOT2(4); SSD_DOT2(6);
#undef SSD_DOT2
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e) lam += hv[e] * ev[e];
                    }
                }
            lam = wave_sum(lam);
            const size_t bh = (size_t)b * H + g * HG + blk * hpb + kh;
            const float cs_r = (tau % a.tpc == 0) ? 0.f : pcr;
            if (lane == 0) a.lamb[((bh * a.ntiles + tau) * NS + sl) * 8 + 4 + w] = fast_exp2(pce - cs_r) * lam;
        };
        issue(0);
        stage(0, 0);
        issue(min(1, hpb - 1));
        __syncthreads();  // pairs with role A's
        for (int k = 0; k < hpb; ++k) {
            use_buffer(k & 1);
            const float cs_r = SC[0], cs_e = SC[1];
            const float cs_t = CS[trow];
            float cs_o[4], dt_o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                cs_o[i] = CS[16 * w + 4 * kg + i];
                dt_o[i] = DT[16 * w + 4 * kg + i];
            }
            // ---- dC: 2^{cs_t - cs_r} dY h + (P1 o W1) B, P1[t][j] = x_j . dy_t ----
            {
                f32x4 p1[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    p1[q] = f32x4{0.f, 0.f, 0.f, 0.f};
                    if (q <= w) {
#pragma unroll
                        for (int kp = 0; kp < KP; ++kp)
                            p1[q] = Tr::mma(Tr::lds_frag(XN + (16 * q + r) * P_LD + 32 * kp + 8 * kg),
                                            Tr::lds_frag(DYN + trow * P_LD + 32 * kp + 8 * kg), p1[q]);
                    }
                }
                f32x4 tmp[NB];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    tmp[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kp = 0; kp < KP; ++kp)
                        tmp[nb] = Tr::mma(Tr::lds_frag(DYN + trow * P_LD + 32 * kp + 8 * kg),
                                          tr_frag<TI>(HN, N_LD, 32 * kp + 8 * kg, 32 * kp + 8 * kg + 4, 16 * nb, lane),
                                          tmp[nb]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) tmp[nb][i] *= fast_exp2(cs_o[i] - cs_r);
                }
#pragma unroll
                for (int k2 = 0; k2 < kBT / 32; ++k2) {
                    if (k2 > kc) continue;
                    const frag m = make_a(p1, k2, true, cs_t, nullptr);
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        const TI *p = BT + (16 * nb + r) * T_LD + 32 * k2 + 4 * kg;
                        tmp[nb] = Tr::mma(m, lds_frag_split<TI>(p, p + 16), tmp[nb]);
                    }
                }
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) accc[nb] += tmp[nb];
            }
            // ---- dB: dt_t [2^{cs_e - cs_t} X E + (P2 o W2) C], P2[t][u] = dy_u . x_t ----
            {
                f32x4 p2[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    p2[q] = f32x4{0.f, 0.f, 0.f, 0.f};
                    if (q >= w) {
#pragma unroll
                        for (int kp = 0; kp < KP; ++kp)
                            p2[q] = Tr::mma(Tr::lds_frag(DYN + (16 * q + r) * P_LD + 32 * kp + 8 * kg),
                                            Tr::lds_frag(XN + trow * P_LD + 32 * kp + 8 * kg), p2[q]);
                    }
                }
                f32x4 tmp[NB];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    tmp[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kp = 0; kp < KP; ++kp)
                        tmp[nb] = Tr::mma(Tr::lds_frag(XN + trow * P_LD + 32 * kp + 8 * kg),
                                          tr_frag<TI>(EN, N_LD, 32 * kp + 8 * kg, 32 * kp + 8 * kg + 4, 16 * nb, lane),
                                          tmp[nb]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) tmp[nb][i] *= fast_exp2(cs_e - cs_o[i]);
                }
#pragma unroll
                for (int k2 = 0; k2 < kBT / 32; ++k2) {
                    if (k2 < kc) continue;
                    const frag m = make_a(p2, k2, false, cs_t, nullptr);
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        const TI *p = CT + (16 * nb + r) * T_LD + 32 * k2 + 4 * kg;
                        tmp[nb] = Tr::mma(m, lds_frag_split<TI>(p, p + 16), tmp[nb]);
                    }
                }
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) accb[nb][i] += dt_o[i] * tmp[nb][i];
            }
            // the next head into the other buffer, as in role A
            stage(min(k + 1, hpb - 1), (k + 1) & 1);
            issue(min(k + 2, hpb - 1));
            __syncthreads();
        }
        if (nblk == 1) {
            // the group's heads are all in this block: dB, dC in the storage type, real tokens only
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = t0 + 16 * w + 4 * kg + i;
                if (t < T) {
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        const size_t o = (((size_t)b * T + t) * G + g) * N + n0 + 16 * nb + r;
                        reinterpret_cast<TI *>(a.dB)[o] = Tr::from_f32(accb[nb][i]);
                        reinterpret_cast<TI *>(a.dC)[o] = Tr::from_f32(accc[nb][i]);
                    }
                }
            }
        } else {
            // dB, dC of this head block: part[b][t][blk][g][n] (fp32), added up by k_bwd_sum_bc
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const size_t o =
                        ((((size_t)b * a.Tpad + t0 + 16 * w + 4 * kg + i) * nblk + blk) * G + g) * N + n0 + 16 * nb + r;
                    a.dBp[o] = accb[nb][i];
                    a.dCp[o] = accc[nb][i];
                }
        }
    }
}

// ---------------------------------------------------------------------------
// k_bwd_fin: one wavefront per (batch, head, tile), a lane per token: Lambda
// down the tile from its end value (a suffix sum across the lanes), ddt =
// x.v + A Lambda, and the tile's shares of dA = sum dt Lambda and
// dD = sum dy.x. k_bwd_heads then adds the shares up per head in a fixed
// order (deterministic).
// ---------------------------------------------------------------------------
template <typename TI>
__global__ __launch_bounds__(256) void k_bwd_fin(BwdFinArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // (b H + h) ntiles + tau
    const int nt = a.ntiles;
    if (wid >= (int64_t)a.batch * a.H * nt) return;
    const int tau = (int)(wid % nt);
    const int64_t bh = wid / nt;
    const int h = (int)(bh % a.H), b = (int)(bh / a.H);
    const int t = tau * kBT + lane;
    const bool real = t < a.T;
    const size_t o = (size_t)bh * a.Tpad + t;
    const size_t od = ((size_t)b * a.T + t) * a.H + h;
    // the n slices' parts of the per-token scalars, added in slice order
    float q = 0.f, rv = 0.f;
    if (real)
        for (int sl = 0; sl < a.ns; ++sl) {
            q += a.qbuf[sl * a.tok_stride + o];
            rv += a.rbuf[sl * a.tok_stride + o];
        }
    float run = q;  // suffix sum over the lanes at and after this one
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
        const float v = __shfl_down(run, m);
        if (lane + m < 64) run += v;
    }
    for (int sl = 0; sl < a.ns; ++sl) {
        const float *lp = a.lamb + (wid * a.ns + sl) * 8;  // k_bwd_tile's 8 wavefront shares of slice sl
        run += ((lp[0] + lp[1]) + (lp[2] + lp[3])) + ((lp[4] + lp[5]) + (lp[6] + lp[7]));
    }
    float sdA = 0.f, sdD = 0.f;
    if (real) {
        reinterpret_cast<TI *>(a.ddt)[od] = Traits<TI>::from_f32(rv + a.A[h] * run);
        sdA = Traits<TI>::to_f32(reinterpret_cast<const TI *>(a.dt)[od]) * run;
        sdD = a.xybuf[o];
    }
#pragma unroll
    for (int m = 32; m > 0; m >>= 1) {
        sdA += __shfl_xor(sdA, m);
        sdD += __shfl_xor(sdD, m);
    }
    if (lane == 0) {
        a.dApart[wid] = sdA;
        a.dDpart[wid] = sdD;
    }
}

// dX from the n slices' fp32 parts, added in slice order, in the storage type.
template <typename TI>
__global__ __launch_bounds__(256) void k_bwd_dx(const float *__restrict__ dXp, TI *__restrict__ dX, int64_t n,
                                                int ns) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= n) return;  // n is a multiple of 4 (P is)
    f32x4 v = *reinterpret_cast<const f32x4 *>(dXp + i);
    for (int sl = 1; sl < ns; ++sl) v += *reinterpret_cast<const f32x4 *>(dXp + (size_t)sl * n + i);
    store4<TI>(dX + i, v);
}

__global__ __launch_bounds__(256) void k_bwd_heads(const float *__restrict__ dApart, const float *__restrict__ dDpart,
                                                   float *__restrict__ dA, float *__restrict__ dD, int batch, int H,
                                                   int nt) {
    __shared__ float sa[256], sd[256];
    const int h = blockIdx.x, tid = threadIdx.x;
    float va = 0.f, vd = 0.f;
    for (int i = tid; i < batch * nt; i += 256) {
        const int b = i / nt, tau = i - b * nt;
        const size_t o = ((size_t)b * H + h) * nt + tau;
        va += dApart[o];
        vd += dDpart[o];
    }
    sa[tid] = va;
    sd[tid] = vd;
    __syncthreads();
    for (int st = 128; st > 0; st >>= 1) {
        if (tid < st) {
            sa[tid] += sa[tid + st];
            sd[tid] += sd[tid + st];
        }
        __syncthreads();
    }
    if (tid == 0) {
        dA[h] = sa[0];
        dD[h] = sd[0];
    }
}

// dB, dC: the head blocks' partial sums added up and stored in the storage type.
template <typename TI>
__global__ __launch_bounds__(256) void k_bwd_sum_bc(const float *__restrict__ dBp, const float *__restrict__ dCp,
                                                    TI *__restrict__ dB, TI *__restrict__ dC, int64_t batch, int T,
                                                    int Tpad, int nblk, int G, int N) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = batch * T * G * N;
    if (i >= total) return;
    const int n = (int)(i % N);
    int64_t x = i / N;
    const int g = (int)(x % G);
    x /= G;
    const int t = (int)(x % T);
    const int64_t b = x / T;
    const size_t base = (((size_t)b * Tpad + t) * nblk * G + g) * N + n;
    float sb = 0.f, sc = 0.f;
    for (int k = 0; k < nblk; ++k) {
        sb += dBp[base + (size_t)k * G * N];
        sc += dCp[base + (size_t)k * G * N];
    }
    dB[i] = Traits<TI>::from_f32(sb);
    dC[i] = Traits<TI>::from_f32(sc);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
// The n slice of k_bwd_tile: the widest of N, N / 2, N / 4 (at least 32
// columns) whose work-group fits a CU's LDS; 0 when none does.
template <typename TI, int P, int N>
static constexpr int bwd_nl() {
    if constexpr (BwdCfg<TI, P, N>::kFits) return N;
    else if constexpr (N >= 64 && BwdCfg<TI, P, N / 2>::kFits) return N / 2;
    else if constexpr (N >= 128 && BwdCfg<TI, P, N / 4>::kFits) return N / 4;
    else return 0;
}

// Shapes the backward covers: k_bwd_tile fits with at most 4 n slices, and the
// state passes (the whole n axis per work-group) fit LDS and registers (fp32
// up to N 128).
template <typename TI, int P, int N>
static constexpr bool bwd_fits() {
    return bwd_nl<TI, P, N>() > 0 && sizeof(SpLds<TI, P, N>) <= 160 * 1024 && (sizeof(TI) == 2 || N <= 128);
}

template <typename TI, typename F>
static auto bwd_shape(int64_t P, int64_t N, F f) {
    using I32 = std::integral_constant<int, 32>;
    using I64 = std::integral_constant<int, 64>;
    using I128 = std::integral_constant<int, 128>;
    using I256 = std::integral_constant<int, 256>;
    auto pick = [&](auto Pc) {
        switch (N) {
            case 32: return f(Pc, I32{});
            case 64: return f(Pc, I64{});
            case 128: return f(Pc, I128{});
            case 256: return f(Pc, I256{});
            default: return decltype(f(Pc, I32{})){};
        }
    };
    if (P == 32) return pick(I32{});
    if (P == 64) return pick(I64{});
    return decltype(f(I32{}, I32{})){};
}

template <typename TI>
static bool bwd_shape_ok(int64_t P, int64_t N) {
    return bwd_shape<TI>(P, N, [](auto Pc, auto Nc) {
        return bwd_fits<TI, decltype(Pc)::value, decltype(Nc)::value>();
    });
}

bool bwd_supported(ssd_dtype dt, int64_t P, int64_t N) {
    return dt == SSD_BF16 ? bwd_shape_ok<bf16>(P, N) : bwd_shape_ok<float>(P, N);
}

template <typename TI>
static int bwd_ns(int64_t P, int64_t N) {
    return bwd_shape<TI>(P, N, [](auto Pc, auto Nc) {
        constexpr int Pv = decltype(Pc)::value, Nv = decltype(Nc)::value, nl = bwd_nl<TI, Pv, Nv>();
        return nl > 0 ? Nv / nl : 0;
    });
}

int bwd_nslices(ssd_dtype dt, int64_t P, int64_t N) {
    return dt == SSD_BF16 ? bwd_ns<bf16>(P, N) : bwd_ns<float>(P, N);
}

template <typename TI, int P, int N>
static ssd_status run_bwd(const BwdArgs &w, hipStream_t s) {
    if constexpr (!bwd_fits<TI, P, N>()) {
        return SSD_ERR_UNSUPPORTED;
    } else {
        constexpr int NL = bwd_nl<TI, P, N>(), NS = N / NL;
        const FwdArgs &f = w.f;
        const int ntiles = (int)(f.Tpad / kBT);
        StatePassArgs sp = {};
        sp.cs2 = f.cs2; sp.dtf = f.dtf; sp.H = (int)f.H; sp.G = (int)f.G; sp.T = (int)f.T;
        sp.Tpad = (int)f.Tpad; sp.ntiles = ntiles; sp.tpc = (int)(f.Q / kBT);
        const int nbh = (int)(f.batch * f.H);
        StatePassArgs rev = sp, fwd = sp;
        rev.U = w.dY; rev.V = f.C; rev.init = w.dF; rev.Sst = w.Est; rev.out = w.dinit;
        fwd.U = f.X; fwd.V = f.B; fwd.init = f.init; fwd.Sst = w.Hst; fwd.out = nullptr;
        const int nsl = state_pass_slices(nbh, N);
        hipError_t e = hipErrorInvalidValue;
        const dim3 grid((unsigned)(2 * nbh * nsl));
        if (nsl == 1) e = launch(k_state_passes<TI, P, N, N>, grid, dim3(64 * SP_NW), s, rev, fwd, nbh);
        if constexpr (N >= 128)
            if (nsl == 2) e = launch(k_state_passes<TI, P, N, N / 2>, grid, dim3(64 * SP_NW), s, rev, fwd, nbh);
        if constexpr (N >= 256)
            if (nsl == 4) e = launch(k_state_passes<TI, P, N, N / 4>, grid, dim3(64 * SP_NW), s, rev, fwd, nbh);
        if (e != hipSuccess) return SSD_ERR_HIP;
        BwdTileArgs ta = {};
        ta.X = f.X; ta.dY = w.dY; ta.B = f.B; ta.C = f.C; ta.dt = f.dt; ta.D = f.D;
        ta.Hst = w.Hst; ta.Est = w.Est; ta.cs2 = f.cs2; ta.dtf = f.dtf;
        ta.dX = w.dX; ta.rbuf = w.rbuf; ta.qbuf = w.qbuf; ta.xybuf = w.xybuf; ta.dBp = w.dBp; ta.dCp = w.dCp;
        ta.H = (int)f.H; ta.G = (int)f.G; ta.T = (int)f.T; ta.Tpad = (int)f.Tpad; ta.ntiles = ntiles;
        ta.tpc = (int)(f.Q / kBT); ta.nblk = w.nblk; ta.lamb = w.lamb;
        ta.dXp = w.dXp; ta.dB = w.dB; ta.dC = w.dC;
        ta.tok_stride = (size_t)(f.batch * f.H * f.Tpad);
        ta.dx_stride = (size_t)(f.batch * f.T * f.H * f.P);
        const int64_t tiles = f.batch * ntiles * f.G * w.nblk * NS;
        if (launch(k_bwd_tile<TI, P, N, NL>, dim3((unsigned)tiles), dim3(512), s, ta) != hipSuccess)
            return SSD_ERR_HIP;
        if constexpr (NS > 1) {
            const int64_t n = f.batch * f.T * f.H * f.P;
            if (launch(k_bwd_dx<TI>, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), s, (const float *)w.dXp,
                       (TI *)w.dX, n, NS) != hipSuccess)
                return SSD_ERR_HIP;
        }
        BwdFinArgs fa = {};
        fa.qbuf = w.qbuf; fa.rbuf = w.rbuf; fa.xybuf = w.xybuf; fa.lamb = w.lamb; fa.dt = f.dt; fa.A = f.A;
        fa.ddt = w.ddt; fa.tok_stride = ta.tok_stride; fa.ns = NS;
        fa.batch = (int)f.batch; fa.T = (int)f.T; fa.Tpad = (int)f.Tpad; fa.H = (int)f.H; fa.ntiles = ntiles;
        fa.dApart = w.dApart; fa.dDpart = w.dDpart;
        const int64_t waves = f.batch * f.H * ntiles;
        if (launch(k_bwd_fin<TI>, dim3((unsigned)((waves + 3) / 4)), dim3(256), s, fa) != hipSuccess ||
            launch(k_bwd_heads, dim3((unsigned)f.H), dim3(256), s, (const float *)w.dApart, (const float *)w.dDpart,
                   w.dA, w.dD, (int)f.batch, (int)f.H, ntiles) != hipSuccess)
            return SSD_ERR_HIP;
        if (w.nblk == 1) return SSD_OK;  // k_bwd_tile wrote dB and dC
        const int64_t n = f.batch * f.T * f.G * N;
        return launch(k_bwd_sum_bc<TI>, dim3((unsigned)((n + 255) / 256)), dim3(256), s, (const float *)w.dBp,
                      (const float *)w.dCp, (TI *)w.dB, (TI *)w.dC, f.batch, (int)f.T, (int)f.Tpad, w.nblk,
                      (int)f.G, N) == hipSuccess
                   ? SSD_OK
                   : SSD_ERR_HIP;
    }
}

template <typename TI, int P>
static ssd_status bwd_n(const BwdArgs &w, hipStream_t s) {
    switch (w.f.N) {
        case 32: return run_bwd<TI, P, 32>(w, s);
        case 64: return run_bwd<TI, P, 64>(w, s);
        case 128: return run_bwd<TI, P, 128>(w, s);
        case 256: return run_bwd<TI, P, 256>(w, s);
        default: return SSD_ERR_UNSUPPORTED;
    }
}

template <typename TI>
static ssd_status bwd_p(const BwdArgs &w, hipStream_t s) {
    switch (w.f.P) {
        case 32: return bwd_n<TI, 32>(w, s);
        case 64: return bwd_n<TI, 64>(w, s);
        default: return SSD_ERR_UNSUPPORTED;
    }
}

ssd_status launch_bwd(const BwdArgs &w, hipStream_t s) {
    return w.f.dtype == SSD_BF16 ? bwd_p<bf16>(w, s) : bwd_p<float>(w, s);
}

}  // namespace ssd
