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
// leaving this one; the forward state pass forms that product from its fp32
// state, and the running sum restarts from it at every tile. dA sums
// dt_t Lambda_t, which cancels heavily; a running sum over the whole
// sequence would carry every rounding error of the per-token scalars (bf16
// operands) into all earlier tokens.
//
// The work follows the chunked form of the forward (the reading report's
// section 3.1: quadratic diagonal blocks, rank-N blocks through states handed
// across block boundaries), in 64-token tiles:
//   k_state_pass<rev>  per (batch, head), tiles in reverse: the adjoint
//                      arriving at every tile from the tokens after it,
//                      E = a ds of the next token (stored in the storage
//                      type), and finally a_0 ds_0, the initial state's
//                      gradient;
//   k_state_pass<fwd>  per (batch, head): the state entering every tile
//                      (stored in the storage type) and Lambda at every
//                      tile's end;
//   k_bwd_tile         per (batch, tile, group, block of heads): everything
//                      inside the tile from h (entering state) and E (arriving
//                      adjoint): y', v, dx, the per-token scalars of Lambda,
//                      and dB, dC summed over the block's heads;
//   k_bwd_fin          per (batch, head, tile): Lambda down the tile, ddt, and
//                      the tile's shares of dA, dD (k_bwd_heads adds them up);
//   k_bwd_sum_bc       dB and dC summed over head blocks, in the storage type.
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

// Four consecutive elements from LDS.
template <typename TI>
__device__ __forceinline__ void lds_ld4(TI *d, const TI *p) {
    if constexpr (sizeof(TI) == 2) {
        const bf16x4 v = *reinterpret_cast<const bf16x4 *>(p);
        d[0] = v[0]; d[1] = v[1]; d[2] = v[2]; d[3] = v[3];
    } else {
        const f32x4 v = *reinterpret_cast<const f32x4 *>(p);
        d[0] = v[0]; d[1] = v[1]; d[2] = v[2]; d[3] = v[3];
    }
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
// k_state_pass: one work-group (8 wavefronts) per (batch, head) walks the
// tiles (backwards when kRev) with the P x N state in matrix-core
// accumulators, wave w owning the state's columns n in blocks w, w + 8, ...
// Before each tile it stores the state it carries into Sst[tile] ([p][n],
// storage type); after the last one it writes the state (fp32) to `out`.
//   forward: S <- 2^{cs_e - cs_r} S + sum_t 2^{cs_e - cs'_t} x_t B_t^T
//   reverse: S <- 2^{cs_e - cs_r} S + sum_t 2^{cs_t - cs_r} dy_t C_t^T
// (U = X or dY, V = B or C).
// ---------------------------------------------------------------------------
template <typename TI, int P, int N, bool kRev>
__global__ __launch_bounds__(512) void k_state_pass(StatePassArgs a) {
    using Tr = Traits<TI>;
    using frag = typename Tr::frag;
    constexpr int ES = Tr::kBytes, PAD = 16 / ES, T_LD = kBT + PAD;
    constexpr int NW = 8, NTH = 64 * NW;  // wavefronts; wave w owns n-blocks w, w + NW, ...
    constexpr int PB = P / 16, NB = N / 16, NBW = (NB + NW - 1) / NW;
    __shared__ __attribute__((aligned(16))) TI UT[P * T_LD];
    __shared__ __attribute__((aligned(16))) TI VT[N * T_LD];
    __shared__ float WT[kBT];
    // the state each tile stores goes through LDS ([p][n], padded rows) so that
    // it leaves as whole 16-byte row pieces: written straight from the
    // accumulators each store instruction would cover 16 rows x 32 bytes
    constexpr int S_LD = N + PAD;
    __shared__ __attribute__((aligned(16))) TI SS[P * S_LD];

    const int H = a.H, G = a.G, T = a.T;
    const int bh = blockIdx.x, b = bh / H, h = bh - b * H, g = (h * G) / H;
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
                v = *reinterpret_cast<const f32x4 *>(a.init + ((size_t)bh * P + 16 * pb + r) * N + 16 * nb + 4 * kg);
            acc[pb][j] = v;
        }
    const int ntiles = a.ntiles;
    // a tile's U, V, per-token exponent terms (and, forward, the adjoint
    // arriving at it), loaded two tiles ahead into one of two register sets
    TileRegs<TI, kBT, P, NTH> ur[2];
    TileRegs<TI, kBT, N, NTH> vr[2];
    float wcs[2] = {0.f, 0.f};                   // this thread's token term (tid < 64)
    float pcs_r[2] = {0.f, 0.f}, pcs_e[2] = {0.f, 0.f};
    TI e4[2][PB][NBW][4];
    auto issue = [&](int tau, auto Sc) {
        constexpr int S = decltype(Sc)::value;
        const int t0 = tau * kBT;
        ur[S].load(ru, (uint32_t)(((size_t)t0 * H + h) * P * ES), (uint32_t)(H * P * ES), tid);
        vr[S].load(rv, (uint32_t)(((size_t)t0 * G + g) * N * ES), (uint32_t)(G * N * ES), tid);
        pcs_r[S] = (tau % a.tpc == 0) ? 0.f : cs[t0 - 1];
        pcs_e[S] = cs[t0 + kBT - 1];
        wcs[S] = kRev ? cs[t0 + (tid & 63)] : cp[t0 + (tid & 63)];
        if constexpr (!kRev) {
            const TI *E = reinterpret_cast<const TI *>(a.Est) + ((size_t)bh * ntiles + tau) * P * N;
#pragma unroll
            for (int pb = 0; pb < PB; ++pb)
#pragma unroll
                for (int j = 0; j < NBW; ++j) {
                    const int nb = w + NW * j;
                    if (nb < NB) lds_ld4<TI>(e4[S][pb][j], E + (16 * pb + r) * N + 16 * nb + 4 * kg);
                }
        }
    };
    auto tile_of = [&](int it) { return kRev ? max(ntiles - 1 - it, 0) : min(it, ntiles - 1); };
    issue(tile_of(0), std::integral_constant<int, 0>{});
    issue(tile_of(1), std::integral_constant<int, 1>{});
    auto step = [&](int it, auto Sc) {
        constexpr int S = decltype(Sc)::value;
        const int tau = tile_of(it);
        TI *dst = reinterpret_cast<TI *>(a.Sst) + ((size_t)bh * ntiles + tau) * P * N;
#pragma unroll
        for (int pb = 0; pb < PB; ++pb)
#pragma unroll
            for (int j = 0; j < NBW; ++j) {
                const int nb = w + NW * j;
                if (nb < NB) store4<TI>(SS + (16 * pb + r) * S_LD + 16 * nb + 4 * kg, acc[pb][j]);
            }
        const float cs_r = pcs_r[S], cs_e = pcs_e[S];
        if (tid < kBT) WT[tid] = kRev ? fast_exp2(wcs[S] - cs_r) : fast_exp2(cs_e - wcs[S]);
        __syncthreads();  // SS and WT visible; the previous tile's reads of UT / VT are done
        {
            constexpr int VPRS = N * ES / 16;  // 16-byte pieces per state row
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
        TI ee[PB][NBW][4];
        if constexpr (!kRev) {
#pragma unroll
            for (int pb = 0; pb < PB; ++pb)
#pragma unroll
                for (int j = 0; j < NBW; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i) ee[pb][j][i] = e4[S][pb][j][i];
        }
        // the tile after next is loaded while this one is computed (past the end: a reload)
        issue(tile_of(it + 2), Sc);
        const float dec = fast_exp2(cs_e - cs_r);
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
        if constexpr (!kRev) {
            // Lambda at the tile's end: <E of this tile, state after it>
            float part = 0.f;
#pragma unroll
            for (int pb = 0; pb < PB; ++pb)
#pragma unroll
                for (int j = 0; j < NBW; ++j) {
                    const int nb = w + NW * j;
                    if (nb < NB) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) part += Tr::to_f32(ee[pb][j][i]) * acc[pb][j][i];
                    }
                }
#pragma unroll
            for (int m = 32; m > 0; m >>= 1) part += __shfl_xor(part, m);
            // one share per wavefront, added up by k_bwd_fin in a fixed order
            if (lane == 0) a.lamb[((size_t)bh * ntiles + tau) * NW + w] = part;
        }
        __syncthreads();
    };
    for (int it = 0; it < ntiles; it += 2) {
        step(it, std::integral_constant<int, 0>{});
        if (it + 1 < ntiles) step(it + 1, std::integral_constant<int, 1>{});
    }
    if (a.out) {
#pragma unroll
        for (int pb = 0; pb < PB; ++pb)
#pragma unroll
            for (int j = 0; j < NBW; ++j) {
                const int nb = w + NW * j;
                if (nb < NB)
                    *reinterpret_cast<f32x4 *>(a.out + ((size_t)bh * P + 16 * pb + r) * N + 16 * nb + 4 * kg) =
                        acc[pb][j];
            }
    }
}

// ---------------------------------------------------------------------------
// k_bwd_tile: LDS layout and the work of one (batch, tile, group, head block).
// ---------------------------------------------------------------------------
template <typename TI, int P, int N>
struct BwdCfg {
    static constexpr int ES = sizeof(TI), PAD = 16 / ES;
    static constexpr int PB = P / 16, NB = N / 16, NK = N / 32, KP = P / 32;
    static constexpr int T_LD = kBT + PAD, P_LD = P + PAD, N_LD = N + PAD;
    // element offsets (storage type)
    static constexpr int BT_OFF = 0;                       // B^T [n][t]
    static constexpr int CT_OFF = BT_OFF + N * T_LD;       // C^T [n][t]
    static constexpr int XT_OFF = CT_OFF + N * T_LD;       // X^T [p][t]
    static constexpr int DYT_OFF = XT_OFF + P * T_LD;      // dY^T [p][t]
    static constexpr int XN_OFF = DYT_OFF + P * T_LD;      // X [t][p]
    static constexpr int DYN_OFF = XN_OFF + kBT * P_LD;    // dY [t][p]
    static constexpr int HN_OFF = DYN_OFF + kBT * P_LD;    // h [p][n]
    static constexpr int EN_OFF = HN_OFF + P * N_LD;       // E [p][n]
    static constexpr int HT_OFF = EN_OFF + P * N_LD;       // h^T [n][p]
    static constexpr int ET_OFF = HT_OFF + N * P_LD;       // E^T [n][p]
    static constexpr int OS_OFF = ET_OFF + N * P_LD;       // dX staging, 16 rows per wave
    static constexpr int ELEMS = OS_OFF + 4 * 16 * P_LD;
    static constexpr int F_OFF = (ELEMS * ES + 15) / 16 * 16;  // bytes: cs, cs', dt of the tile
    static constexpr int LDS = F_OFF + 3 * kBT * 4;
    static constexpr bool kFits = LDS <= 160 * 1024 && P % 32 == 0 && N % 32 == 0;
};

// 8 wavefronts in two roles over the same staged tile and head: waves 0-3
// (16 token rows each) form y', v, dX and the per-token scalars; waves 4-7
// (same rows) form x.dy products, dC and dB. The roles share no results, so
// the two waves on each SIMD overlap.
template <typename TI, int P, int N>
__global__ __launch_bounds__(512, 1) void k_bwd_tile(BwdTileArgs a) {
    using Tr = Traits<TI>;
    using frag = typename Tr::frag;
    using Cfg = BwdCfg<TI, P, N>;
    constexpr int ES = Cfg::ES, PB = Cfg::PB, NB = Cfg::NB, NK = Cfg::NK, KP = Cfg::KP;
    constexpr int T_LD = Cfg::T_LD, P_LD = Cfg::P_LD, N_LD = Cfg::N_LD;
    __shared__ __attribute__((aligned(16))) char smem[Cfg::LDS];
    TI *const L = reinterpret_cast<TI *>(smem);
    TI *BT = L + Cfg::BT_OFF, *CT = L + Cfg::CT_OFF, *XT = L + Cfg::XT_OFF, *DYT = L + Cfg::DYT_OFF;
    TI *XN = L + Cfg::XN_OFF, *DYN = L + Cfg::DYN_OFF, *HN = L + Cfg::HN_OFF, *EN = L + Cfg::EN_OFF;
    TI *HT = L + Cfg::HT_OFF, *ET = L + Cfg::ET_OFF;
    float *CS = reinterpret_cast<float *>(smem + Cfg::F_OFF), *CP = CS + kBT, *DT = CP + kBT;

    const int H = a.H, G = a.G, T = a.T, HG = H / G, nblk = a.nblk, hpb = HG / nblk;
    int x = blockIdx.x;
    const int blk = x % nblk;
    x /= nblk;
    const int g = x % G;
    x /= G;
    const int tau = x % a.ntiles;
    const int b = x / a.ntiles;
    const int t0 = tau * kBT;
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
    stage_T<TI, kBT, N, NTH, false>(rb, (uint32_t)(((size_t)t0 * G + g) * N * ES), b_tok, BT, T_LD, tid,
                                    [](int) { return 1.f; });
    stage_T<TI, kBT, N, NTH, false>(rc, (uint32_t)(((size_t)t0 * G + g) * N * ES), b_tok, CT, T_LD, tid,
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
        const uint32_t grow = (uint32_t)((t0 * G + g) * N * ES);
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
        float pcs = 0.f, pcp = 0.f, pdt = 0.f;  // token t0 + (tid & 63) of the prefetched head
        auto issue = [&](int k) {
            const int h = g * HG + blk * hpb + k;
            const size_t bh = (size_t)b * H + h;
            const uint32_t xo = (uint32_t)(((size_t)t0 * H + h) * P * ES);
            xr.load(rx, xo, x_tok, rt);
            dyr.load(rdy, xo, x_tok, rt);
            const int t = t0 + (tid & 63);
            pcs = a.cs2[bh * a.Tpad + t];
            pcp = a.dtf[bh * a.Tpad + t];
            pdt = t < T ? Tr::to_f32(reinterpret_cast<const TI *>(a.dt)[((size_t)b * T + t) * H + h]) : 0.f;
        };
        issue(0);
        for (int k = 0; k < hpb; ++k) {
            const int h = g * HG + blk * hpb + k;
            const size_t bh = (size_t)b * H + h;
            const float *cs = a.cs2 + bh * a.Tpad + t0;
            const float cs_r = (tau % a.tpc == 0) ? 0.f : cs[-1];
            const float cs_e = cs[kBT - 1];
            const float Dh = a.D[h];
            const uint32_t xo = (uint32_t)(((size_t)t0 * H + h) * P * ES);
            __syncthreads();  // the previous head's reads are done
            if (tid < kBT) {
                CS[tid] = pcs;
                CP[tid] = pcp;
                DT[tid] = pdt;
            }
            xr.template store_T<false>(XT, T_LD, rt, [](int) { return 1.f; });
            xr.store_N(XN, P_LD, rt);
            dyr.template store_T<false>(DYT, T_LD, rt, [](int) { return 1.f; });
            dyr.store_N(DYN, P_LD, rt);
            __syncthreads();
            issue(min(k + 1, hpb - 1));  // past the last head: a harmless reload
            const float cs_t = CS[trow];
            float cs_o[4], dt_o[4];  // output rows t = 16 w + 4 kg + i
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                cs_o[i] = CS[16 * w + 4 * kg + i];
                dt_o[i] = DT[16 * w + 4 * kg + i];
            }
            // ---- y' (scan output) and v = ds B, both [t][p] ----
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
                        const TI *p = XT + (16 * pb + r) * T_LD + 32 * k2 + 4 * kg;
                        const frag xb = lds_frag_split<TI>(p, p + 16);
                        ay[pb] = Tr::mma(m, xb, ay[pb]);
                        if constexpr (kSplit) ay[pb] = Tr::mma(lo, xb, ay[pb]);
                    }
                }
                if (k2 >= kc) {
                    frag lo;
                    const frag m = make_a(g2, k2, false, cs_t, kSplit ? &lo : nullptr);
#pragma unroll
                    for (int pb = 0; pb < PB; ++pb) {
                        const TI *p = DYT + (16 * pb + r) * T_LD + 32 * k2 + 4 * kg;
                        const frag db = lds_frag_split<TI>(p, p + 16);
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
                lds_ld4<TI>(xs, XT + (16 * pb + r) * T_LD + 16 * w + 4 * kg);
                lds_ld4<TI>(ds, DYT + (16 * pb + r) * T_LD + 16 * w + 4 * kg);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float xv = Tr::to_f32(xs[i]), dv = Tr::to_f32(ds[i]);
                    sxv[i] += xv * av[pb][i];
                    sdy[i] += dv * ay[pb][i];
                    sxy[i] += dv * xv;
                    OS[(4 * kg + i) * P_LD + 16 * pb + r] = Tr::from_f32(dt_o[i] * av[pb][i] + Dh * dv);
                }
            }
#pragma unroll
            for (int m = 1; m < 16; m <<= 1)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sxv[i] += __shfl_xor(sxv[i], m);
                    sdy[i] += __shfl_xor(sdy[i], m);
                    sxy[i] += __shfl_xor(sxy[i], m);
                }
            if (r == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const size_t o = bh * a.Tpad + t0 + 16 * w + 4 * kg + i;
                    a.rbuf[o] = sxv[i];
                    a.qbuf[o] = sdy[i] - dt_o[i] * sxv[i];
                    a.xybuf[o] = sxy[i];
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            constexpr int VPR = P * ES / 16;
            for (int v = lane; v < 16 * VPR; v += 64) {
                const int rl = v / VPR, cv = v % VPR;
                const u32x4 d =
                    *reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(OS + rl * P_LD) + cv * 16);
                buf_st128(d, rdx, xo + (uint32_t)(16 * w + rl) * x_tok + (uint32_t)(cv * 16));
            }
        }
    } else {
        // ================= role B: dC and dB, summed over the heads =================
        f32x4 accb[NB], accc[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            accb[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
            accc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        TileRegs<TI, P, N, 256> hr, er;
        auto issue = [&](int k) {
            const int h = g * HG + blk * hpb + k;
            const size_t so = (((size_t)b * H + h) * a.ntiles + tau) * (size_t)(P * N);
            hr.load(make_rsrc(reinterpret_cast<const TI *>(a.Hst) + so, (uint32_t)(P * N * ES)), 0u,
                    (uint32_t)(N * ES), rt);
            er.load(make_rsrc(reinterpret_cast<const TI *>(a.Est) + so, (uint32_t)(P * N * ES)), 0u,
                    (uint32_t)(N * ES), rt);
        };
        issue(0);
        for (int k = 0; k < hpb; ++k) {
            const int h = g * HG + blk * hpb + k;
            const size_t bh = (size_t)b * H + h;
            const float *cs = a.cs2 + bh * a.Tpad + t0;
            const float cs_r = (tau % a.tpc == 0) ? 0.f : cs[-1];
            const float cs_e = cs[kBT - 1];
            __syncthreads();  // the previous head's reads are done
            hr.store_N(HN, N_LD, rt);
            hr.template store_T<false>(HT, P_LD, rt, [](int) { return 1.f; });
            er.store_N(EN, N_LD, rt);
            er.template store_T<false>(ET, P_LD, rt, [](int) { return 1.f; });
            __syncthreads();
            issue(min(k + 1, hpb - 1));
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
                                          Tr::lds_frag(HT + (16 * nb + r) * P_LD + 32 * kp + 8 * kg), tmp[nb]);
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
                                          Tr::lds_frag(ET + (16 * nb + r) * P_LD + 32 * kp + 8 * kg), tmp[nb]);
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
        }
        // dB, dC of this head block: part[b][t][blk][g][n] (fp32)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const size_t o =
                    ((((size_t)b * a.Tpad + t0 + 16 * w + 4 * kg + i) * nblk + blk) * G + g) * N + 16 * nb + r;
                a.dBp[o] = accb[nb][i];
                a.dCp[o] = accc[nb][i];
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
    const float q = real ? a.qbuf[o] : 0.f;
    float run = q;  // suffix sum over the lanes at and after this one
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
        const float v = __shfl_down(run, m);
        if (lane + m < 64) run += v;
    }
    {
        const float *lp = a.lamb + wid * 8;  // the state pass's 8 wavefront shares
        run += ((lp[0] + lp[1]) + (lp[2] + lp[3])) + ((lp[4] + lp[5]) + (lp[6] + lp[7]));
    }
    float sdA = 0.f, sdD = 0.f;
    if (real) {
        reinterpret_cast<TI *>(a.ddt)[od] = Traits<TI>::from_f32(a.rbuf[o] + a.A[h] * run);
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
template <typename TI, int P, int N>
static constexpr bool bwd_fits() {
    return BwdCfg<TI, P, N>::kFits;
}

template <typename TI>
static bool bwd_shape_ok(int64_t P, int64_t N) {
    auto f = [](auto Pc, auto Nc) { return bwd_fits<TI, decltype(Pc)::value, decltype(Nc)::value>(); };
    using I32 = std::integral_constant<int, 32>;
    using I64 = std::integral_constant<int, 64>;
    using I128 = std::integral_constant<int, 128>;
    if (P == 32 && N == 32) return f(I32{}, I32{});
    if (P == 32 && N == 64) return f(I32{}, I64{});
    if (P == 32 && N == 128) return f(I32{}, I128{});
    if (P == 64 && N == 32) return f(I64{}, I32{});
    if (P == 64 && N == 64) return f(I64{}, I64{});
    if (P == 64 && N == 128) return f(I64{}, I128{});
    return false;
}

bool bwd_supported(ssd_dtype dt, int64_t P, int64_t N) {
    return dt == SSD_BF16 ? bwd_shape_ok<bf16>(P, N) : bwd_shape_ok<float>(P, N);
}

template <typename TI, int P, int N>
static ssd_status run_bwd(const BwdArgs &w, hipStream_t s) {
    if constexpr (!bwd_fits<TI, P, N>()) {
        return SSD_ERR_UNSUPPORTED;
    } else {
        const FwdArgs &f = w.f;
        const int ntiles = (int)(f.Tpad / kBT);
        StatePassArgs sp = {};
        sp.cs2 = f.cs2; sp.dtf = f.dtf; sp.H = (int)f.H; sp.G = (int)f.G; sp.T = (int)f.T;
        sp.Tpad = (int)f.Tpad; sp.ntiles = ntiles; sp.tpc = (int)(f.Q / kBT);
        const dim3 grid_bh((unsigned)(f.batch * f.H));
        sp.U = w.dY; sp.V = f.C; sp.init = w.dF; sp.Sst = w.Est; sp.out = w.dinit;
        if (launch(k_state_pass<TI, P, N, true>, grid_bh, dim3(512), s, sp) != hipSuccess) return SSD_ERR_HIP;
        sp.U = f.X; sp.V = f.B; sp.init = f.init; sp.Sst = w.Hst; sp.out = nullptr;
        sp.Est = w.Est; sp.lamb = w.lamb;
        if (launch(k_state_pass<TI, P, N, false>, grid_bh, dim3(512), s, sp) != hipSuccess) return SSD_ERR_HIP;
        BwdTileArgs ta = {};
        ta.X = f.X; ta.dY = w.dY; ta.B = f.B; ta.C = f.C; ta.dt = f.dt; ta.D = f.D;
        ta.Hst = w.Hst; ta.Est = w.Est; ta.cs2 = f.cs2; ta.dtf = f.dtf;
        ta.dX = w.dX; ta.rbuf = w.rbuf; ta.qbuf = w.qbuf; ta.xybuf = w.xybuf; ta.dBp = w.dBp; ta.dCp = w.dCp;
        ta.H = (int)f.H; ta.G = (int)f.G; ta.T = (int)f.T; ta.Tpad = (int)f.Tpad; ta.ntiles = ntiles;
        ta.tpc = (int)(f.Q / kBT); ta.nblk = w.nblk;
        const int64_t tiles = f.batch * ntiles * f.G * w.nblk;
        if (launch(k_bwd_tile<TI, P, N>, dim3((unsigned)tiles), dim3(512), s, ta) != hipSuccess) return SSD_ERR_HIP;
        BwdFinArgs fa = {};
        fa.qbuf = w.qbuf; fa.rbuf = w.rbuf; fa.xybuf = w.xybuf; fa.lamb = w.lamb; fa.dt = f.dt; fa.A = f.A;
        fa.ddt = w.ddt;
        fa.batch = (int)f.batch; fa.T = (int)f.T; fa.Tpad = (int)f.Tpad; fa.H = (int)f.H; fa.ntiles = ntiles;
        fa.dApart = w.dApart; fa.dDpart = w.dDpart;
        const int64_t waves = f.batch * f.H * ntiles;
        if (launch(k_bwd_fin<TI>, dim3((unsigned)((waves + 3) / 4)), dim3(256), s, fa) != hipSuccess ||
            launch(k_bwd_heads, dim3((unsigned)f.H), dim3(256), s, (const float *)w.dApart, (const float *)w.dDpart,
                   w.dA, w.dD, (int)f.batch, (int)f.H, ntiles) != hipSuccess)
            return SSD_ERR_HIP;
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
