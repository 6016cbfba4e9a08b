// Chunked SSD forward for gfx950.
//
// The method ("Transformers are SSMs" reading report, section 3.1): split the
// sequence into chunks of Q tokens; inside a chunk the output is an
// attention-like quadratic product with the decay mask (the diagonal blocks),
// and everything a chunk receives from earlier chunks passes through one
// P x N state per (batch, head), handed from each chunk to the next (the
// low-rank off-diagonal blocks).
//
// Three kernels, launched in this order on the caller's stream:
//   k_dt_cumsum   per (batch, chunk, head block): dt -> chunk-local inclusive
//                 prefix sum of dt*A in base 2 (cs2), and cs' = cs2 - log2(dt),
//                 both laid out (batch, head, token) fp32. With cs', the
//                 weight dt_j exp2(cs_i - cs_j) of token j seen from token i is
//                 one exponential, exp2(cs_i - cs'_j).
//   k_chunk_cb    per (batch, chunk, group, row tile): G = C B^T for the lower
//                 64 x 64 tiles of each chunk's Q x Q block (matrix cores).
//                 C B^T depends on the group only, so it is formed once and
//                 shared by every head of the group.
//   k_chunk_walk  per (batch, head): walks the chunks in order with the state
//                 held in matrix-core accumulators. Per 64-token row tile it
//                 forms Y = exp(cs_i) C_i h_in^T            (state -> output)
//                                + sum_{J<I} (L o G)_IJ dt X_J (earlier tiles)
//                                + (L o G)_II dt X_I          (masked diagonal)
//                                + D x_i                      (skip term)
//                 and updates the state h <- decay * h + X^T diag(w) B
//                 (chunk state and state passing fused). X, Y and the state
//                 cross HBM once; the state never leaves the chip until the
//                 final state is written.
//
// Masks are never stored. For tiles below the diagonal the decay factorises
// through the tile's last token e: L_ij = exp(cs_i - cs_e) exp(cs_e - cs_j),
// both factors <= 1, so the column factor goes into a scaled copy of X and the
// row factor is applied to the 16x16 accumulators. On the diagonal tile the
// mask is built per element in registers, with j > i selected to zero before
// the exponential is used.
#include <utility>

#include "ssd_common.h"
#include "ssd_internal.h"

namespace ssd {

// ---------------------------------------------------------------------------
// k_dt_cumsum: one work-group per (batch, chunk, block of 16 heads)
// ---------------------------------------------------------------------------
constexpr int kCumsumHeads = 16;

template <typename TI, int Q>
__global__ __launch_bounds__(256) void k_dt_cumsum(const TI *__restrict__ dt,
                                                   const float *__restrict__ A,
                                                   float *__restrict__ cs2,
                                                   float *__restrict__ dtf, int T, int H,
                                                   int nC, int Tpad) {
    constexpr int ES = Traits<TI>::kBytes;
    constexpr int LD = Q + 1;
    __shared__ float tile[kCumsumHeads * LD];
    const int hblocks = (H + kCumsumHeads - 1) / kCumsumHeads;
    int x = blockIdx.x;
    const int c = x % nC;
    x /= nC;
    const int hb = x % hblocks;
    const int b = x / hblocks;
    const int h0 = hb * kCumsumHeads;
    const int Hb = min(kCumsumHeads, H - h0);
    const int t0 = c * Q;
    const rsrc_t r = make_rsrc(reinterpret_cast<const char *>(dt) + (size_t)b * T * H * ES,
                               (uint32_t)((size_t)T * H * ES));
    // one token row per thread: all of its loads are issued before any is used
    for (int t = threadIdx.x; t < Q; t += 256) {
        float v[kCumsumHeads];
#pragma unroll
        for (int hl = 0; hl < kCumsumHeads; ++hl) {
            const uint32_t off =
                (hl < Hb && t0 + t < T) ? (uint32_t)(((t0 + t) * H + h0 + hl) * ES) : kOOB;
            if constexpr (ES == 2) {
                v[hl] = (float)__builtin_bit_cast(bf16, buf_ld16(r, off));
            } else {
                v[hl] = __builtin_bit_cast(float, buf_ld32(r, off));
            }
        }
#pragma unroll
        for (int hl = 0; hl < kCumsumHeads; ++hl) tile[hl * LD + t] = v[hl];
    }
    __syncthreads();
    constexpr int PER = Q / 64;  // tokens per lane
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    for (int hl = w; hl < Hb; hl += 4) {
        const int h = h0 + hl;
        const float a2 = A[h] * kLog2e;
        float d[PER], s[PER];
        float run = 0.f;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            d[k] = tile[hl * LD + lane * PER + k];
            run += d[k] * a2;
            s[k] = run;
        }
        // exclusive scan of the per-lane sums across the wavefront
        float incl = run;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float up = __shfl_up(incl, off, 64);
            if (lane >= off) incl += up;
        }
        const float excl = incl - run;
        float *o = cs2 + ((size_t)b * H + h) * Tpad + t0 + lane * PER;
        float *od = dtf + ((size_t)b * H + h) * Tpad + t0 + lane * PER;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            o[k] = s[k] + excl;
            // log2(0) = -inf, so a zero step (or a padded token) gets cs' = +inf
            // and every factor exp2(x - cs') built from it is exactly 0
            od[k] = s[k] + excl - __builtin_amdgcn_logf(d[k]);
        }
    }
}

// ---------------------------------------------------------------------------
// k_chunk_cb: G[b, g, c, pair(I, J)] = C_I B_J^T, J <= I, one 64 x 64 tile
// per work-group; every operand load is issued before the first product.
// ---------------------------------------------------------------------------
__host__ __device__ constexpr int pair_index(int I, int J) { return I * (I + 1) / 2 + J; }

template <typename TI, int Q, int N>
__global__ __launch_bounds__(256) void k_chunk_cb(const TI *__restrict__ Bm,
                                                  const TI *__restrict__ Cm, TI *__restrict__ Gout,
                                                  int T, int G, int nC, uint32_t g_bytes) {
    using Tr = Traits<TI>;
    using frag = typename Tr::frag;
    constexpr int ES = Tr::kBytes;
    constexpr int NT = Q / 64;
    constexpr int NP = NT * (NT + 1) / 2;
    constexpr int NK = (N + 31) / 32;
    int x = blockIdx.x;
    const int pr = x % NP;
    x /= NP;
    const int g = x % G;
    x /= G;
    const int c = x % nC;
    const int b = x / nC;
    int I = 0;
    while ((I + 1) * (I + 2) / 2 <= pr) ++I;
    const int J = pr - I * (I + 1) / 2;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r = lane & 15, kg = lane >> 4;
    const size_t slab = (size_t)T * G * N * ES;
    const rsrc_t rb = make_rsrc(reinterpret_cast<const char *>(Bm) + b * slab, (uint32_t)slab);
    const rsrc_t rc = make_rsrc(reinterpret_cast<const char *>(Cm) + b * slab, (uint32_t)slab);
    const rsrc_t rg = make_rsrc(Gout, g_bytes);
    const int t0 = c * Q;
    const int ti = t0 + I * 64 + 16 * w + r;  // this lane's A row (token)
    frag ca[NK], bb[4][NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
        const int n0 = kk * 32 + 8 * kg;
        ca[kk] = Tr::load_frag(rc, (ti < T && n0 < N) ? (uint32_t)(((ti * G + g) * N + n0) * ES) : kOOB);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            const int tj = t0 + J * 64 + 16 * cb + r;
            bb[cb][kk] =
                Tr::load_frag(rb, (tj < T && n0 < N) ? (uint32_t)(((tj * G + g) * N + n0) * ES) : kOOB);
        }
    }
    f32x4 acc[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) acc[cb] = Tr::mma(ca[kk], bb[cb][kk], acc[cb]);
    const size_t tile = ((((size_t)b * G + g) * nC + c) * NP + pr) * 4096;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * w + 4 * kg + i, col = 16 * cb + r;
            const uint32_t off = (uint32_t)((tile + row * 64 + col) * ES);
            // copy the element out first: a bit_cast taken directly on a
            // vector-element lvalue reads element 0 with this compiler
            const float v = acc[cb][i];
            if constexpr (ES == 2) {
                buf_st16(__builtin_bit_cast(uint16_t, Tr::from_f32(v)), rg, off);
            } else {
                buf_st32(__builtin_bit_cast(uint32_t, v), rg, off);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// k_chunk_walk
//
// One work-group per (batch, head) walks the chunks in order, 64-token tile by
// tile, with the P x N fp32 state in matrix-core accumulators. Its 8
// wavefronts take two roles that run side by side on every SIMD:
//   output waves (0-3), 16 output rows each: load this tile's C rows and C B^T
//     rows; form exp2(cs_i) C_i h_in^T (h_in fragments held in registers for
//     the chunk) + the chunk's earlier tiles through C B^T and the scaled X
//     copy (factorised decay) + the masked diagonal block + D x; store Y.
//   state waves (4-7), a quarter of the state's columns each: issue the next
//     tile's X, B and log-decay loads; update h <- decay h + Xs^T B with this
//     tile (Xs: X scaled by exp2(cs_e - cs'_j), e = the tile's last token);
//     at a chunk's end write h as the next chunk's h_in copy; stage the next
//     tile into the other LDS slots.
// One barrier per tile (two where a buffer cannot be doubled).
// LDS: a ring of NT+1 scaled-X tile slots (a chunk's earlier tiles stay
// readable while the next is staged), two unscaled-X slots, B^T and h_in
// copies (doubled when they fit), per-wave output rows, and two chunk-sized
// log-decay buffers.
// ---------------------------------------------------------------------------
template <typename TI, int Q, int P, int N>
struct WalkCfg {
    static constexpr int ES = Traits<TI>::kBytes;
    static constexpr int NT = Q / 64;
    static constexpr int NP = NT * (NT + 1) / 2;
    static constexpr int PB = P / 16;
    static constexpr int NB = N / 16;
    static constexpr int NTH = 512;                  // 4 output + 4 state wavefronts
    static constexpr int NBW = (NB + 3) / 4;         // state n-blocks per state wave
    static constexpr int NK = (N + 31) / 32;         // 32-wide k-steps over N
    static constexpr int PAD = 16 / ES;
    static constexpr int XS = NT + 1;                // scaled-X tile slots (ring)
    static constexpr int XH_LD = XS * 64 + PAD;
    static constexpr int XT_LD = 2 * 64 + PAD;       // unscaled X: two tile slots
    static constexpr int BT_LD = 64 + PAD;
    static constexpr int HS_LD = NK * 32 + PAD;
    static constexpr int YS_LD = P + PAD;
    static constexpr int UX = 16 * (P / 8);          // staging units: 4 tokens x 8 columns
    static constexpr int UB = 16 * (N / 8);
    static constexpr int RX = (UX + 255) / 256;      // units per state-wave thread
    static constexpr int RB = (UB + 255) / 256;
    static constexpr bool kHSReg = PB * NK * ES <= 32;  // h_in fragments kept in registers
    static constexpr int XH_OFF = 0;
    static constexpr int XH_BYTES = P * XH_LD * ES;
    static constexpr int XT_OFF = XH_OFF + XH_BYTES;
    static constexpr int XT_BYTES = P * XT_LD * ES;
    static constexpr int YS_OFF = XT_OFF + XT_BYTES;
    static constexpr int YS_BYTES = 64 * YS_LD * ES;
    static constexpr int CS_OFF = YS_OFF + YS_BYTES;  // 2 x (cs2[Q], cs'[Q]) fp32
    static constexpr int CS_BYTES = 2 * 2 * Q * 4;
    static constexpr int HS_OFF = CS_OFF + CS_BYTES;
    static constexpr int HS_BYTES = P * HS_LD * ES;
    static constexpr int BT_BYTES = N * BT_LD * ES;
    static constexpr int BASE = HS_OFF + HS_BYTES + BT_BYTES;
    static constexpr bool kBT2 = BASE + BT_BYTES <= 160 * 1024;             // double B^T
    static constexpr bool kHS2 = BASE + (kBT2 ? BT_BYTES : 0) + HS_BYTES <= 160 * 1024;
    static constexpr int BT_OFF = HS_OFF + (kHS2 ? 2 : 1) * HS_BYTES;
    static constexpr int LDS = BT_OFF + (kBT2 ? 2 : 1) * BT_BYTES;
    static constexpr bool kFits = LDS <= 160 * 1024;
};

template <int... Is, typename F>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, Is...>) {
    (f(std::integral_constant<int, Is>{}), ...);
}
template <int Count, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, Count>{});
}

template <typename TI>
__device__ __forceinline__ void lds_store4(TI *p, TI v0, TI v1, TI v2, TI v3) {
    if constexpr (sizeof(TI) == 2) {
        bf16x4 v = {v0, v1, v2, v3};
        *reinterpret_cast<bf16x4 *>(p) = v;
    } else {
        f32x4 v = {v0, v1, v2, v3};
        *reinterpret_cast<f32x4 *>(p) = v;
    }
}

template <typename TI>
__device__ __forceinline__ void lds_load4(TI *d, const TI *p) {
    if constexpr (sizeof(TI) == 2) {
        *reinterpret_cast<uint64_t *>(d) = *reinterpret_cast<const uint64_t *>(p);
    } else {
        const f32x4 v = *reinterpret_cast<const f32x4 *>(p);
        d[0] = v[0]; d[1] = v[1]; d[2] = v[2]; d[3] = v[3];
    }
}

// A compiler-level ordering point for LDS traffic within one wavefront: LDS
// operations of a wavefront execute in order, so a read issued after a write
// sees it once the compiler keeps them in that order.
__device__ __forceinline__ void wave_lds_order() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

template <typename TI, int Q, int P, int N>
__global__ __launch_bounds__((WalkCfg<TI, Q, P, N>::NTH), 1) void k_chunk_walk(WalkArgs a) {
    using Tr = Traits<TI>;
    using Cfg = WalkCfg<TI, Q, P, N>;
    using frag = typename Tr::frag;
    constexpr int ES = Cfg::ES, NT = Cfg::NT, NP = Cfg::NP, PB = Cfg::PB, NB = Cfg::NB;
    constexpr int NBW = Cfg::NBW, NK = Cfg::NK, XS = Cfg::XS;
    constexpr int RX = Cfg::RX, RB = Cfg::RB, UX = Cfg::UX, UB = Cfg::UB;
    constexpr int XH_LD = Cfg::XH_LD, XT_LD = Cfg::XT_LD, BT_LD = Cfg::BT_LD, HS_LD = Cfg::HS_LD;
    constexpr int YS_LD = Cfg::YS_LD;
    constexpr bool kHSReg = Cfg::kHSReg, kBT2 = Cfg::kBT2, kHS2 = Cfg::kHS2;
    __shared__ __attribute__((aligned(16))) char smem[Cfg::LDS];
    TI *XH = reinterpret_cast<TI *>(smem + Cfg::XH_OFF);
    TI *XT = reinterpret_cast<TI *>(smem + Cfg::XT_OFF);
    TI *YS = reinterpret_cast<TI *>(smem + Cfg::YS_OFF);
    float *CSB = reinterpret_cast<float *>(smem + Cfg::CS_OFF);  // [buf][cs2 Q | cs' Q]
    TI *HSB = reinterpret_cast<TI *>(smem + Cfg::HS_OFF);
    TI *BTB = reinterpret_cast<TI *>(smem + Cfg::BT_OFF);

    const int H = a.H, G = a.G, T = a.T, nC = a.nC;
    // blockIdx -> (b, h): consecutive logical indices share an XCD (dispatch
    // goes round-robin over the 8 XCDs), so the heads of one batch element,
    // which read the same B, C and C B^T, share one L2.
    const int W = a.batch * H;
    int L = blockIdx.x;
    if ((W & 7) == 0) L = (blockIdx.x & 7) * (W >> 3) + (blockIdx.x >> 3);
    const int b = L / H, h = L - b * H;
    const int g = (h * G) / H;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, scalar
    const bool out_wave = wv < 4;
    const int w = wv & 3;              // index within the role
    const int st = tid & 255;          // thread index within the role
    const int r = lane & 15, kg = lane >> 4;

    const size_t xslab = (size_t)T * H * P * ES;
    const size_t bslab = (size_t)T * G * N * ES;
    const rsrc_t rx = make_rsrc(reinterpret_cast<const char *>(a.X) + b * xslab, (uint32_t)xslab);
    const rsrc_t ry = make_rsrc(reinterpret_cast<char *>(a.Y) + b * xslab, (uint32_t)xslab);
    const rsrc_t rbm = make_rsrc(reinterpret_cast<const char *>(a.B) + b * bslab, (uint32_t)bslab);
    const rsrc_t rc = make_rsrc(reinterpret_cast<const char *>(a.C) + b * bslab, (uint32_t)bslab);
    const rsrc_t rg = make_rsrc(a.Gbuf, a.g_bytes);
    const float *cs_row = a.cs2 + ((size_t)b * H + h) * a.Tpad;
    const float *cp_row = a.dtf + ((size_t)b * H + h) * a.Tpad;  // cs' = cs2 - log2(dt)
    const float Dh = a.D[h];
    const uint32_t x_tok = (uint32_t)(H * P * ES), b_tok = (uint32_t)(G * N * ES);

    // ---- state-wave data: staging offsets and registers ----
    // staging units are wave-uniform whenever their count is a multiple of 64
    auto x_unit = [&](int k) { return (UX % 64 == 0) ? (64 * w + 256 * k < UX) : (st + 256 * k < UX); };
    auto b_unit = [&](int k) { return (UB % 64 == 0) ? (64 * w + 256 * k < UB) : (st + 256 * k < UB); };
    // Every state-wave lane issues every load, a lane without a unit at an
    // out-of-range offset (it reads zeros and moves no data), and tiles past
    // the end reload the last one: with no load under a branch, the
    // compiler's wait counts stay exact and loads two tiles ahead stay in
    // flight.
    uint32_t vx[RX], vb[RB];
#pragma unroll
    for (int k = 0; k < RX; ++k) {
        const int u = st + 256 * k;
        vx[k] = oob_if(!x_unit(k), (uint32_t)(4 * (u % 16)) * x_tok + (uint32_t)(8 * ((u / 16) % (P / 8)) * ES));
    }
#pragma unroll
    for (int k = 0; k < RB; ++k) {
        const int u = st + 256 * k;
        vb[k] = oob_if(!b_unit(k), (uint32_t)(4 * (u % 16)) * b_tok + (uint32_t)(8 * ((u / 16) % (N / 8)) * ES));
    }
    // Loads run kDepth tiles ahead of the staging; with two register sets the
    // set of tile t is t % 2, which is static when a chunk has an even number
    // of tiles.
    constexpr int kDepth = (NT % 2 == 0) ? 2 : 1;
    frag xr[kDepth][RX][4], br[kDepth][RB][4];
    f32x4 xcp[kDepth][RX];   // cs' of the unit's 4 tokens
    float xce[kDepth] = {};  // cs2 of the staged tile's last token
    auto issue_stage = [&](int tt, auto Sc) {  // X, B and log-decays of the tile at token tt
        constexpr int S = decltype(Sc)::value;
        const uint32_t sx = (uint32_t)(tt * H + h) * (uint32_t)(P * ES);
        const uint32_t sb = (uint32_t)(tt * G + g) * (uint32_t)(N * ES);
#pragma unroll
        for (int k = 0; k < RX; ++k) {
#pragma unroll
            for (int i = 0; i < 4; ++i) xr[S][k][i] = Tr::load_frag_s(rx, vx[k] + i * x_tok, sx);
            xcp[S][k] = *reinterpret_cast<const f32x4 *>(cp_row + tt + 4 * ((st + 256 * k) % 16));
        }
        xce[S] = cs_row[tt + 63];
#pragma unroll
        for (int k = 0; k < RB; ++k) {
#pragma unroll
            for (int i = 0; i < 4; ++i) br[S][k][i] = Tr::load_frag_s(rbm, vb[k] + i * b_tok, sb);
        }
    };
    auto stage = [&](auto Sc, int xslot, int tslot) {
        constexpr int S = decltype(Sc)::value;
        TI *BT = BTB + (kBT2 ? tslot : 0) * N * BT_LD;
#pragma unroll
        for (int k = 0; k < RX; ++k)
            if (x_unit(k)) {
                const int u = st + 256 * k;
                const int tq = u % 16, po = (u / 16) % (P / 8);
                float sc[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) sc[i] = fast_exp2(xce[S] - xcp[S][k][i]);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int row = 8 * po + e;
                    lds_store4<TI>(XT + row * XT_LD + tslot * 64 + 4 * tq, xr[S][k][0][e], xr[S][k][1][e],
                                   xr[S][k][2][e], xr[S][k][3][e]);
                    lds_store4<TI>(XH + row * XH_LD + xslot * 64 + 4 * tq,
                                   Tr::from_f32(Tr::frag_get(xr[S][k][0], e) * sc[0]),
                                   Tr::from_f32(Tr::frag_get(xr[S][k][1], e) * sc[1]),
                                   Tr::from_f32(Tr::frag_get(xr[S][k][2], e) * sc[2]),
                                   Tr::from_f32(Tr::frag_get(xr[S][k][3], e) * sc[3]));
                }
            }
#pragma unroll
        for (int k = 0; k < RB; ++k)
            if (b_unit(k)) {
                const int u = st + 256 * k;
                const int tq = u % 16, no = (u / 16) % (N / 8);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    lds_store4<TI>(BT + (8 * no + e) * BT_LD + 4 * tq, br[S][k][0][e], br[S][k][1][e],
                                   br[S][k][2][e], br[S][k][3][e]);
            }
    };
    // state accumulators (state waves): tile (pb, nb = w + 4j), rows p = 16pb + 4kg + i, col n = 16nb + r
    f32x4 hacc[PB][NBW];
    auto write_hs = [&](TI *HSw) {
#pragma unroll
        for (int pb = 0; pb < PB; ++pb)
#pragma unroll
            for (int j = 0; j < NBW; ++j) {
                const int nb = w + 4 * j;
                if (nb < NB) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        HSw[(16 * pb + 4 * kg + i) * HS_LD + 16 * nb + r] = Tr::from_f32(hacc[pb][j][i]);
                }
            }
    };

    // ---- output-wave data ----
    uint32_t vc[NK], vg[2];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
        const int n0 = kk * 32 + 8 * kg;
        vc[kk] = oob_if(n0 >= N, (uint32_t)(16 * w + r) * b_tok + (uint32_t)(n0 * ES));
    }
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) vg[k2] = (uint32_t)(((16 * w + r) * 64 + 32 * k2 + 8 * kg) * ES);
    frag hsf[kHSReg ? PB : 1][kHSReg ? NK : 1];

    // ---- prologue ----
    if (!out_wave) {
#pragma unroll
        for (int pb = 0; pb < PB; ++pb)
#pragma unroll
            for (int j = 0; j < NBW; ++j) {
                const int nb = w + 4 * j;
                f32x4 v = {0.f, 0.f, 0.f, 0.f};
                if (a.init && nb < NB) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int p = 16 * pb + 4 * kg + i, n = 16 * nb + r;
                        v[i] = a.init[(((size_t)b * H + h) * P + p) * N + n];
                    }
                }
                hacc[pb][j] = v;
            }
        write_hs(HSB);
        issue_stage(0, std::integral_constant<int, 0>{});
        stage(std::integral_constant<int, 0>{}, 0, 0);
        if constexpr (kDepth == 2) {
            issue_stage(nC * NT > 1 ? 64 : 0, std::integral_constant<int, 1>{});
        }
    }
    for (int k = tid; k < Q; k += Cfg::NTH) {
        CSB[k] = cs_row[k];
        CSB[Q + k] = cp_row[k];
    }
    if constexpr (N % 32 != 0) {
        for (int k = tid; k < (kHS2 ? 2 : 1) * P * (NK * 32 - N); k += Cfg::NTH) {
            const int q = k / (P * (NK * 32 - N)), kr = k % (P * (NK * 32 - N));
            const int p = kr / (NK * 32 - N), n = N + kr % (NK * 32 - N);
            HSB[q * P * HS_LD + p * HS_LD + n] = Tr::from_f32(0.f);
        }
    }
    __syncthreads();

    // Each wavefront runs one role for the whole walk (the role is uniform
    // over the wavefront); both loops reach the same barriers, one per tile
    // (two where kMidSync), so the work-group stays in step.
    constexpr bool kMidSync = !kBT2 || (!kHS2 && (NT == 1 || !kHSReg));
    if (out_wave) {
        // C rows and C B^T blocks of the next tile are loaded while this one
        // is computed: C right after its last use, C B^T after the diagonal.
        frag cf[NK], gf[NT][2];
        auto load_c = [&](int tt) {  // C rows of the tile at token tt
            const uint32_t sb = (uint32_t)(tt * G + g) * (uint32_t)(N * ES);
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) cf[kk] = Tr::load_frag_s(rc, vc[kk], sb);
        };
        auto load_g = [&](int cc, auto Ic) {  // C B^T blocks (I, J <= I) of chunk cc
            constexpr int I = decltype(Ic)::value;
            const size_t base = (((size_t)b * G + g) * nC + cc) * NP;
#pragma unroll
            for (int J = 0; J <= I; ++J) {
                const uint32_t sg = (uint32_t)((base + pair_index(I, J)) * 4096 * ES);
#pragma unroll
                for (int k2 = 0; k2 < 2; ++k2) gf[J][k2] = Tr::load_frag_s(rg, vg[k2], sg);
            }
        };
        // same issue order as inside the loop (C rows first), so that the
        // compiler's wait counts at the loop head fit both ways in
        load_c(0);
        __builtin_amdgcn_sched_barrier(0);
        load_g(0, std::integral_constant<int, 0>{});
        for (int c = 0; c < nC; ++c) {
            const int t0 = c * Q;
            const float *CSL = CSB + (c & 1) * 2 * Q;  // cs2 of this chunk
            const float *CPL = CSL + Q;                // cs' of this chunk
            const TI *HSr = HSB + (kHS2 ? (c & 1) : 0) * P * HS_LD;
            static_for<NT>([&](auto Ic) {
                constexpr int I = decltype(Ic)::value;
                const int tile0 = I * 64;
                const int tau = c * NT + I;
                const TI *XTc = XT + (tau & 1) * 64;
                // ================= output rows tile0 + 16w .. +15 =================
                if constexpr (I == 0 && kHSReg) {
#pragma unroll
                    for (int pb = 0; pb < PB; ++pb)
#pragma unroll
                        for (int kk = 0; kk < NK; ++kk)
                            hsf[pb][kk] = Tr::lds_frag(HSr + (16 * pb + r) * HS_LD + kk * 32 + 8 * kg);
                }
                const int irow = tile0 + 16 * w + r;  // chunk-local token of this lane's A row
                float cs_rows[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) cs_rows[i] = CSL[tile0 + 16 * w + 4 * kg + i];
                f32x4 acc[PB];
#pragma unroll
                for (int pb = 0; pb < PB; ++pb) acc[pb] = f32x4{0.f, 0.f, 0.f, 0.f};
                // state -> output
#pragma unroll
                for (int kk = 0; kk < NK; ++kk) {
#pragma unroll
                    for (int pb = 0; pb < PB; ++pb) {
                        frag hb;
                        if constexpr (kHSReg) {
                            hb = hsf[pb][kk];
                        } else {
                            hb = Tr::lds_frag(HSr + (16 * pb + r) * HS_LD + kk * 32 + 8 * kg);
                        }
                        acc[pb] = Tr::mma(cf[kk], hb, acc[pb]);
                    }
                }
                if constexpr (I + 1 < NT) {
                    load_c(t0 + tile0 + 64);
                } else {
                    load_c(c + 1 < nC ? t0 + Q : t0);  // past the end: a harmless reload
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float f = fast_exp2(cs_rows[i]);
#pragma unroll
                    for (int pb = 0; pb < PB; ++pb) acc[pb][i] *= f;
                }
                // earlier tiles of this chunk
#pragma unroll
                for (int J = 0; J < I; ++J) {
                    const int js = (tau - I + J) % XS;
                    f32x4 tmp[PB];
#pragma unroll
                    for (int pb = 0; pb < PB; ++pb) tmp[pb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int k2 = 0; k2 < 2; ++k2) {
#pragma unroll
                        for (int pb = 0; pb < PB; ++pb) {
                            const frag xb =
                                Tr::lds_frag(XH + (16 * pb + r) * XH_LD + js * 64 + 32 * k2 + 8 * kg);
                            tmp[pb] = Tr::mma(gf[J][k2], xb, tmp[pb]);
                        }
                    }
                    const float cs_je = CSL[J * 64 + 63];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float f = fast_exp2(cs_rows[i] - cs_je);
#pragma unroll
                        for (int pb = 0; pb < PB; ++pb) acc[pb][i] += f * tmp[pb][i];
                    }
                }
                // diagonal tile: weight exp2(cs_i - cs'_j) per element, j > i selected to zero
                {
                    const float cs_i = CSL[irow];
#pragma unroll
                    for (int k2 = 0; k2 < 2; ++k2) {
                        if (32 * k2 > 16 * w + 15) continue;  // wave-uniform: above the diagonal
                        const int j0 = tile0 + 32 * k2 + 8 * kg;
                        const f32x4 cpa = *reinterpret_cast<const f32x4 *>(CPL + j0);
                        const f32x4 cpb = *reinterpret_cast<const f32x4 *>(CPL + j0 + 4);
                        frag ma;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float cpj = e < 4 ? cpa[e] : cpb[e - 4];
                            const float v = Tr::frag_get(gf[I][k2], e) * fast_exp2(cs_i - cpj);
                            Tr::frag_set(ma, e, (j0 + e <= irow) ? v : 0.f);
                        }
#pragma unroll
                        for (int pb = 0; pb < PB; ++pb) {
                            const frag xb = Tr::lds_frag(XTc + (16 * pb + r) * XT_LD + 32 * k2 + 8 * kg);
                            acc[pb] = Tr::mma(ma, xb, acc[pb]);
                        }
                    }
                }
                if constexpr (I + 1 < NT) {
                    load_g(c, std::integral_constant<int, I + 1>{});
                } else {
                    load_g(c + 1 < nC ? c + 1 : c, std::integral_constant<int, 0>{});
                }
                // skip term, staging through this wave's own rows, store
#pragma unroll
                for (int pb = 0; pb < PB; ++pb) {
                    TI xs4[4];
                    lds_load4<TI>(xs4, XTc + (16 * pb + r) * XT_LD + 16 * w + 4 * kg);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int rl = 16 * w + 4 * kg + i;  // tile-local token
                        YS[rl * YS_LD + 16 * pb + r] = Tr::from_f32(acc[pb][i] + Dh * Tr::to_f32(xs4[i]));
                    }
                }
                wave_lds_order();
                {
                    constexpr int VPR = P * ES / 16;  // 16-byte vectors per row
                    const uint32_t sy = (uint32_t)((t0 + tile0 + 16 * w) * H + h) * (uint32_t)(P * ES);
#pragma unroll
                    for (int v = lane; v < 16 * VPR; v += 64) {
                        const int rl = v / VPR, cv = v % VPR;
                        const u32x4 d =
                            *reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(YS) +
                                                             (16 * w + rl) * YS_LD * ES + cv * 16);
                        buf_st128s(d, ry, (uint32_t)rl * x_tok + (uint32_t)(cv * 16), sy);
                    }
                }
                // a single B^T slot, or a single h_in copy that the output waves
                // still read this tile, must be read before it is overwritten
                if constexpr (kMidSync) __syncthreads();
                __syncthreads();
            });
        }
    } else {
        float csn = 0.f, cpn = 0.f;
        for (int c = 0; c < nC; ++c) {
            const int t0 = c * Q;
            const float *CSL = CSB + (c & 1) * 2 * Q;  // cs2 of this chunk
            static_for<NT>([&](auto Ic) {
                constexpr int I = decltype(Ic)::value;
                const int tile0 = I * 64;
                const int tau = c * NT + I;
                const int xslot = tau % XS, tslot = tau & 1;
                // ================= state update and staging =================
                if constexpr (I == 0) {
                    // the next chunk's log-decays (Q <= 256: one per thread),
                    // issued first and written at the chunk's last tile
                    const int kn = (c + 1 < nC ? t0 + Q : t0) + min(st, Q - 1);
                    csn = cs_row[kn];
                    cpn = cp_row[kn];
                }
                issue_stage(min(tau + kDepth, nC * NT - 1) * 64,
                            std::integral_constant<int, kDepth == 2 ? (I & 1) : 0>{});
                const TI *BT = BTB + (kBT2 ? tslot : 0) * N * BT_LD;
                const float cs_e = CSL[tile0 + 63];
                const float prev = (I > 0) ? CSL[tile0 - 1] : 0.f;
                const float dec = fast_exp2(cs_e - prev);
#pragma unroll
                for (int pb = 0; pb < PB; ++pb)
#pragma unroll
                    for (int j = 0; j < NBW; ++j) hacc[pb][j] *= dec;
#pragma unroll
                for (int k2 = 0; k2 < 2; ++k2) {
                    frag xa[PB];
#pragma unroll
                    for (int pb = 0; pb < PB; ++pb)
                        xa[pb] = Tr::lds_frag(XH + (16 * pb + r) * XH_LD + xslot * 64 + 32 * k2 + 8 * kg);
#pragma unroll
                    for (int j = 0; j < NBW; ++j) {
                        const int nb = w + 4 * j;
                        if (nb < NB) {
                            const frag bb = Tr::lds_frag(BT + (16 * nb + r) * BT_LD + 32 * k2 + 8 * kg);
#pragma unroll
                            for (int pb = 0; pb < PB; ++pb) hacc[pb][j] = Tr::mma(xa[pb], bb, hacc[pb][j]);
                        }
                    }
                }
                // a single B^T slot, or a single h_in copy that the output waves
                // still read this tile, must be read before it is overwritten
                if constexpr (kMidSync) __syncthreads();
                if constexpr (I == NT - 1) {
                    if (c + 1 < nC && st < Q) {
                        float *CSN = CSB + ((c + 1) & 1) * 2 * Q;
                        CSN[st] = csn;
                        CSN[Q + st] = cpn;
                    }
                }
                if constexpr (I == NT - 1) write_hs(HSB + (kHS2 ? ((c + 1) & 1) : 0) * P * HS_LD);
                // (after the last tile this stages a reload into slots nobody reads)
                stage(std::integral_constant<int, kDepth == 2 ? ((I + 1) & 1) : 0>{}, (tau + 1) % XS, (tau + 1) & 1);
                __syncthreads();
            });
        }
        if (a.final_state) {
#pragma unroll
            for (int pb = 0; pb < PB; ++pb)
#pragma unroll
                for (int j = 0; j < NBW; ++j) {
                    const int nb = w + 4 * j;
                    if (nb < NB) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int p = 16 * pb + 4 * kg + i, n = 16 * nb + r;
                            a.final_state[(((size_t)b * H + h) * P + p) * N + n] = hacc[pb][j][i];
                        }
                    }
                }
        }
    }
}

// ---------------------------------------------------------------------------
// host-side launches for one instantiation
// ---------------------------------------------------------------------------
template <typename TI, int Q, int N>
static ssd_status run_prepare(const FwdArgs &f, hipStream_t s) {
    const int nC = (int)f.nC;
    const int hblocks = (int)((f.H + kCumsumHeads - 1) / kCumsumHeads);
    if (launch(k_dt_cumsum<TI, Q>, dim3((unsigned)(f.batch * hblocks * nC)), dim3(256), s,
               (const TI *)f.dt, f.A, f.cs2, f.dtf, (int)f.T, (int)f.H, nC, (int)f.Tpad) != hipSuccess)
        return SSD_ERR_HIP;
    constexpr int NT = Q / 64, NP = NT * (NT + 1) / 2;
    if (launch(k_chunk_cb<TI, Q, N>, dim3((unsigned)(f.batch * nC * f.G * NP)), dim3(256), s,
               (const TI *)f.B, (const TI *)f.C, (TI *)f.Gbuf, (int)f.T, (int)f.G, nC,
               (uint32_t)f.g_bytes) != hipSuccess)
        return SSD_ERR_HIP;
    return SSD_OK;
}

template <typename TI, int Q, int P, int N>
static ssd_status run_walk(const FwdArgs &f, hipStream_t s) {
    using Cfg = WalkCfg<TI, Q, P, N>;
    if constexpr (!Cfg::kFits) {
        return SSD_ERR_UNSUPPORTED;
    } else {
        WalkArgs wa;
        wa.X = f.X; wa.B = f.B; wa.C = f.C; wa.Y = f.Y; wa.Gbuf = f.Gbuf;
        wa.cs2 = f.cs2; wa.dtf = f.dtf; wa.D = f.D; wa.init = f.init; wa.final_state = f.final_state;
        wa.batch = (int)f.batch; wa.T = (int)f.T; wa.H = (int)f.H; wa.G = (int)f.G; wa.nC = (int)f.nC;
        wa.Tpad = (int)f.Tpad; wa.g_bytes = (uint32_t)f.g_bytes;
        return launch(k_chunk_walk<TI, Q, P, N>, dim3((unsigned)(f.batch * f.H)), dim3(Cfg::NTH), s, wa) ==
                       hipSuccess
                   ? SSD_OK
                   : SSD_ERR_HIP;
    }
}

template <typename TI, int Q, int P>
static ssd_status walk_n(const FwdArgs &f, hipStream_t s) {
    switch (f.N) {
        case 16: return run_walk<TI, Q, P, 16>(f, s);
        case 32: return run_walk<TI, Q, P, 32>(f, s);
        case 64: return run_walk<TI, Q, P, 64>(f, s);
        case 128: return run_walk<TI, Q, P, 128>(f, s);
        case 256: return run_walk<TI, Q, P, 256>(f, s);
        default: return SSD_ERR_UNSUPPORTED;
    }
}

template <typename TI, int Q>
static ssd_status walk_p(const FwdArgs &f, hipStream_t s) {
    switch (f.P) {
        case 16: return walk_n<TI, Q, 16>(f, s);
        case 32: return walk_n<TI, Q, 32>(f, s);
        case 64: return walk_n<TI, Q, 64>(f, s);
        case 128: return walk_n<TI, Q, 128>(f, s);
        default: return SSD_ERR_UNSUPPORTED;
    }
}

template <typename TI, int Q>
static ssd_status prepare_n(const FwdArgs &f, hipStream_t s) {
    switch (f.N) {
        case 16: return run_prepare<TI, Q, 16>(f, s);
        case 32: return run_prepare<TI, Q, 32>(f, s);
        case 64: return run_prepare<TI, Q, 64>(f, s);
        case 128: return run_prepare<TI, Q, 128>(f, s);
        case 256: return run_prepare<TI, Q, 256>(f, s);
        default: return SSD_ERR_UNSUPPORTED;
    }
}

template <typename TI, bool kWalk>
static ssd_status dispatch_q(const FwdArgs &f, hipStream_t s) {
    switch (f.Q) {
        case 64: return kWalk ? walk_p<TI, 64>(f, s) : prepare_n<TI, 64>(f, s);
        case 128: return kWalk ? walk_p<TI, 128>(f, s) : prepare_n<TI, 128>(f, s);
        case 256: return kWalk ? walk_p<TI, 256>(f, s) : prepare_n<TI, 256>(f, s);
        default: return SSD_ERR_UNSUPPORTED;
    }
}

ssd_status launch_prepare(const FwdArgs &f, hipStream_t s) {
    return f.dtype == SSD_BF16 ? dispatch_q<bf16, false>(f, s) : dispatch_q<float, false>(f, s);
}

ssd_status launch_walk(const FwdArgs &f, hipStream_t s) {
    return f.dtype == SSD_BF16 ? dispatch_q<bf16, true>(f, s) : dispatch_q<float, true>(f, s);
}

template <typename TI, int Q, int P, int N>
static constexpr int lds_of() { return WalkCfg<TI, Q, P, N>::LDS; }

template <typename TI>
static int lds_table(int64_t Q, int64_t P, int64_t N) {
#define SSD_LDS_N(Qv, Pv)                                   \
    switch (N) {                                            \
        case 16: return lds_of<TI, Qv, Pv, 16>();           \
        case 32: return lds_of<TI, Qv, Pv, 32>();           \
        case 64: return lds_of<TI, Qv, Pv, 64>();           \
        case 128: return lds_of<TI, Qv, Pv, 128>();         \
        case 256: return lds_of<TI, Qv, Pv, 256>();         \
        default: return -1;                                 \
    }
#define SSD_LDS_P(Qv)                                       \
    switch (P) {                                            \
        case 16: SSD_LDS_N(Qv, 16)                          \
        case 32: SSD_LDS_N(Qv, 32)                          \
        case 64: SSD_LDS_N(Qv, 64)                          \
        case 128: SSD_LDS_N(Qv, 128)                        \
        default: return -1;                                 \
    }
    switch (Q) {
        case 64: SSD_LDS_P(64)
        case 128: SSD_LDS_P(128)
        case 256: SSD_LDS_P(256)
        default: return -1;
    }
#undef SSD_LDS_P
#undef SSD_LDS_N
}

int fwd_lds_bytes(ssd_dtype dt, int64_t Q, int64_t P, int64_t N) {
    return dt == SSD_BF16 ? lds_table<bf16>(Q, P, N) : lds_table<float>(Q, P, N);
}

}  // namespace ssd
