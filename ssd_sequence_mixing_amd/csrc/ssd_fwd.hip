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
//                 prefix sum of dt*A in base 2 (cs2), plus dt re-laid out as
//                 (batch, head, token) fp32, both read contiguously later.
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
            od[k] = d[k];
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
// ---------------------------------------------------------------------------
template <typename TI, int Q, int P, int N>
struct WalkCfg {
    static constexpr int ES = Traits<TI>::kBytes;
    static constexpr int NT = Q / 64;
    static constexpr int NP = NT * (NT + 1) / 2;
    static constexpr int PB = P / 16;
    static constexpr int NB = N / 16;
    static constexpr int NW = 4;                  // wavefronts per work-group
    static constexpr int NTH = 64 * NW;
    static constexpr int NBW = (NB + NW - 1) / NW;  // state n-blocks per wave
    static constexpr int WPR = NW / 4;              // waves sharing one 16-row output block
    static constexpr int PBW = (PB + WPR - 1) / WPR;  // output p-blocks per wave
    static constexpr int NK = (N + 31) / 32;
    static constexpr int PAD = 16 / ES;
    static constexpr int XT_LD = Q + PAD;        // X^T rows (p), token-contiguous, whole chunk
    static constexpr int BT_LD = 64 + PAD;       // B^T rows (n), token-contiguous, one tile
    static constexpr int HS_LD = NK * 32 + PAD;  // state rows (p), n-contiguous
    static constexpr int YS_LD = P + PAD;        // output staging rows (token)
    // staging units per 64-token tile: 4 consecutive tokens x 8 consecutive columns
    static constexpr int UX = 16 * (P / 8);
    static constexpr int UB = 16 * (N / 8);
    static constexpr int RX = (UX + NTH - 1) / NTH;
    static constexpr int RB = (UB + NTH - 1) / NTH;
    static constexpr int XT_OFF = 0;
    static constexpr int XT_BYTES = P * XT_LD * ES;
    static constexpr int XH_OFF = XT_OFF + XT_BYTES;
    static constexpr int BT_OFF = XH_OFF + XT_BYTES;
    static constexpr int BT_BYTES = N * BT_LD * ES;
    static constexpr int HS_OFF = BT_OFF + BT_BYTES;
    static constexpr int HS_BYTES = P * HS_LD * ES;
    static constexpr int YS_OFF = HS_OFF + HS_BYTES;
    static constexpr int YS_BYTES = 64 * YS_LD * ES;
    static constexpr int CS_OFF = YS_OFF + YS_BYTES;  // 2 buffers x (cs2[Q], dt[Q]) fp32
    static constexpr int LDS = CS_OFF + 2 * 2 * Q * 4;
    static constexpr bool kFits = LDS <= 160 * 1024;
};

// Global data one 64-token tile needs, held in registers so that the next
// tile's loads are in flight while the current tile computes.
template <typename TI, int Q, int P, int N>
struct WalkRegs {
    using Cfg = WalkCfg<TI, Q, P, N>;
    using frag = typename Traits<TI>::frag;
    frag xr[Cfg::RX][4];   // X: 4 tokens x 8 columns per staging unit
    frag br[Cfg::RB][4];   // B: 4 tokens x 8 columns per staging unit
    frag cf[Cfg::NK];      // C rows of this lane's A row (state -> output)
    frag gf[Cfg::NT][2];   // C B^T rows of tiles J <= I (two 32-wide k-steps each)
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

template <typename TI, int Q, int P, int N>
__global__ __launch_bounds__((WalkCfg<TI, Q, P, N>::NTH), 1) void k_chunk_walk(WalkArgs a) {
    using Tr = Traits<TI>;
    using Cfg = WalkCfg<TI, Q, P, N>;
    using Regs = WalkRegs<TI, Q, P, N>;
    using frag = typename Tr::frag;
    constexpr int ES = Cfg::ES, NT = Cfg::NT, NP = Cfg::NP, PB = Cfg::PB, NB = Cfg::NB;
    constexpr int NW = Cfg::NW, NTH = Cfg::NTH, NBW = Cfg::NBW, PBW = Cfg::PBW, NK = Cfg::NK;
    constexpr int WPR = Cfg::WPR;
    constexpr int XT_LD = Cfg::XT_LD, BT_LD = Cfg::BT_LD, HS_LD = Cfg::HS_LD, YS_LD = Cfg::YS_LD;
    __shared__ __attribute__((aligned(16))) char smem[Cfg::LDS];
    TI *XT = reinterpret_cast<TI *>(smem + Cfg::XT_OFF);
    TI *XH = reinterpret_cast<TI *>(smem + Cfg::XH_OFF);
    TI *BT = reinterpret_cast<TI *>(smem + Cfg::BT_OFF);
    TI *HS = reinterpret_cast<TI *>(smem + Cfg::HS_OFF);
    TI *YS = reinterpret_cast<TI *>(smem + Cfg::YS_OFF);
    float *CSB = reinterpret_cast<float *>(smem + Cfg::CS_OFF);  // [buf][cs2 Q | dt Q]

    const int H = a.H, G = a.G, T = a.T, nC = a.nC;
    // blockIdx -> (b, h): consecutive logical indices share an XCD (dispatch
    // goes round-robin over the 8 XCDs), so the heads of one batch element,
    // which read the same B, C and G, share one L2.
    const int W = a.batch * H;
    int L = blockIdx.x;
    if ((W & 7) == 0) L = (blockIdx.x & 7) * (W >> 3) + (blockIdx.x >> 3);
    const int b = L / H, h = L - b * H;
    const int g = (h * G) / H;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, scalar
    const int r = lane & 15, kg = lane >> 4;
    const int rb = w & 3;   // output row block (16 tokens) of this wave
    const int ph = w >> 2;  // output p-blocks ph, ph + WPR, ... of this wave
    // X staging units go to threads 0.., B staging units to threads ..NTH-1
    const int xu0 = tid, bu0 = NTH - 1 - tid;

    const size_t xslab = (size_t)T * H * P * ES;
    const size_t bslab = (size_t)T * G * N * ES;
    const rsrc_t rx = make_rsrc(reinterpret_cast<const char *>(a.X) + b * xslab, (uint32_t)xslab);
    const rsrc_t ry = make_rsrc(reinterpret_cast<char *>(a.Y) + b * xslab, (uint32_t)xslab);
    const rsrc_t rbm = make_rsrc(reinterpret_cast<const char *>(a.B) + b * bslab, (uint32_t)bslab);
    const rsrc_t rc = make_rsrc(reinterpret_cast<const char *>(a.C) + b * bslab, (uint32_t)bslab);
    const rsrc_t rg = make_rsrc(a.Gbuf, a.g_bytes);
    const float *cs_row = a.cs2 + ((size_t)b * H + h) * a.Tpad;
    const float *dt_row = a.dtf + ((size_t)b * H + h) * a.Tpad;
    const float Dh = a.D[h];

    // issue every global load tile (c, I) needs, into registers
    auto load_tile = [&](Regs &R, int c, auto Ic) {
        constexpr int I = decltype(Ic)::value;
        const int t0 = c * Q, tile0 = I * 64;
#pragma unroll
        for (int k = 0; k < Cfg::RX; ++k) {
            const int u = xu0 + NTH * k;
            const int tq = u % 16, po = (u / 16) % (P / 8);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = t0 + tile0 + 4 * tq + i;
                R.xr[k][i] = Tr::load_frag(
                    rx, oob_if(u >= Cfg::UX || t >= T, (uint32_t)(((t * H + h) * P + 8 * po) * ES)));
            }
        }
#pragma unroll
        for (int k = 0; k < Cfg::RB; ++k) {
            const int u = bu0 + NTH * k;
            const int tq = u % 16, no = (u / 16) % (N / 8);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = t0 + tile0 + 4 * tq + i;
                R.br[k][i] = Tr::load_frag(
                    rbm, oob_if(u >= Cfg::UB || t >= T, (uint32_t)(((t * G + g) * N + 8 * no) * ES)));
            }
        }
        const int ti = t0 + tile0 + 16 * rb + r;
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
            const int n0 = kk * 32 + 8 * kg;
            R.cf[kk] = Tr::load_frag(
                rc, oob_if(ti >= T || n0 >= N, (uint32_t)(((ti * G + g) * N + n0) * ES)));
        }
#pragma unroll
        for (int J = 0; J <= I; ++J) {
            const size_t gt = ((((size_t)b * G + g) * nC + c) * NP + pair_index(I, J)) * 4096;
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2)
                R.gf[J][k2] =
                    Tr::load_frag(rg, (uint32_t)((gt + (16 * rb + r) * 64 + 32 * k2 + 8 * kg) * ES));
        }
    };

    // state accumulators: tile (pb, nb = w + NW*j), rows p = 16pb + 4kg + i, col n = 16nb + r
    f32x4 hacc[PB][NBW];
#pragma unroll
    for (int pb = 0; pb < PB; ++pb)
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
            const int nb = w + NW * j;
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

    Regs R[2];
    for (int k = tid; k < Q; k += NTH) {
        CSB[k] = cs_row[k];
        CSB[Q + k] = dt_row[k];
    }
    load_tile(R[0], 0, std::integral_constant<int, 0>{});

    for (int c = 0; c < nC; ++c) {
        const int t0 = c * Q;
        const float *CSL = CSB + (c & 1) * 2 * Q;
        const float *DTL = CSL + Q;
        float *CSN = CSB + ((c + 1) & 1) * 2 * Q;  // next chunk's slot
        float csn = 0.f, dtn = 0.f;
        static_for<NT>([&](auto Ic) {
            constexpr int I = decltype(Ic)::value;
            constexpr int cur = (NT == 1) ? 0 : (I & 1);
            constexpr int nxt = cur ^ 1;
            Regs &RC = R[cur];
            const int tile0 = I * 64;
            if constexpr (I == 0) {
                // state entering this chunk -> matrix-core operand copy
#pragma unroll
                for (int pb = 0; pb < PB; ++pb)
#pragma unroll
                    for (int j = 0; j < NBW; ++j) {
                        const int nb = w + NW * j;
                        if (nb < NB) {
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                HS[(16 * pb + 4 * kg + i) * HS_LD + 16 * nb + r] =
                                    Tr::from_f32(hacc[pb][j][i]);
                        }
                    }
                if constexpr (N % 32 != 0) {
                    for (int k = tid; k < P * (NK * 32 - N); k += NTH) {
                        const int p = k / (NK * 32 - N), n = N + k % (NK * 32 - N);
                        HS[p * HS_LD + n] = Tr::from_f32(0.f);
                    }
                }
            }
            const float cs_e = CSL[tile0 + 63];  // tile's last token
            // ---- stage the prefetched X tile (unscaled and column-scaled) and B tile
#pragma unroll
            for (int k = 0; k < Cfg::RX; ++k) {
                const int u = xu0 + NTH * k;
                // wave-uniform whenever UX is a multiple of 64
                if ((Cfg::UX % 64 == 0) ? (64 * w + NTH * k < Cfg::UX) : (u < Cfg::UX)) {
                    const int tq = u % 16, po = u / 16;
                    const int jc = tile0 + 4 * tq;
                    float sc[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) sc[i] = DTL[jc + i] * fast_exp2(cs_e - CSL[jc + i]);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int row = 8 * po + e;
                        lds_store4<TI>(XT + row * XT_LD + jc, RC.xr[k][0][e], RC.xr[k][1][e],
                                       RC.xr[k][2][e], RC.xr[k][3][e]);
                        lds_store4<TI>(XH + row * XT_LD + jc,
                                       Tr::from_f32(Tr::frag_get(RC.xr[k][0], e) * sc[0]),
                                       Tr::from_f32(Tr::frag_get(RC.xr[k][1], e) * sc[1]),
                                       Tr::from_f32(Tr::frag_get(RC.xr[k][2], e) * sc[2]),
                                       Tr::from_f32(Tr::frag_get(RC.xr[k][3], e) * sc[3]));
                    }
                }
            }
#pragma unroll
            for (int k = 0; k < Cfg::RB; ++k) {
                const int u = bu0 + NTH * k;
                if ((Cfg::UB % 64 == 0) ? (64 * (NW - 1 - w) + NTH * k < Cfg::UB) : (u < Cfg::UB)) {
                    const int tq = u % 16, no = u / 16;
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        lds_store4<TI>(BT + (8 * no + e) * BT_LD + 4 * tq, RC.br[k][0][e],
                                       RC.br[k][1][e], RC.br[k][2][e], RC.br[k][3][e]);
                }
            }
            __syncthreads();

            // ---- prefetch the next tile while this one computes
            // (past the last chunk the loads fall outside every range and return 0)
            if constexpr (I + 1 < NT) {
                load_tile(R[nxt], c, std::integral_constant<int, I + 1>{});
            } else {
                load_tile(R[nxt], c + 1, std::integral_constant<int, 0>{});
            }
            if constexpr (I == 0) {
                if (c + 1 < nC && tid < Q) {  // Q <= NTH: one value per thread
                    csn = cs_row[t0 + Q + tid];
                    dtn = dt_row[t0 + Q + tid];
                }
            }

            // ---- output rows tile0 + 16rb .. +15 (A-operand row r), p-blocks ph, ph + 2, ...
            const int irow = tile0 + 16 * rb + r;  // chunk-local token of this lane's A row
            f32x4 acc[PBW];
#pragma unroll
            for (int j = 0; j < PBW; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
            // state -> output: C_i . h_in
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) {
                const int n0 = kk * 32 + 8 * kg;
#pragma unroll
                for (int j = 0; j < PBW; ++j) {
                    const int pb = ph + WPR * j;
                    if (pb < PB) {
                        const frag hb = Tr::lds_frag(HS + (16 * pb + r) * HS_LD + n0);
                        acc[j] = Tr::mma(RC.cf[kk], hb, acc[j]);
                    }
                }
            }
            float cs_rows[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) cs_rows[i] = CSL[tile0 + 16 * rb + 4 * kg + i];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float f = fast_exp2(cs_rows[i]);
#pragma unroll
                for (int j = 0; j < PBW; ++j) acc[j][i] *= f;
            }
            // earlier tiles of this chunk: G_IJ (unmasked, J < I) times the scaled X copy
#pragma unroll
            for (int J = 0; J < I; ++J) {
                f32x4 tmp[PBW];
#pragma unroll
                for (int j = 0; j < PBW; ++j) tmp[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k2 = 0; k2 < 2; ++k2) {
#pragma unroll
                    for (int j = 0; j < PBW; ++j) {
                        const int pb = ph + WPR * j;
                        if (pb < PB) {
                            const frag xb =
                                Tr::lds_frag(XH + (16 * pb + r) * XT_LD + J * 64 + 32 * k2 + 8 * kg);
                            tmp[j] = Tr::mma(RC.gf[J][k2], xb, tmp[j]);
                        }
                    }
                }
                const float cs_je = CSL[J * 64 + 63];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float f = fast_exp2(cs_rows[i] - cs_je);
#pragma unroll
                    for (int j = 0; j < PBW; ++j) acc[j][i] += f * tmp[j][i];
                }
            }
            // diagonal tile: mask built per element, j > i selected to zero
            {
                const float cs_i = CSL[irow];
#pragma unroll
                for (int k2 = 0; k2 < 2; ++k2) {
                    if (32 * k2 > 16 * rb + 15) continue;  // wave-uniform: block above the diagonal
                    frag ma;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int jc = tile0 + 32 * k2 + 8 * kg + e;
                        const float v =
                            Tr::frag_get(RC.gf[I][k2], e) * fast_exp2(cs_i - CSL[jc]) * DTL[jc];
                        Tr::frag_set(ma, e, (jc <= irow) ? v : 0.f);
                    }
#pragma unroll
                    for (int j = 0; j < PBW; ++j) {
                        const int pb = ph + WPR * j;
                        if (pb < PB) {
                            const frag xb =
                                Tr::lds_frag(XT + (16 * pb + r) * XT_LD + tile0 + 32 * k2 + 8 * kg);
                            acc[j] = Tr::mma(ma, xb, acc[j]);
                        }
                    }
                }
            }
            // skip term and output staging
#pragma unroll
            for (int j = 0; j < PBW; ++j) {
                const int pb = ph + WPR * j;
                if (pb < PB) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int rl = 16 * rb + 4 * kg + i;  // tile-local token
                        const float xv = Tr::to_f32(XT[(16 * pb + r) * XT_LD + tile0 + rl]);
                        YS[rl * YS_LD + 16 * pb + r] = Tr::from_f32(acc[j][i] + Dh * xv);
                    }
                }
            }
            __syncthreads();
            {
                constexpr int VPR = P * ES / 16;  // 16-byte vectors per row
#pragma unroll
                for (int v = tid; v < 64 * VPR; v += NTH) {
                    const int rl = v / VPR, cv = v % VPR;
                    const int t = t0 + tile0 + rl;
                    const u32x4 d =
                        *reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(YS) +
                                                         rl * YS_LD * ES + cv * 16);
                    buf_st128(d, ry, oob_if(t >= T, (uint32_t)((t * H + h) * P * ES + cv * 16)));
                }
            }

            // ---- state update for this tile: h <- decay * h + (scaled X)^T B
            {
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
                        xa[pb] = Tr::lds_frag(XH + (16 * pb + r) * XT_LD + tile0 + 32 * k2 + 8 * kg);
#pragma unroll
                    for (int j = 0; j < NBW; ++j) {
                        const int nb = w + NW * j;
                        if (nb < NB) {
                            const frag bb = Tr::lds_frag(BT + (16 * nb + r) * BT_LD + 32 * k2 + 8 * kg);
#pragma unroll
                            for (int pb = 0; pb < PB; ++pb) hacc[pb][j] = Tr::mma(xa[pb], bb, hacc[pb][j]);
                        }
                    }
                }
            }
            if constexpr (I == NT - 1) {
                if (c + 1 < nC && tid < Q) {  // Q <= NTH
                    CSN[tid] = csn;
                    CSN[Q + tid] = dtn;
                }
            }
            if constexpr (NT == 1) R[0] = R[1];
            __syncthreads();
        });
    }

    if (a.final_state) {
#pragma unroll
        for (int pb = 0; pb < PB; ++pb)
#pragma unroll
            for (int j = 0; j < NBW; ++j) {
                const int nb = w + NW * j;
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
