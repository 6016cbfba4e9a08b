// The chunk walk with the state held where it is used (gfx950, bf16 storage).
//
// Same computation as k_chunk_walk in ssd_fwd.hip (the chunked method of the
// "Transformers are SSMs" reading report, section 3.1, with chunks cut into
// 64-token tiles and the state handed from tile to tile), arranged so that no
// wavefront reads the whole state through LDS and every global access moves
// whole 64-byte (or larger) pieces of rows.
//
// One work-group per (batch, head, column slice of PW columns), 8 wavefronts
// in two roles, each role split 2 x 2 by (a, b), b the half of the columns:
//   state waves 4-7 keep the state block h[p in half b][n in half a] in fp32
//     matrix-core accumulators, update it per tile from X^T and B^T in LDS,
//     and publish it in bf16 (4 KB per wave at P 64, N 128) as the operand of
//     the next tile's state -> output product. They also stage B^T for the
//     next tile (B loaded two tiles ahead).
//   output waves 0-3 form the transposed output Y^T[p in half b][i] for the
//     tokens i of half a: state -> output from the published state (both n
//     halves of its columns), the diagonal block from C B^T and the weighted
//     X, and the skip term; the output goes through LDS and leaves as whole
//     rows during the next tile, where the gate y SiLU(z) is applied with z
//     read in the same row pieces. They also stage, for the next tile, the C
//     rows (whole lines, into LDS), the X rows (after the layer's causal
//     convolution and SiLU when it is fused in) and X weighted by its decay
//     factors, written token-major (X^T) for the two products whose
//     contraction runs over tokens.
// Each SIMD runs one wavefront of each role; one barrier per tile.
//
// The n axis of the state is permuted inside every 32-wide block: LDS row rho
// of B^T (and accumulator row rho of the state) holds n = sigma(rho) with
//   rho = 32 m + 16 s + 4 q + u  ->  n = 32 m + 8 q + 4 s + u,
// so that the 8 values a lane holds for one k-step of the state -> output
// product (two 4-row accumulator pieces) are 8 consecutive n of C: the C
// fragments are plain 16-byte LDS reads, and the state is read and written
// in global memory as 16-byte pieces.
//
// The output is formed transposed (rows p, columns tokens). Lanes 16 apart
// swap accumulator halves (v_permlane16_swap) so that each lane then holds 8
// consecutive columns of one token: the skip term, the gate and the store
// work on 16-byte row pieces taken straight from the accumulators.
//
// Decay weights as in ssd_fwd.hip (log-decays in base 2, cs' = cs - log2 dt):
// a tile whose decay cs_r - cs_e is at most kFDMax is factored about its
// start, X~_j = 2^(cs_r - cs'_j) x_j,
//   Y_i = 2^(cs_i - cs_r) (C_i h_r + sum_j G_ij X~_j) + D x_i,  h_e = 2^(cs_e - cs_r) (h_r + X~^T B);
// other tiles keep X as it is and put the weights elsewhere: on B^T for the
// state, Bw_j = 2^(cs_e - cs'_j) B_j <= dt_j B_j, h_e = 2^(cs_e - cs_r) h_r + X^T Bw,
// and per element on C B^T for the diagonal block, G_ij 2^(cs_i - cs'_j).
#include <type_traits>
#include <utility>

#include "ssd_common.h"
#include "ssd_internal.h"

namespace ssd {

namespace {

constexpr float kRsFDMax = 64.f;  // as kFDMax in ssd_fwd.hip

template <int Q, int PW, int N>
struct RsCfg {
    static constexpr int TT = 64;                 // tile tokens
    static constexpr int NT = Q / TT;             // tiles per chunk
    static constexpr int NH = N / 2, PH = PW / 2; // a wave's share of n and p
    static constexpr int NBH = NH / 16, PBH = PH / 16;
    static constexpr int NM = NH / 32;            // 32-wide k-steps over an n half
    static constexpr int NK = N / 32;             // 32-wide k-steps over N
    static constexpr int KS = TT / 32;            // 32-token k-steps over a tile
    static constexpr int IB = TT / 2 / 16;        // 16-token blocks of a wave's output
    static constexpr int LD = TT + 8;             // row length of the token-major LDS tiles
    static constexpr int XT_BYTES = PW * LD * 2;  // one slot of X^T
    static constexpr int BT_BYTES = N * LD * 2;   // one slot of B^T
    static constexpr int XF = NM * PBH;           // fragments one state wave publishes per tile
    static constexpr int XCH_BYTES = 4 * XF * 64 * 16;
    static constexpr int CLD = N + 8;             // row length of the C tile
    static constexpr int C_BYTES = TT * CLD * 2;
    static constexpr int YLD = PW + 8;            // row length of the output staging tile
    static constexpr int YS_BYTES = TT * YLD * 2;
    static constexpr int XW_OFF = 0;                      // X^T (weighted in factored tiles), 2 slots
    static constexpr int YS_OFF = XW_OFF + 2 * XT_BYTES;  // output rows, 2 slots
    static constexpr int BT_OFF = YS_OFF + 2 * YS_BYTES;  // B^T (weighted in the other tiles), 2 slots
    static constexpr int XCH_OFF = BT_OFF + 2 * BT_BYTES; // state exchange, 2 slots
    static constexpr int C_OFF = XCH_OFF + 2 * XCH_BYTES; // C, 2 slots
    static constexpr int XRLD = PW + 8;           // row length of the token-major X tile (skip term)
    static constexpr int XR_BYTES = TT * XRLD * 2;
    static constexpr int XR_OFF = C_OFF + 2 * C_BYTES;    // X rows, 2 slots
    static constexpr int CS_OFF = XR_OFF + 2 * XR_BYTES;
    static constexpr int CS_BYTES = 2 * 2 * Q * 4;       // 2 chunks x (cs2, cs')
    static constexpr int LDS = CS_OFF + CS_BYTES;
    // staging units (256 lanes of one role each)
    static constexpr int XCW = PW / 4, BCW = N / 8;      // 8-byte pieces per row of X, 16-byte ones of B and C
    static constexpr int UX = (TT / 4) * XCW;            // X units: 4 tokens x 4 columns
    static constexpr int UB = (TT / 4) * BCW;            // B units: 4 tokens x 8 n
    static constexpr int UC = TT / 4 * BCW;              // C pieces per output wave: 16 tokens x 8 n
    static constexpr int RX = (UX + 255) / 256, RB = (UB + 255) / 256, RC = (UC + 63) / 64;
    static constexpr int kDepth = (NT % 2 == 0) ? 2 : 1;
    // log-decays for the staging of the next tile come from LDS when a chunk
    // has at least two tiles (the next chunk's are written a tile early)
    static constexpr bool kCsLds = NT >= 2;
    static constexpr bool kOk = PW % 32 == 0 && N % 64 == 0 && Q % TT == 0 && LDS <= 160 * 1024 &&
                                UX % 64 == 0 && UB % 64 == 0 && UC % 64 == 0;
};

template <int... Is, typename F>
__device__ __forceinline__ void rs_static_for_impl(F &&f, std::integer_sequence<int, Is...>) {
    (f(std::integral_constant<int, Is>{}), ...);
}
template <int Count, typename F>
__device__ __forceinline__ void rs_static_for(F &&f) {
    rs_static_for_impl(f, std::make_integer_sequence<int, Count>{});
}

// LDS row of B^T (and accumulator row of the state) that holds state index n.
__device__ __forceinline__ constexpr int rs_row_of_n(int n) {
    return (n & ~31) + 16 * ((n & 7) >> 2) + 4 * ((n >> 3) & 3) + (n & 3);
}

// Token-major LDS tiles (X^T, B^T) keep each row's 16-byte pieces (8 tokens)
// in a permuted order, piece k of row rho at position k ^ swz(rho). The
// permutation is the same for every aligned group of 8 rows, so the
// matrix-core reads (8 consecutive rows per bank cycle) stay conflict-free,
// and it spreads the staging writes: a 16-lane write group holds 8 staging
// units of 2 consecutive token quads, whose rows differ in the bits that
// swz folds into the piece position (rows 4 c + e of X^T, rows rho(8 c + e)
// of B^T, c the unit's column group).
__device__ __forceinline__ constexpr int rs_xswz(int p) { return ((p >> 3) & 1) | (((p >> 4) & 1) << 1); }
__device__ __forceinline__ constexpr int rs_bswz(int rho) { return ((rho >> 3) & 1) | (((rho >> 5) & 1) << 1); }

// staging unit u: token quad (u / 8) % 16, column group 8 (u / 128) + u % 8
__device__ __forceinline__ constexpr int rs_unit_tq(int u) { return (u >> 3) & 15; }
__device__ __forceinline__ constexpr int rs_unit_col(int u) { return 8 * (u >> 7) + (u & 7); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const bf16x2 v = {(bf16)lo, (bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}
// Bit casts go through these by-value scalars: a bit cast applied directly to
// an element of an ext_vector value reads element 0 whatever the index.
__device__ __forceinline__ uint32_t f32_bits(float v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ float bits_f32(uint32_t v) { return __builtin_bit_cast(float, v); }
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// The output gate y SiLU(z) = y z / (1 + e^-z) with the hardware's 2^x and
// reciprocal (each within about 1 ulp in fp32; the result is rounded to bf16):
// 4 instructions instead of a full-precision exp and divide.
__device__ __forceinline__ float rs_gate(float y, float z) {
    return y * z * __builtin_amdgcn_rcpf(1.f + fast_exp2(-kLog2e * z));
}

}  // namespace

template <int Q, int PW, int N, bool kGate, bool kConv>
__global__ __launch_bounds__(512, 1) void k_walk_rs(WalkArgs a) {
    using Tr = Traits<bf16>;
    using frag = bf16x8;
    using Cfg = RsCfg<Q, PW, N>;
    constexpr int TT = Cfg::TT, NT = Cfg::NT, NH = Cfg::NH, PH = Cfg::PH, NBH = Cfg::NBH, PBH = Cfg::PBH;
    constexpr int NM = Cfg::NM, NK = Cfg::NK, KS = Cfg::KS, IB = Cfg::IB, LD = Cfg::LD, XF = Cfg::XF;
    constexpr int RX = Cfg::RX, RB = Cfg::RB, RC = Cfg::RC, BCW = Cfg::BCW, kDepth = Cfg::kDepth;
    constexpr bool kCsLds = Cfg::kCsLds;
    __shared__ __attribute__((aligned(16))) char smem[Cfg::LDS];
    bf16 *XW = reinterpret_cast<bf16 *>(smem + Cfg::XW_OFF);
    bf16 *YSB = reinterpret_cast<bf16 *>(smem + Cfg::YS_OFF);
    bf16 *BTB = reinterpret_cast<bf16 *>(smem + Cfg::BT_OFF);
    char *XCH = smem + Cfg::XCH_OFF;
    float *CSB = reinterpret_cast<float *>(smem + Cfg::CS_OFF);

    const int H = a.H, G = a.G, T = a.T, P = a.P, NS = a.NS;
    const int ntiles = a.nC * NT;
    // blockIdx -> (b, h, segment, slice) as in k_chunk_walk: consecutive logical
    // indices share an XCD (dispatch goes round-robin over the 8 XCDs)
    const int SL = a.SL, S = a.S;
    const int W = a.batch * H * SL * NS;
    int L = blockIdx.x;
    if ((W & 7) == 0) L = (blockIdx.x & 7) * (W >> 3) + (blockIdx.x >> 3);
    const int ps = L % NS;
    const int seg = (L / NS) % SL;
    const int bhi = (L / NS) / SL;
    const int b = bhi / H, h = bhi - b * H;
    const int g = (h * G) / H;
    const int p0 = ps * PW;
    int s0, slen;
    if (a.cu) {
        s0 = min(max(a.cu[b], 0), a.total);
        const int s1 = min(max(a.cu[b + 1], s0), a.total);
        slen = min(s1 - s0, T);
    } else {
        s0 = b * T;
        slen = T;
    }
    const int nCb = (slen + Q - 1) / Q;
    const int cb = seg * a.cps, ce = min(cb + a.cps, nCb);
    const int last_tile = max(ce * NT - 1, cb * NT);
    const size_t bhs = (size_t)bhi;
    const float *init_mat = (seg == 0) ? (a.init ? a.init + bhs * P * N : nullptr)
                                       : a.seg + (bhs * (S - 1) * a.segk + seg * a.segk - 1) * P * N;
    float *out_mat = (seg == S - 1 && a.final_state) ? a.final_state + bhs * P * N : nullptr;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, kg = lane >> 4;
    const int st = tid & 255;  // thread index within the role
    // both roles use the same (a, b) split: a the n half (state) or token half
    // (output), b the half of the slice's columns
    const int ah = wv & 1, bh = (wv >> 1) & 1;

    const size_t xslab = (size_t)slen * H * P * 2, x0 = (size_t)s0 * H * P * 2;
    const size_t bslab = (size_t)slen * G * N * 2, b0 = (size_t)s0 * G * N * 2;
    const rsrc_t rx = make_rsrc(reinterpret_cast<const char *>(a.X) + x0, (uint32_t)xslab);
    const float *cs_row = a.cs2 + ((size_t)b * H + h) * a.Tpad;
    const float *cp_row = a.dtf + ((size_t)b * H + h) * a.Tpad;  // cs' = cs2 - log2(dt)
    const uint32_t x_tok = (uint32_t)(H * P * 2), b_tok = (uint32_t)(G * N * 2);
    const uint32_t hp0 = (uint32_t)((h * P + p0) * 2);

    for (int k = tid; k < Q; k += 512) {
        CSB[k] = cs_row[cb * Q + k];
        CSB[Q + k] = cp_row[cb * Q + k];
    }
    // element offset of 16-byte piece k (8 tokens) of row p in an X^T slot / row rho of a B^T slot
    auto xw_off = [](int p, int k) __attribute__((always_inline)) { return p * LD + 8 * (k ^ rs_xswz(p)); };
    auto bt_off = [](int rho, int k) __attribute__((always_inline)) { return rho * LD + 8 * (k ^ rs_bswz(rho)); };
    // exchange slot: [slot][writer (b, a)][fragment][lane], 16 bytes each
    auto xch_frag = [&](int slot, int w, int f) __attribute__((always_inline)) {
        return reinterpret_cast<u32x4 *>(XCH + slot * Cfg::XCH_BYTES + ((w * XF + f) * 64 + lane) * 16);
    };

    // X staging (units of 4 tokens x 4 columns, loaded two tiles ahead, each
    // role lane st taking the same units): the output waves' job, or the state
    // waves' when the input convolution is fused in (it would otherwise sit on
    // the output waves, the role every tile waits for)
    constexpr bool kXS = kConv;
    uint32_t vx[RX];
#pragma unroll
    for (int k = 0; k < RX; ++k) {
        const int u = st + 256 * k;
        vx[k] = oob_if(u >= Cfg::UX, (uint32_t)(4 * rs_unit_tq(u)) * x_tok + (uint32_t)(8 * rs_unit_col(u)));
    }
    u32x2 xr[kDepth][RX][4];
    // input convolution: the 3 tokens before each unit, and the unit's
    // columns' taps and bias (a lane's units keep their columns on every tile)
    u32x2 xhalo[kDepth][RX][kConv ? 3 : 1];
    f32x4 ctap[RX][kConv ? 4 : 1];
    float cbias[RX][kConv ? 4 : 1];
    auto init_conv = [&]() __attribute__((always_inline)) {
        if constexpr (kConv) {
#pragma unroll
            for (int k = 0; k < RX; ++k) {
                const int u = st + 256 * k;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int col = h * P + p0 + (u < Cfg::UX ? 4 * rs_unit_col(u) + e : 0);
                    ctap[k][e] = *reinterpret_cast<const f32x4 *>(a.conv_w + 4 * (size_t)col);
                    cbias[k][e] = a.conv_b ? a.conv_b[col] : 0.f;
                }
            }
        }
    };
    auto issue_x = [&](int tt, auto Sc) __attribute__((always_inline)) {
        constexpr int Sx = decltype(Sc)::value;
        const uint32_t sx = (uint32_t)tt * x_tok + hp0;
#pragma unroll
        for (int k = 0; k < RX; ++k) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                xr[Sx][k][i] = __builtin_amdgcn_raw_buffer_load_b64(rx, vx[k] + i * x_tok, sx, 0);
            if constexpr (kConv) {
                const int u = st + 256 * k;
                const int row0 = tt + 4 * rs_unit_tq(u) - 3;  // token of halo row 0 (before the sequence: 0)
#pragma unroll
                for (int i = 0; i < 3; ++i)
                    xhalo[Sx][k][i] = __builtin_amdgcn_raw_buffer_load_b64(
                        rx, oob_if(u >= Cfg::UX || row0 + i < 0,
                                   (uint32_t)(row0 + i) * x_tok + hp0 + (uint32_t)(8 * rs_unit_col(u))),
                        0, 0);
            }
        }
    };
    // writes the weighted X of a tile (and the plain X in per-element
    // tiles) into X slot `slot`; cr / ce: cs2 before the tile and at its
    // last token, cpk(k): cs' of unit k's 4 tokens
    auto stage_x = [&](auto Sc, int slot, float cr, float ce, auto &&cpk) __attribute__((always_inline)) {
        constexpr int Sx = decltype(Sc)::value;
        const bool fd = (cr - ce <= kRsFDMax);
        bf16 *XWs = XW + slot * PW * LD;
        bf16 *XRs = reinterpret_cast<bf16 *>(smem + Cfg::XR_OFF + slot * Cfg::XR_BYTES);
#pragma unroll
        for (int k = 0; k < RX; ++k) {
            const int u = st + 256 * k;
            if (u >= Cfg::UX) continue;  // wave-uniform (UX is a multiple of 64)
            const int tq = rs_unit_tq(u), c4 = rs_unit_col(u);
            // the unit's 4 tokens x 4 columns (after the input convolution
            // when there is one, rounded to bf16: the scan's input and the
            // skip term's)
            u32x2 xin[4];
            if constexpr (kConv) {
                // x' = SiLU(b + w0 x_{t-3} + w1 x_{t-2} + w2 x_{t-1} + w3 x_t)
                float xo[4][4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float xv[7];  // tokens 4 tq - 3 .. 4 tq + 3 of column 4 c4 + e
#pragma unroll
                    for (int i = 0; i < 3; ++i)
                        xv[i] = (e & 1) ? bf16_hi(xhalo[Sx][k][i][e >> 1]) : bf16_lo(xhalo[Sx][k][i][e >> 1]);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        xv[3 + i] = (e & 1) ? bf16_hi(xr[Sx][k][i][e >> 1]) : bf16_lo(xr[Sx][k][i][e >> 1]);
                    const f32x4 w = ctap[k][e];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float v = cbias[k][e] + w[0] * xv[i] + w[1] * xv[i + 1] + w[2] * xv[i + 2] +
                                        w[3] * xv[i + 3];
                        xo[i][e] = v * __builtin_amdgcn_rcpf(1.f + fast_exp2(-kLog2e * v));
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    xin[i] = u32x2{pack_bf16x2(xo[i][0], xo[i][1]), pack_bf16x2(xo[i][2], xo[i][3])};
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) xin[i] = xr[Sx][k][i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<u32x2 *>(XRs + (4 * tq + i) * Cfg::XRLD + 4 * c4) = xin[i];
            // factored tiles: X~_j = 2^(cs_r - cs'_j) x_j; the others: x_j as it is
            const f32x4 cp = cpk(k);
            float cw[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) cw[i] = fd ? fast_exp2(cr - cp[i]) : 1.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // column 4 c4 + e, its 4 tokens 4 tq .. 4 tq + 3: half of 16-byte piece tq / 2
                float xv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) xv[i] = (e & 1) ? bf16_hi(xin[i][e >> 1]) : bf16_lo(xin[i][e >> 1]);
                *reinterpret_cast<u32x2 *>(XWs + xw_off(4 * c4 + e, tq >> 1) + 4 * (tq & 1)) =
                    u32x2{pack_bf16x2(xv[0] * cw[0], xv[1] * cw[1]), pack_bf16x2(xv[2] * cw[2], xv[3] * cw[3])};
            }
        }
    };
    // stages a tile whose log-decays are read from global memory
    auto stage_x_global = [&](auto Sc, int tau) __attribute__((always_inline)) {
        const int tt = tau * TT;
        const float cr = (tt % Q == 0) ? 0.f : cs_row[tt - 1];
        const float ce = cs_row[tt + TT - 1];
        stage_x(Sc, tau & 1, cr, ce, [&](int k) __attribute__((always_inline)) {
            return *reinterpret_cast<const f32x4 *>(cp_row + tt + 4 * rs_unit_tq(st + 256 * k));
        });
    };


    if (wv < 4) {
        // ============================ output waves ============================
        const float Dh = a.D[h];
        const rsrc_t rg = make_rsrc(a.Gbuf, a.g_bytes);
        const rsrc_t rcm = make_rsrc(reinterpret_cast<const char *>(a.C) + b0, (uint32_t)bslab);
        const rsrc_t rz = make_rsrc(reinterpret_cast<const char *>(a.z) + (kGate ? x0 : 0),
                                    kGate ? (uint32_t)xslab : 0u);
        const size_t gbase = ((size_t)b * G + g) * ntiles;
        // After the pairwise lane swap of the epilogue a lane holds 8 consecutive
        // columns of its token per pair of p-blocks: column offset pbase + 32 q.
        constexpr int NPQ = (PBH + 1) / 2;
        const int pbase = (PBH >= 2) ? 16 * (kg & 1) + 8 * (kg >> 1) : 4 * kg;
        uint32_t vgo[IB];
#pragma unroll
        for (int ib = 0; ib < IB; ++ib) {
            const int il = 32 * ah + 16 * ib + r;  // tile-local token of this lane's column
            vgo[ib] = (uint32_t)((il * TT + 8 * kg) * 2);
        }
        using xvec = typename std::conditional<(PBH >= 2), u32x4, u32x2>::type;
        frag gf[IB][KS];          // C B^T fragments: k-step ks covers tokens 32 ks + 8 kg .. + 7
        auto load_g = [&](int tau) __attribute__((always_inline)) {
            const uint32_t sg = (uint32_t)((gbase + tau) * (size_t)(TT * TT * 2));
#pragma unroll
            for (int ib = 0; ib < IB; ++ib)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    gf[ib][ks] = Tr::load_frag_s(rg, oob_if(ks > ah, vgo[ib] + ks * 64), sg);
        };
        // C staging: this wave loads 16 of the 32 rows its token half needs
        // (rows 32 ah + 16 bh ..) a tile ahead as whole lines, and writes them
        // into the next tile's LDS slot before the barrier
        uint32_t vcs[RC];
#pragma unroll
        for (int k = 0; k < RC; ++k) {
            const int u = lane + 64 * k;
            vcs[k] = (uint32_t)(32 * ah + 16 * bh + u / BCW) * b_tok + (uint32_t)(16 * (u % BCW));
        }
        u32x4 crg[RC];
        auto load_cs = [&](int tt) __attribute__((always_inline)) {
            const uint32_t sb = (uint32_t)(tt * G + g) * (uint32_t)(N * 2);
#pragma unroll
            for (int k = 0; k < RC; ++k) crg[k] = buf_ld128s(rcm, vcs[k], sb);
        };
        auto store_cs = [&](int slot) __attribute__((always_inline)) {
            bf16 *CLw = reinterpret_cast<bf16 *>(smem + Cfg::C_OFF + slot * Cfg::C_BYTES);
#pragma unroll
            for (int k = 0; k < RC; ++k) {
                const int u = lane + 64 * k;
                *reinterpret_cast<u32x4 *>(CLw + (32 * ah + 16 * bh + u / BCW) * Cfg::CLD + 8 * (u % BCW)) = crg[k];
            }
        };
        // The output rows of tile tau, staged in LDS slot tau % 2 by all four
        // output waves, leave as whole rows at the start of tile tau + 1: 16
        // rows per wave, PW / 8 lanes per row.
        const rsrc_t ry = make_rsrc(reinterpret_cast<char *>(a.Y) + x0, (uint32_t)xslab);
        constexpr int YP = PW / 8;             // 16-byte pieces per row
        constexpr int YRI = 64 / YP;           // rows per store instruction
        // The gate y * SiLU(z) acts here, on the output rounded to bf16, with z
        // read in the same whole-row pieces a tile ahead of its rows' store.
        u32x4 zrow[kGate ? 16 / YRI : 1];
        auto load_z = [&](int tau) __attribute__((always_inline)) {
            if constexpr (kGate) {
                const uint32_t sy = (uint32_t)(tau * TT) * x_tok + hp0;
#pragma unroll
                for (int k = 0; k < 16 / YRI; ++k) {
                    const int row = 16 * wv + YRI * k + lane / YP, pc = lane % YP;
                    zrow[k] = buf_ld128s(rz, (uint32_t)row * x_tok + (uint32_t)(16 * pc), sy);
                }
            }
        };
        auto store_y = [&](int tau) __attribute__((always_inline)) {
            const bf16 *YSs = YSB + (tau & 1) * TT * Cfg::YLD;
            const uint32_t sy = (uint32_t)(tau * TT) * x_tok + hp0;
#pragma unroll
            for (int k = 0; k < 16 / YRI; ++k) {
                const int row = 16 * wv + YRI * k + lane / YP, pc = lane % YP;
                u32x4 v = *reinterpret_cast<const u32x4 *>(YSs + row * Cfg::YLD + 8 * pc);
                if constexpr (kGate) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        v[e] = pack_bf16x2(rs_gate(bf16_lo(v[e]), bf16_lo(zrow[k][e])),
                                           rs_gate(bf16_hi(v[e]), bf16_hi(zrow[k][e])));
                }
                buf_st128s(v, ry, (uint32_t)row * x_tok + (uint32_t)(16 * pc), sy);
            }
        };

        const int tile_b = cb * NT;
        load_z(tile_b);
        load_cs(tile_b * TT);
        if constexpr (!kXS) issue_x(tile_b * TT, std::integral_constant<int, 0>{});
        store_cs(tile_b & 1);
        if constexpr (!kXS) {
            stage_x_global(std::integral_constant<int, 0>{}, tile_b);
            if constexpr (kDepth == 2) issue_x(min(tile_b + 1, last_tile) * TT, std::integral_constant<int, 1>{});
        }
        load_g(tile_b);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        for (int c = cb; c < ce; ++c) {
            const float *CSL = CSB + ((c - cb) & 1) * 2 * Q;
            const float *CPL = CSL + Q;
            rs_static_for<NT>([&](auto Ic) __attribute__((always_inline)) {
                constexpr int I = decltype(Ic)::value;
                const int tile0 = I * TT;
                const int tau = c * NT + I;
                const int slot = tau & 1;
                load_cs(min(tau + 1, last_tile) * TT);
                if constexpr (!kXS)
                    issue_x(min(tau + kDepth, last_tile) * TT, std::integral_constant<int, kDepth == 2 ? (I & 1) : 0>{});
                // the previous tile's output (its rows were completed before the
                // barrier), then the gate values of this tile's rows
                if (tau > cb * NT) {
                    store_y(tau - 1);
                    load_z(tau);
                }
                // the state at the tile's start, rows p of half bh, both n halves
                frag hs[2][NM][PBH];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int m = 0; m < NM; ++m)
#pragma unroll
                        for (int pb = 0; pb < PBH; ++pb)
                            hs[hh][m][pb] = __builtin_bit_cast(frag, *xch_frag(slot, 2 * bh + hh, m * PBH + pb));
                // C rows of this wave's tokens
                const bf16 *CL = reinterpret_cast<const bf16 *>(smem + Cfg::C_OFF + slot * Cfg::C_BYTES);
                frag cf[IB][NK];  // k-step kk covers n = 32 kk + 8 kg .. + 7
#pragma unroll
                for (int ib = 0; ib < IB; ++ib)
#pragma unroll
                    for (int kk = 0; kk < NK; ++kk)
                        cf[ib][kk] = Tr::lds_frag(CL + (32 * ah + 16 * ib + r) * Cfg::CLD + 32 * kk + 8 * kg);
                const float cs_ref = (I > 0) ? CSL[tile0 - 1] : 0.f;
                const float cs_end = CSL[tile0 + TT - 1];
                float cs_i[IB];
#pragma unroll
                for (int ib = 0; ib < IB; ++ib) cs_i[ib] = CSL[tile0 + 32 * ah + 16 * ib + r];
                // the next tile's weighted X into the other slots, while this
                // tile's operands arrive (its X slot was last read a tile ago)
                if constexpr (!kXS) {
                    constexpr int SxN = kDepth == 2 ? ((I + 1) & 1) : 0;
                    if constexpr (kCsLds) {
                        // (after the last tile this stages data nobody reads)
                        const float *CSn = (I + 1 < NT) ? CSL : CSB + ((c + 1 - cb) & 1) * 2 * Q;
                        const int tn = ((I + 1) % NT) * TT;
                        const float cr = (I + 1 < NT) ? CSn[tn - 1] : 0.f;
                        stage_x(std::integral_constant<int, SxN>{}, (tau + 1) & 1, cr, CSn[tn + TT - 1],
                                [&](int k) __attribute__((always_inline)) {
                                    return *reinterpret_cast<const f32x4 *>(CSn + Q + tn + 4 * rs_unit_tq(st + 256 * k));
                                });
                    } else {
                        stage_x_global(std::integral_constant<int, SxN>{}, min(tau + 1, last_tile));
                    }
                }
                // state -> output: Y^T[p][i] = sum_n h[p][n] C[i][n]
                f32x4 yacc[IB][PBH];
#pragma unroll
                for (int ib = 0; ib < IB; ++ib)
#pragma unroll
                    for (int pb = 0; pb < PBH; ++pb) yacc[ib][pb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < NK; ++kk)
#pragma unroll
                    for (int pb = 0; pb < PBH; ++pb)
#pragma unroll
                        for (int ib = 0; ib < IB; ++ib)
                            yacc[ib][pb] = Tr::mma(hs[kk / NM][kk % NM][pb], cf[ib][kk], yacc[ib][pb]);
                const bool fd = (cs_ref - cs_end <= kRsFDMax);
                // the diagonal block's X (weighted in factored tiles)
                const bf16 *XD = XW + slot * PW * LD;
                frag xd[KS][PBH];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                    for (int pb = 0; pb < PBH; ++pb)
                        xd[ks][pb] = Tr::lds_frag(XD + xw_off(PH * bh + 16 * pb + r, 4 * ks + kg));
                // row factors 2^(cs_i - cs_ref): one token per lane and 16-token block
                float fr[IB];
#pragma unroll
                for (int ib = 0; ib < IB; ++ib) fr[ib] = fast_exp2(cs_i[ib] - cs_ref);
#pragma unroll
                for (int ib = 0; ib < IB; ++ib)
#pragma unroll
                    for (int pb = 0; pb < PBH; ++pb) yacc[ib][pb] *= fd ? 1.f : fr[ib];
                if (!fd) {
                    // per-element weights on C B^T: G_ij 2^(cs_i - cs'_j), j <= i
#pragma unroll
                    for (int ib = 0; ib < IB; ++ib) {
                        const int il = 32 * ah + 16 * ib + r;
#pragma unroll
                        for (int ks = 0; ks < KS; ++ks) {
                            const int j0 = 32 * ks + 8 * kg;
                            const f32x4 cpa = *reinterpret_cast<const f32x4 *>(CPL + tile0 + j0);
                            const f32x4 cpb = *reinterpret_cast<const f32x4 *>(CPL + tile0 + j0 + 4);
#pragma unroll
                            for (int e = 0; e < 8; ++e) {
                                const float cpj = e < 4 ? cpa[e] : cpb[e - 4];
                                const float v = Tr::frag_get(gf[ib][ks], e) * fast_exp2(cs_i[ib] - cpj);
                                Tr::frag_set(gf[ib][ks], e, (j0 + e <= il) ? v : 0.f);
                            }
                        }
                    }
                }
                // diagonal block: Y^T[p][i] += sum_{j <= i} X~^T[p][j] G[i][j]. The
                // first token half's k-step over tokens 32..63 multiplies zeros
                // (its C B^T fragments read as 0), so every wave runs the same
                // matrix-core ops with no branch next to them.
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                    for (int pb = 0; pb < PBH; ++pb)
#pragma unroll
                        for (int ib = 0; ib < IB; ++ib) yacc[ib][pb] = Tr::mma(xd[ks][pb], gf[ib][ks], yacc[ib][pb]);
#pragma unroll
                for (int ib = 0; ib < IB; ++ib)
#pragma unroll
                    for (int pb = 0; pb < PBH; ++pb) yacc[ib][pb] *= fd ? fr[ib] : 1.f;
                load_g(min(tau + 1, last_tile));
                // skip term, gate, store. Pairs of p-blocks swap halves between
                // lanes 16 apart, after which a lane holds 8 consecutive columns of its token.
                const bf16 *XRs = reinterpret_cast<const bf16 *>(smem + Cfg::XR_OFF + slot * Cfg::XR_BYTES);
                bf16 *YSs = YSB + slot * TT * Cfg::YLD;
#pragma unroll
                for (int ib = 0; ib < IB; ++ib)
#pragma unroll
                    for (int q = 0; q < NPQ; ++q) {
                        constexpr int NE = (PBH >= 2) ? 8 : 4;
                        float y[NE];
                        if constexpr (PBH >= 2) {
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const auto sw = __builtin_amdgcn_permlane16_swap(f32_bits(yacc[ib][2 * q][i]),
                                                                                 f32_bits(yacc[ib][2 * q + 1][i]), false, false);
                                y[i] = bits_f32(sw[0]);
                                y[4 + i] = bits_f32(sw[1]);
                            }
                        } else {
#pragma unroll
                            for (int i = 0; i < 4; ++i) y[i] = yacc[ib][0][i];
                        }
                        // x of this lane's token and columns, from the X rows staged in LDS
                        const xvec xv = *reinterpret_cast<const xvec *>(
                            XRs + (32 * ah + 16 * ib + r) * Cfg::XRLD + PH * bh + 32 * q + pbase);
#pragma unroll
                        for (int e = 0; e < NE; e += 2) {
                            y[e] += Dh * bf16_lo(xv[e / 2]);
                            y[e + 1] += Dh * bf16_hi(xv[e / 2]);
                        }
                        xvec o;
#pragma unroll
                        for (int e = 0; e < NE; e += 2) o[e / 2] = pack_bf16x2(y[e], y[e + 1]);
                        *reinterpret_cast<xvec *>(YSs + (32 * ah + 16 * ib + r) * Cfg::YLD + PH * bh + 32 * q + pbase) = o;
                    }
                // the next tile's C rows into the other slot
                store_cs((tau + 1) & 1);
                __syncthreads();
            });
        }
        // the last tile's output (the state waves pass the same barrier)
        __syncthreads();
        if (ce > cb) store_y(ce * NT - 1);
    } else {
        // ============================ state waves ============================
        const rsrc_t rbm = make_rsrc(reinterpret_cast<const char *>(a.B) + b0, (uint32_t)bslab);
        // transposed state: hacc[nb][pb][i] = h[p = PH bh + 16 pb + r][n = sigma(rho)],
        // rho = NH ah + 16 nb + 4 kg + i, i.e. n = NH ah + 32 (nb / 2) + 8 kg + 4 (nb % 2) + i
        f32x4 hacc[NBH][PBH];
#pragma unroll
        for (int nb = 0; nb < NBH; ++nb)
#pragma unroll
            for (int pb = 0; pb < PBH; ++pb) {
                f32x4 v = {0.f, 0.f, 0.f, 0.f};
                if (init_mat) {
                    const int p = p0 + PH * bh + 16 * pb + r;
                    const int n = NH * ah + 32 * (nb / 2) + 8 * kg + 4 * (nb % 2);
                    v = *reinterpret_cast<const f32x4 *>(init_mat + (size_t)p * N + n);
                }
                hacc[nb][pb] = v;
            }
        // publishes the state in bf16 as the A operand of the state -> output
        // product: row p, the 8 consecutive n of k-step m of this half
        auto publish = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
                for (int pb = 0; pb < PBH; ++pb) {
                    const f32x4 lo = hacc[2 * m][pb], hi = hacc[2 * m + 1][pb];
                    *xch_frag(slot, 2 * bh + ah, m * PBH + pb) =
                        u32x4{pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]), pack_bf16x2(hi[0], hi[1]),
                              pack_bf16x2(hi[2], hi[3])};
                }
        };
        // B staging: units of 4 tokens x 8 n, loaded two tiles ahead
        uint32_t vb[RB];
#pragma unroll
        for (int k = 0; k < RB; ++k) {
            const int u = st + 256 * k;
            vb[k] = oob_if(u >= Cfg::UB, (uint32_t)(4 * rs_unit_tq(u)) * b_tok + (uint32_t)(16 * rs_unit_col(u)));
        }
        u32x4 br[kDepth][RB][4];
        auto issue_b = [&](int tt, auto Sc) __attribute__((always_inline)) {
            constexpr int Sx = decltype(Sc)::value;
            const uint32_t sb = (uint32_t)(tt * G + g) * (uint32_t)(N * 2);
#pragma unroll
            for (int k = 0; k < RB; ++k)
#pragma unroll
                for (int i = 0; i < 4; ++i) br[Sx][k][i] = buf_ld128s(rbm, vb[k] + i * b_tok, sb);
        };
        // writes B^T of a tile into slot `slot`: as it is in factored tiles,
        // weighted by w_j = 2^(cs_e - cs'_j) in the others; cr / ce: cs2 before
        // the tile and at its last token, cpk(k): cs' of unit k's 4 tokens
        auto stage_b = [&](auto Sc, int slot, float cr, float ce, auto &&cpk) __attribute__((always_inline)) {
            constexpr int Sx = decltype(Sc)::value;
            const bool fd = (cr - ce <= kRsFDMax);
            bf16 *BT = BTB + slot * N * LD;
#pragma unroll
            for (int k = 0; k < RB; ++k) {
                const int u = st + 256 * k;
                if (u >= Cfg::UB) continue;  // wave-uniform (UB is a multiple of 64)
                const int tq = rs_unit_tq(u), c8 = rs_unit_col(u);
                if (fd) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        // element e of the 8 n of this unit, for its 4 tokens
                        uint32_t w[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) w[i] = br[Sx][k][i][e >> 1];
                        // tokens 0 and 1 in the low and high halves of the first word, 2 and 3 of the second
                        const u32x2 v = (e & 1) ? u32x2{(w[0] >> 16) | (w[1] & 0xffff0000u), (w[2] >> 16) | (w[3] & 0xffff0000u)}
                                                : u32x2{(w[0] & 0xffffu) | (w[1] << 16), (w[2] & 0xffffu) | (w[3] << 16)};
                        *reinterpret_cast<u32x2 *>(BT + bt_off(rs_row_of_n(8 * c8 + e), tq >> 1) + 4 * (tq & 1)) = v;
                    }
                } else {
                    const f32x4 cp = cpk(k);
                    float wt[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) wt[i] = fast_exp2(ce - cp[i]);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        float bv[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            bv[i] = ((e & 1) ? bf16_hi(br[Sx][k][i][e >> 1]) : bf16_lo(br[Sx][k][i][e >> 1])) * wt[i];
                        *reinterpret_cast<u32x2 *>(BT + bt_off(rs_row_of_n(8 * c8 + e), tq >> 1) + 4 * (tq & 1)) =
                            u32x2{pack_bf16x2(bv[0], bv[1]), pack_bf16x2(bv[2], bv[3])};
                    }
                }
            }
        };
        // stages a tile whose log-decays are read from global memory
        auto stage_b_global = [&](auto Sc, int tau) __attribute__((always_inline)) {
            const int tt = tau * TT;
            const float cr = (tt % Q == 0) ? 0.f : cs_row[tt - 1];
            const float ce = cs_row[tt + TT - 1];
            stage_b(Sc, tau & 1, cr, ce, [&](int k) __attribute__((always_inline)) {
                return *reinterpret_cast<const f32x4 *>(cp_row + tt + 4 * rs_unit_tq(st + 256 * k));
            });
        };
        const int tile_b = cb * NT;
        if constexpr (kXS) init_conv();
        publish(tile_b & 1);
        issue_b(tile_b * TT, std::integral_constant<int, 0>{});
        if constexpr (kXS) issue_x(tile_b * TT, std::integral_constant<int, 0>{});
        stage_b_global(std::integral_constant<int, 0>{}, tile_b);
        if constexpr (kXS) stage_x_global(std::integral_constant<int, 0>{}, tile_b);
        if constexpr (kDepth == 2) {
            issue_b(min(tile_b + 1, last_tile) * TT, std::integral_constant<int, 1>{});
            if constexpr (kXS) issue_x(min(tile_b + 1, last_tile) * TT, std::integral_constant<int, 1>{});
        }
        __syncthreads();
        float csn = 0.f, cpn = 0.f;
        for (int c = cb; c < ce; ++c) {
            const int t0 = c * Q;
            const float *CSL = CSB + ((c - cb) & 1) * 2 * Q;
            rs_static_for<NT>([&](auto Ic) __attribute__((always_inline)) {
                constexpr int I = decltype(Ic)::value;
                const int tile0 = I * TT;
                const int tau = c * NT + I;
                const int slot = tau & 1;
                if constexpr (I == 0) {
                    // the next chunk's log-decays (Q <= 256: one per thread), issued
                    // first and written a tile before the chunk's last (or at it,
                    // for single-tile chunks, whose staging reads global memory)
                    const int kn = (c + 1 < ce ? t0 + Q : t0) + min(st, Q - 1);
                    csn = cs_row[kn];
                    cpn = cp_row[kn];
                }
                issue_b(min(tau + kDepth, last_tile) * TT, std::integral_constant<int, kDepth == 2 ? (I & 1) : 0>{});
                if constexpr (kXS)
                    issue_x(min(tau + kDepth, last_tile) * TT, std::integral_constant<int, kDepth == 2 ? (I & 1) : 0>{});
                // the next tile's B^T (and X) into the other slots first (last read a
                // tile ago), while the output waves read their operands
                {
                    constexpr int SxN = kDepth == 2 ? ((I + 1) & 1) : 0;
                    if constexpr (kCsLds) {
                        // (after the last tile this stages data nobody reads)
                        const float *CSn = (I + 1 < NT) ? CSL : CSB + ((c + 1 - cb) & 1) * 2 * Q;
                        const int tn = ((I + 1) % NT) * TT;
                        const float cr = (I + 1 < NT) ? CSn[tn - 1] : 0.f;
                        auto cpk = [&](int k) __attribute__((always_inline)) {
                            return *reinterpret_cast<const f32x4 *>(CSn + Q + tn + 4 * rs_unit_tq(st + 256 * k));
                        };
                        stage_b(std::integral_constant<int, SxN>{}, (tau + 1) & 1, cr, CSn[tn + TT - 1], cpk);
                        if constexpr (kXS) stage_x(std::integral_constant<int, SxN>{}, (tau + 1) & 1, cr, CSn[tn + TT - 1], cpk);
                    } else {
                        stage_b_global(std::integral_constant<int, SxN>{}, min(tau + 1, last_tile));
                        if constexpr (kXS) stage_x_global(std::integral_constant<int, SxN>{}, min(tau + 1, last_tile));
                    }
                }
                // state update: factored tiles h <- dec (h + B^T X~), the others
                // h <- dec h + Bw^T X
                const float cs_ref = (I > 0) ? CSL[tile0 - 1] : 0.f;
                const float cs_end = CSL[tile0 + TT - 1];
                const bool fd = (cs_ref - cs_end <= kRsFDMax);
                const float dec = fast_exp2(cs_end - cs_ref);
                const float pre = fd ? 1.f : dec, post = fd ? dec : 1.f;
                const bf16 *XWs = XW + slot * PW * LD;
                const bf16 *BT = BTB + slot * N * LD;
                frag xw[KS][PBH];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                    for (int pb = 0; pb < PBH; ++pb)
                        xw[ks][pb] = Tr::lds_frag(XWs + xw_off(PH * bh + 16 * pb + r, 4 * ks + kg));
#pragma unroll
                for (int nb = 0; nb < NBH; ++nb)
#pragma unroll
                    for (int pb = 0; pb < PBH; ++pb) hacc[nb][pb] *= pre;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                    for (int nb = 0; nb < NBH; ++nb) {
                        const frag bt = Tr::lds_frag(BT + bt_off(NH * ah + 16 * nb + r, 4 * ks + kg));
#pragma unroll
                        for (int pb = 0; pb < PBH; ++pb) hacc[nb][pb] = Tr::mma(bt, xw[ks][pb], hacc[nb][pb]);
                    }
#pragma unroll
                for (int nb = 0; nb < NBH; ++nb)
#pragma unroll
                    for (int pb = 0; pb < PBH; ++pb) hacc[nb][pb] *= post;
                publish((tau + 1) & 1);
                if constexpr (I == (kCsLds ? NT - 2 : NT - 1)) {
                    if (c + 1 < ce && st < Q) {
                        float *CSN = CSB + ((c + 1 - cb) & 1) * 2 * Q;
                        CSN[st] = csn;
                        CSN[Q + st] = cpn;
                    }
                }
                __syncthreads();
            });
        }
        __syncthreads();  // pairs with the output waves' barrier before the last rows leave
        if (out_mat) {
#pragma unroll
            for (int nb = 0; nb < NBH; ++nb)
#pragma unroll
                for (int pb = 0; pb < PBH; ++pb) {
                    const int p = p0 + PH * bh + 16 * pb + r;
                    const int n = NH * ah + 32 * (nb / 2) + 8 * kg + 4 * (nb % 2);
                    *reinterpret_cast<f32x4 *>(out_mat + (size_t)p * N + n) = hacc[nb][pb];
                }
        }
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
template <int Q, int PW, int N>
static ssd_status run_walk_rs(const FwdArgs &f, hipStream_t s) {
    if constexpr (!RsCfg<Q, PW, N>::kOk) {
        return SSD_ERR_UNSUPPORTED;
    } else {
        WalkArgs wa;
        wa.X = f.X; wa.B = f.B; wa.C = f.C; wa.Y = f.Y; wa.Gbuf = f.Gbuf;
        wa.cs2 = f.cs2; wa.dtf = f.dtf; wa.D = f.D; wa.init = f.init; wa.final_state = f.final_state;
        wa.batch = (int)f.batch; wa.T = (int)f.T; wa.H = (int)f.H; wa.G = (int)f.G; wa.nC = (int)f.nC;
        wa.Tpad = (int)f.Tpad; wa.P = (int)f.P; wa.NS = f.ns; wa.g_bytes = (uint32_t)f.g_bytes;
        wa.S = f.S; wa.cps = f.cps; wa.seg = f.seg; wa.SL = f.S;
        wa.segk = f.conv_w ? 1 : f.segk;  // the convolution walks' pre-pass takes whole segments
        wa.cu = f.cu; wa.total = (int)f.total; wa.z = f.z;
        wa.conv_w = f.conv_w; wa.conv_b = f.conv_b;
        const int64_t heads = f.batch * f.H * f.ns;
        const dim3 grid((unsigned)(heads * f.S));
        hipError_t e;
        if (f.conv_w)
            e = f.z ? launch(k_walk_rs<Q, PW, N, true, true>, grid, dim3(512), s, wa)
                    : launch(k_walk_rs<Q, PW, N, false, true>, grid, dim3(512), s, wa);
        else
            e = f.z ? launch(k_walk_rs<Q, PW, N, true, false>, grid, dim3(512), s, wa)
                    : launch(k_walk_rs<Q, PW, N, false, false>, grid, dim3(512), s, wa);
        return e == hipSuccess ? SSD_OK : SSD_ERR_HIP;
    }
}

template <int Q, int PW>
static ssd_status walk_rs_n(const FwdArgs &f, hipStream_t s) {
    switch (f.N) {
        case 64: return run_walk_rs<Q, PW, 64>(f, s);
        case 128: return run_walk_rs<Q, PW, 128>(f, s);
        default: return SSD_ERR_UNSUPPORTED;
    }
}

template <int Q>
static ssd_status walk_rs_p(const FwdArgs &f, hipStream_t s) {
    switch (f.P / f.ns) {
        case 32: return walk_rs_n<Q, 32>(f, s);
        case 64: return walk_rs_n<Q, 64>(f, s);
        default: return SSD_ERR_UNSUPPORTED;
    }
}

bool walk_rs_supported(const FwdArgs &f) {
    if (f.dtype != SSD_BF16 || f.tt != 64) return false;
    const int64_t pw = f.P / f.ns;
    return (pw == 32 || pw == 64) && (f.N == 64 || f.N == 128) && (f.Q == 64 || f.Q == 128 || f.Q == 256);
}

ssd_status launch_walk_rs(const FwdArgs &f, hipStream_t s) {
    switch (f.Q) {
        case 64: return walk_rs_p<64>(f, s);
        case 128: return walk_rs_p<128>(f, s);
        case 256: return walk_rs_p<256>(f, s);
        default: return SSD_ERR_UNSUPPORTED;
    }
}

}  // namespace ssd
