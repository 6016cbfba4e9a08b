// The end states of a split sequence's segments (all but the last), for the
// state passing between segments (the chunked method of the "Transformers are
// SSMs" reading report, section 3.1, at segment granularity).
//
// Segment s, entered with zero (segment 0 with the caller's initial state h0),
// ends in
//   end_s = sum_{t in s} 2^(decay from t to the segment's end) dt_t x_t B_t^T
//           (+ 2^(D_0) h0 for s = 0, D_0 the first segment's total log-decay).
// With the chunk-local base-2 log-decays cs2 (inclusive) and cs' = cs2 -
// log2 dt from the preparation, a token t of chunk c weighs 2^(S_c - cs'_t),
// S_c the sum of the last cs2 of chunks c .. (the segment's last). No weight
// exceeds dt_t, so the sum is a plain contraction over tokens with no state
// carried from tile to tile: each work-group streams its segment through the
// matrix cores with the loads two tiles ahead. Tiles are taken from the
// segment's end backwards, so S_c is accumulated from its smallest terms.
//
// One work-group (4 wavefronts) per (batch, head, segment, n slice of up to
// 128, p slice of up to 64). A wavefront keeps one 16-column p-block and a
// share of the 16-row n-blocks, so its X fragment is read once per k-step;
// block (nb, pb) holds out^T[n = 16 nb + 4 kg + i][p = 16 pb + r], written as
// 16-byte pieces of 4 consecutive n.
#include <type_traits>

#include "ssd_common.h"
#include "ssd_internal.h"

namespace ssd {

namespace {

struct SegArgs {
    const void *X, *B;
    const float *cs2, *dtf;    // workspace log-decays, (batch, H, Tpad)
    const float *init;         // (batch, H, P, N) or null
    float *seg;                // (batch, H, S - 1, P, N): written
    int T, H, G, P, N, Q, nC, Tpad, S, cps;
};

template <typename TI, int NSL, int PW>
struct SegCfg {
    static constexpr int ES = Traits<TI>::kBytes;
    static constexpr int TT = 64;                    // tile tokens
    static constexpr int VE = 16 / ES;               // elements per 16-byte piece
    // token-major row length: bf16 rows are not padded (their 16-byte pieces
    // are permuted instead, see tok_off), so that three work-groups fit a CU;
    // fp32 rows are padded by 16 bytes
    static constexpr int LD = ES == 2 ? TT : TT + 16 / ES;
    static constexpr int NBLK = NSL / 16, PBLK = PW / 16;
    // wavefront w keeps p-block w % PBLK and every (4 / PBLK)-th n-block from w / PBLK
    static constexpr int NSTEP = 4 / PBLK;
    static constexpr int BPW = (NBLK + NSTEP - 1) / NSTEP;  // accumulator blocks per wavefront
    static constexpr int UB = (TT / 4) * (NSL / VE); // B units: 4 tokens x one 16-byte piece
    static constexpr int UX = (TT / 4) * (PW / VE);  // X units likewise
    static constexpr int RB = (UB + 255) / 256, RX = (UX + 255) / 256;
    static constexpr int BT_ELEMS = NSL * LD, XT_ELEMS = PW * LD;
};

// Element offset of token column c (a multiple of 4) of row rho in a
// token-major LDS tile. bf16: piece c / 8 of the row sits at position
// (c / 8) ^ (rho % 8), so the 8 rows a matrix-core read covers per bank cycle
// (16 bytes each at one piece index) fall in 8 different pieces.
template <typename TI, int LD>
__device__ __forceinline__ int tok_off(int rho, int c) {
    if constexpr (sizeof(TI) == 2) return rho * LD + 8 * ((c >> 3) ^ (rho & 7)) + (c & 7);
    else return rho * LD + c;
}

// element e of a 16-byte piece, as fp32
template <typename TI> __device__ __forceinline__ float piece_elem(const u32x4 &v, int e);
template <> __device__ __forceinline__ float piece_elem<bf16>(const u32x4 &v, int e) {
    const uint32_t w = v[e >> 1];
    return __builtin_bit_cast(float, (e & 1) ? (w & 0xffff0000u) : (w << 16));
}
template <> __device__ __forceinline__ float piece_elem<float>(const u32x4 &v, int e) {
    const uint32_t w = v[e];
    return __builtin_bit_cast(float, w);
}
// element e of 4 tokens' 16-byte pieces w[0..3] into 4 consecutive entries
// of an LDS row, moved as bits (bf16: two halves per word with v_perm_b32)
__device__ __forceinline__ void put_col(bf16 *dst, const u32x4 (&w)[4], int e) {
    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;  // high or low halves of both words
    const int q = e >> 1;
    *reinterpret_cast<u32x2 *>(dst) = u32x2{__builtin_amdgcn_perm(w[1][q], w[0][q], sel),
                                            __builtin_amdgcn_perm(w[3][q], w[2][q], sel)};
}
__device__ __forceinline__ void put_col(float *dst, const u32x4 (&w)[4], int e) {
    *reinterpret_cast<u32x4 *>(dst) = u32x4{w[0][e], w[1][e], w[2][e], w[3][e]};
}
// 4 consecutive tokens of one row into LDS
__device__ __forceinline__ void put4(bf16 *dst, float a, float b, float c, float d) {
    const bf16x2 lo = {(bf16)a, (bf16)b}, hi = {(bf16)c, (bf16)d};
    *reinterpret_cast<u32x2 *>(dst) = u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}
__device__ __forceinline__ void put4(float *dst, float a, float b, float c, float d) {
    *reinterpret_cast<f32x4 *>(dst) = f32x4{a, b, c, d};
}

}  // namespace

template <typename TI, int NSL, int PW>
__global__ __launch_bounds__(256, sizeof(TI) == 2 ? 3 : 1) void k_seg_states(SegArgs a) {
    using Tr = Traits<TI>;
    using Cfg = SegCfg<TI, NSL, PW>;
    constexpr int TT = Cfg::TT, VE = Cfg::VE, LD = Cfg::LD, ES = Cfg::ES;
    constexpr int NBLK = Cfg::NBLK, PBLK = Cfg::PBLK, NSTEP = Cfg::NSTEP, BPW = Cfg::BPW, RB = Cfg::RB,
                  RX = Cfg::RX;
    static_assert(PBLK == 1 || PBLK == 2 || PBLK == 4, "p slice of 16, 32 or 64 columns");
    __shared__ __attribute__((aligned(16))) TI smem[2 * (Cfg::BT_ELEMS + Cfg::XT_ELEMS)];
    TI *BTB = smem;                      // [slot][n][token]
    TI *XTB = smem + 2 * Cfg::BT_ELEMS;  // [slot][p][token], weighted

    const int H = a.H, G = a.G, T = a.T, P = a.P, N = a.N, S = a.S, Q = a.Q;
    // blockIdx -> logical index: dispatch goes round-robin over the 8 XCDs, so
    // consecutive logical indices are given to one XCD. The heads of a group
    // (which read the same B slice) and the slices of a head (the same X) are
    // consecutive: they meet in one L2.
    // logical = ((((b G + g) (S - 1) + seg) nsl + ns) psl + ps) HG + hi
    const int nsl = N / NSL, psl = P / PW, HG = H / G;
    const int W = (int)gridDim.x;
    int x = blockIdx.x;
    if ((W & 7) == 0) x = (x & 7) * (W >> 3) + (x >> 3);
    const int hi = x % HG;
    x /= HG;
    const int ps = x % psl;
    x /= psl;
    const int ns = x % nsl;
    x /= nsl;
    const int seg = x % (S - 1);
    x /= (S - 1);
    const int g = x % G;
    const int b = x / G;
    const int h = g * HG + hi;
    const int bhi = b * H + h;
    const int p0 = ps * PW, n0 = ns * NSL;
    const int tpc = Q / TT;                                 // tiles per chunk
    const int cb = seg * a.cps, ce = min(cb + a.cps, a.nC);
    const int ntl = (ce - cb) * tpc;                        // tiles of this segment
    const int t_first = cb * Q;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, kg = lane >> 4;
    const int pbw = wv % PBLK, nbw = wv / PBLK;  // this wave's p-block and first n-block

    const size_t xslab = (size_t)T * H * P * ES, x0 = (size_t)b * T * H * P * ES;
    const size_t bslab = (size_t)T * G * N * ES, b0 = (size_t)b * T * G * N * ES;
    const rsrc_t rx = make_rsrc(reinterpret_cast<const char *>(a.X) + x0, (uint32_t)xslab);
    const rsrc_t rb = make_rsrc(reinterpret_cast<const char *>(a.B) + b0, (uint32_t)bslab);
    const float *cs_row = a.cs2 + (size_t)bhi * a.Tpad;
    const float *cp_row = a.dtf + (size_t)bhi * a.Tpad;     // cs'
    const uint32_t x_tok = (uint32_t)(H * P * ES), b_tok = (uint32_t)(G * N * ES);

    // staging units of this thread: tokens 4 tq .. + 3 and 16-byte piece pc of the slice
    uint32_t vb[RB], vx[RX];
#pragma unroll
    for (int k = 0; k < RB; ++k) {
        const int u = tid + 256 * k;
        vb[k] = oob_if(u >= Cfg::UB, (uint32_t)(4 * (u % (TT / 4))) * b_tok +
                                         (uint32_t)((g * N + n0 + (u / (TT / 4)) * VE) * ES));
    }
#pragma unroll
    for (int k = 0; k < RX; ++k) {
        const int u = tid + 256 * k;
        vx[k] = oob_if(u >= Cfg::UX, (uint32_t)(4 * (u % (TT / 4))) * x_tok +
                                         (uint32_t)((h * P + p0 + (u / (TT / 4)) * VE) * ES));
    }
    // two register sets: the loads of a tile are issued a whole step before
    // the one that stages it
    u32x4 br[2][RB][4], xr[2][RX][4];
    f32x4 cpr[2][RX];
    auto issue = [&](int tile, auto Rc) __attribute__((always_inline)) {  // tile index within the segment
        constexpr int R = decltype(Rc)::value;
        const int tt = t_first + tile * TT;
#pragma unroll
        for (int k = 0; k < RB; ++k)
#pragma unroll
            for (int i = 0; i < 4; ++i) br[R][k][i] = buf_ld128s(rb, vb[k] + i * b_tok, (uint32_t)tt * b_tok);
#pragma unroll
        for (int k = 0; k < RX; ++k) {
#pragma unroll
            for (int i = 0; i < 4; ++i) xr[R][k][i] = buf_ld128s(rx, vx[k] + i * x_tok, (uint32_t)tt * x_tok);
            cpr[R][k] = *reinterpret_cast<const f32x4 *>(cp_row + tt + 4 * ((tid + 256 * k) % (TT / 4)));
        }
    };
    // writes the tile held in register set R into LDS slot `slot`, X weighted by 2^(sc - cs')
    auto stage = [&](auto Rc, int slot, float sc) __attribute__((always_inline)) {
        constexpr int R = decltype(Rc)::value;
        TI *BT = BTB + slot * Cfg::BT_ELEMS;
        TI *XT = XTB + slot * Cfg::XT_ELEMS;
#pragma unroll
        for (int k = 0; k < RB; ++k) {
            const int u = tid + 256 * k;
            if (u >= Cfg::UB) continue;
            const int tq = u % (TT / 4), pc = u / (TT / 4);
#pragma unroll
            for (int e = 0; e < VE; ++e) put_col(BT + tok_off<TI, LD>(pc * VE + e, 4 * tq), br[R][k], e);
        }
#pragma unroll
        for (int k = 0; k < RX; ++k) {
            const int u = tid + 256 * k;
            if (u >= Cfg::UX) continue;
            const int tq = u % (TT / 4), pc = u / (TT / 4);
            float w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = fast_exp2(sc - cpr[R][k][i]);
#pragma unroll
            for (int e = 0; e < VE; ++e)
                put4(XT + tok_off<TI, LD>(pc * VE + e, 4 * tq), piece_elem<TI>(xr[R][k][0], e) * w[0],
                     piece_elem<TI>(xr[R][k][1], e) * w[1], piece_elem<TI>(xr[R][k][2], e) * w[2],
                     piece_elem<TI>(xr[R][k][3], e) * w[3]);
        }
    };
    auto chunk_total = [&](int tile) __attribute__((always_inline)) {  // last cs2 of the tile's chunk
        return cs_row[(cb + tile / tpc) * Q + Q - 1];
    };

    f32x4 acc[BPW];
#pragma unroll
    for (int j = 0; j < BPW; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // The segment's tiles, last first: tile ntl - 1 - i is computed in step i
    // from LDS slot i % 2. Register set i % 2 held it (staged a step ago) and
    // takes the loads of the tile two before it; set (i + 1) % 2 holds the
    // tile before it, loaded a step ago, staged into the other slot after the
    // products. S_c of the most recently staged tile's chunk is `sc`; a tile
    // that is the last of its chunk adds that chunk's total on staging.
    float sc = 0.f;
    if (ntl > 0) {
        issue(ntl - 1, std::integral_constant<int, 0>{});
        issue(max(ntl - 2, 0), std::integral_constant<int, 1>{});
        sc = chunk_total(ntl - 1);
        stage(std::integral_constant<int, 0>{}, 0, sc);
    }
    __syncthreads();
    auto step = [&](int i, auto Rc) __attribute__((always_inline)) {
        constexpr int R = decltype(Rc)::value;  // i % 2
        const int tile = ntl - 1 - i;
        issue(max(tile - 2, 0), std::integral_constant<int, R>{});
        const TI *BT = BTB + R * Cfg::BT_ELEMS;
        const TI *XT = XTB + R * Cfg::XT_ELEMS;
#pragma unroll
        for (int ks = 0; ks < TT / 32; ++ks) {
            const auto fx = Tr::lds_frag(XT + tok_off<TI, LD>(16 * pbw + r, 32 * ks + 8 * kg));
#pragma unroll
            for (int j = 0; j < BPW; ++j) {
                const int nb = nbw + NSTEP * j;
                if (NBLK % NSTEP != 0 && nb >= NBLK) continue;  // wave-uniform
                acc[j] = Tr::mma(Tr::lds_frag(BT + tok_off<TI, LD>(16 * nb + r, 32 * ks + 8 * kg)), fx, acc[j]);
            }
        }
        // the tile before this one into the other slot (last read a step ago)
        if (tile > 0) {
            if (tile % tpc == 0) sc += chunk_total(tile - 1);  // tile - 1 ends an earlier chunk
            stage(std::integral_constant<int, 1 - R>{}, 1 - R, sc);
        }
        __syncthreads();
    };
    // whole pairs of steps with no branch between them, then the last one
    const int npair = ntl - ntl % 2;
    for (int i = 0; i < npair; i += 2) {
        step(i, std::integral_constant<int, 0>{});
        step(i + 1, std::integral_constant<int, 1>{});
    }
    if (npair < ntl) step(npair, std::integral_constant<int, 0>{});
    // segment 0 starts from the caller's initial state: + 2^(D_0) h0 (sc is D_0 here)
    const size_t bhs = (size_t)bhi;
    const float *h0 = (seg == 0 && a.init) ? a.init + bhs * P * N : nullptr;
    const float d0 = fast_exp2(sc);
    float *out = a.seg + (bhs * (S - 1) + seg) * P * N;
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
        const int nb = nbw + NSTEP * j;
        if (NBLK % NSTEP != 0 && nb >= NBLK) continue;
        const int p = p0 + 16 * pbw + r, n = n0 + 16 * nb + 4 * kg;
        f32x4 v = acc[j];
        if (h0) v += d0 * *reinterpret_cast<const f32x4 *>(h0 + (size_t)p * N + n);
        *reinterpret_cast<f32x4 *>(out + (size_t)p * N + n) = v;
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
template <typename TI, int NSL, int PW>
static ssd_status run_seg_states(const FwdArgs &f, hipStream_t s) {
    SegArgs sa;
    sa.X = f.X; sa.B = f.B; sa.cs2 = f.cs2; sa.dtf = f.dtf; sa.init = f.init; sa.seg = f.seg;
    sa.T = (int)f.T; sa.H = (int)f.H; sa.G = (int)f.G; sa.P = (int)f.P; sa.N = (int)f.N; sa.Q = (int)f.Q;
    sa.nC = (int)f.nC; sa.Tpad = (int)f.Tpad; sa.S = f.S; sa.cps = f.cps;
    const int64_t wgs = f.batch * f.H * (f.S - 1) * (f.N / NSL) * (f.P / PW);
    return launch(k_seg_states<TI, NSL, PW>, dim3((unsigned)wgs), dim3(256), s, sa) == hipSuccess ? SSD_OK
                                                                                                  : SSD_ERR_HIP;
}

template <typename TI, int NSL>
static ssd_status seg_states_p(const FwdArgs &f, hipStream_t s) {
    switch (f.P) {
        case 16: return run_seg_states<TI, NSL, 16>(f, s);
        case 32: return run_seg_states<TI, NSL, 32>(f, s);
        case 64:
        case 128: return run_seg_states<TI, NSL, 64>(f, s);
        default: return SSD_ERR_UNSUPPORTED;
    }
}

template <typename TI>
static ssd_status seg_states_n(const FwdArgs &f, hipStream_t s) {
    switch (f.N) {
        case 16: return seg_states_p<TI, 16>(f, s);
        case 32: return seg_states_p<TI, 32>(f, s);
        case 64: return seg_states_p<TI, 64>(f, s);
        case 128:
        case 256: return seg_states_p<TI, 128>(f, s);
        default: return SSD_ERR_UNSUPPORTED;
    }
}

ssd_status launch_seg_states(const FwdArgs &f, hipStream_t s) {
    if (f.S <= 1) return SSD_OK;
    return f.dtype == SSD_BF16 ? seg_states_n<bf16>(f, s) : seg_states_n<float>(f, s);
}

}  // namespace ssd
