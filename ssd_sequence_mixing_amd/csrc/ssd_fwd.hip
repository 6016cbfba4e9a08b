// Chunked SSD forward for gfx950.
//
// The method ("Transformers are SSMs" reading report, section 3.1): split the
// sequence into chunks of Q tokens; inside a chunk the output is an
// attention-like quadratic product with the decay mask (the diagonal blocks),
// and everything a chunk receives from earlier chunks passes through one
// P x N state per (batch, head), handed from each chunk to the next (the
// low-rank off-diagonal blocks).
//
// Here every chunk is further cut into 64-token tiles and the state is handed
// from tile to tile inside the chunk as well. A chunk's Q x Q quadratic block
// is exactly its 64 x 64 diagonal sub-blocks plus, for each lower sub-block,
// a rank-N term that factors through the state at the sub-block boundary, so
// the result is the same; the work per tile no longer grows with its position
// in the chunk, and only diagonal C B^T tiles are ever formed. The chunk
// length still fixes the segment sums: log-decays are accumulated from each
// chunk's first token.
//
// Two kernels on the caller's stream. k_prepare does two independent jobs in
// one launch:
//   dt_cumsum     per (batch, chunk, head block): dt -> chunk-local inclusive
//                 prefix sum of dt*A in base 2 (cs2), and cs' = cs2 - log2(dt),
//                 both laid out (batch, head, token) fp32. With cs', the
//                 weight dt_j exp2(cs_i - cs_j) of token j seen from token i is
//                 one exponential, exp2(cs_i - cs'_j).
//   tile_cb       per (batch, tile, group): G = C B^T of the tile's 64 tokens
//                 (matrix cores), stored with the entries above the diagonal
//                 zeroed. It depends on the group only, so it is formed once
//                 and shared by every head of the group.
//   k_chunk_walk  per (batch, head): walks the tiles in order with the state
//                 held in matrix-core accumulators. For tile rows i it forms
//                   Y_i = exp2(cs_i - cs_r) C_i h_r^T          (state -> output)
//                       + sum_{j <= i} G_ij exp2(cs_i - cs'_j) X_j (masked diagonal)
//                       + D x_i                                 (skip term)
//                 (r: the token before the tile, h_r the state after it) and
//                 updates h <- exp2(cs_e - cs_r) h + X^T diag(w) B with
//                 w_j = exp2(cs_e - cs'_j), e the tile's last token. X, Y and
//                 the state cross HBM once; the state never leaves the chip
//                 until the final state is written.
//
// In a tile whose decay cs_r - cs_e is at most kFDMax the weights are
// factored about the tile's start: exp2(cs_i - cs'_j) = exp2(cs_i - cs_r)
// exp2(cs_r - cs'_j). The second factor goes on a weighted copy of X,
// Xw_j = exp2(cs_r - cs'_j) x_j, so that
//   Y_i = exp2(cs_i - cs_r) (C_i h_r^T + sum_j G_ij Xw_j) + D x_i
//   h   <- exp2(cs_e - cs_r) (h + Xw^T B)
// with G already masked: no weight is formed per element. Other tiles use
// the per-element form above, where every factor is <= dt.
#include <utility>

#include "ssd_common.h"
#include "ssd_internal.h"

namespace ssd {

// ---------------------------------------------------------------------------
// The tokens of batch element b: [start, start + len). In a packed
// variable-length batch (cu = cumulative sequence lengths, on the device)
// element b is sequence b, clamped to [0, total) and to at most T tokens;
// otherwise every element has T tokens.
// ---------------------------------------------------------------------------
struct SeqRange {
    int start, len;
};
__device__ __forceinline__ SeqRange seq_range(const int *cu, int total, int b, int T) {
    if (!cu) return {b * T, T};
    const int s0 = min(max(cu[b], 0), total);
    const int s1 = min(max(cu[b + 1], s0), total);
    return {s0, min(s1 - s0, T)};
}

// ---------------------------------------------------------------------------
// dt_cumsum: one work-group per (batch, chunk, block of 16 heads)
// ---------------------------------------------------------------------------
constexpr int kCumsumHeads = 16;

template <typename TI, int Q>
__device__ __forceinline__ void dt_cumsum(int blk, const TI *__restrict__ dt, const float *__restrict__ A,
                                          float *__restrict__ cs2, float *__restrict__ dtf, int Tmax, int H,
                                          int nC, int Tpad, const int *cu, int total,
                                          const float *__restrict__ dt_bias, int softplus, float *tile) {
    constexpr int ES = Traits<TI>::kBytes;
    constexpr int LD = Q + 1;  // the caller's tile holds kCumsumHeads * LD floats
    const int hblocks = (H + kCumsumHeads - 1) / kCumsumHeads;
    int x = blk;
    const int c = x % nC;
    x /= nC;
    const int hb = x % hblocks;
    const int b = x / hblocks;
    const int h0 = hb * kCumsumHeads;
    const int Hb = min(kCumsumHeads, H - h0);
    const int t0 = c * Q;
    const SeqRange sq = seq_range(cu, total, b, Tmax);
    const int T = sq.len;
    const rsrc_t r = make_rsrc(reinterpret_cast<const char *>(dt) + (size_t)sq.start * H * ES,
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
        // the optional prologue (bias, softplus) applies to real tokens only:
        // padding keeps dt = 0
        if (dt_bias || softplus) {
#pragma unroll
            for (int hl = 0; hl < kCumsumHeads; ++hl)
                if (hl < Hb && t0 + t < T) v[hl] = dt_prologue(v[hl], dt_bias ? dt_bias[h0 + hl] : 0.f, softplus);
        }
#pragma unroll
        for (int hl = 0; hl < kCumsumHeads; ++hl) tile[hl * LD + t] = v[hl];
    }
    __syncthreads();
    // Thread (head hl, segment sg) takes Q / 16 consecutive tokens: a serial
    // prefix over them, then an exclusive scan of the 16 segment totals
    // across the 16 lanes of the head, then 16-byte stores.
    constexpr int SEG = Q / 16;
    const int hl = threadIdx.x >> 4, sg = threadIdx.x & 15;
    if (hl < Hb) {
        const int h = h0 + hl;
        const float a2 = A[h] * kLog2e;
        float d[SEG], sv[SEG];
        float run = 0.f;
#pragma unroll
        for (int k = 0; k < SEG; ++k) {
            d[k] = tile[hl * LD + sg * SEG + k];
            run += d[k] * a2;
            sv[k] = run;
        }
        float incl = run;
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
            const float up = __shfl_up(incl, off, 16);
            if (sg >= off) incl += up;
        }
        const float excl = incl - run;
        float *o = cs2 + ((size_t)b * H + h) * Tpad + t0 + sg * SEG;
        float *od = dtf + ((size_t)b * H + h) * Tpad + t0 + sg * SEG;
#pragma unroll
        for (int k = 0; k < SEG; k += 4) {
            f32x4 v, w;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[e] = sv[k + e] + excl;
                // log2(0) = -inf, so a zero step (or a padded token) gets cs' = +inf
                // and every factor exp2(x - cs') built from it is exactly 0
                w[e] = v[e] - __builtin_amdgcn_logf(d[k + e]);
            }
            *reinterpret_cast<f32x4 *>(o + k) = v;
            *reinterpret_cast<f32x4 *>(od + k) = w;
        }
    }
}

// ---------------------------------------------------------------------------
// tile_cb: G[b, g, tile] = C_tile B_tile^T (TT x TT, row = query token i,
// column = key token j), with the entries j > i stored as zero (the causal
// mask of the diagonal block), for one band of 64 rows of one tile per work-group,
// wave w owning rows 16w..16w+15 of the band. Only the column blocks the walk
// reads (up to the band's diagonal) are formed. The product is formed
// transposed (B rows as the A operand) so that each lane holds four
// consecutive columns of one row: one 4-element store each.
// ---------------------------------------------------------------------------
template <typename TI, int N, int TT>
__device__ __forceinline__ void tile_cb(int blk, const TI *__restrict__ Bm, const TI *__restrict__ Cm,
                                        TI *__restrict__ Gout, int Tmax, int G, int ntiles, uint32_t g_bytes,
                                        const int *cu, int total, TI *bsh) {
    using Tr = Traits<TI>;
    using frag = typename Tr::frag;
    constexpr int ES = Tr::kBytes;
    constexpr int NK = (N + 31) / 32;
    constexpr int BANDS = TT / 64;
    int x = blk;
    const int band = x % BANDS;
    x /= BANDS;
    const int g = x % G;
    x /= G;
    const int tau = x % ntiles;
    const int b = x / ntiles;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r = lane & 15, kg = lane >> 4;
    const SeqRange sq = seq_range(cu, total, b, Tmax);
    const int T = sq.len;
    const size_t slab = (size_t)T * G * N * ES;
    const size_t sb0 = (size_t)sq.start * G * N * ES;
    const rsrc_t rb = make_rsrc(reinterpret_cast<const char *>(Bm) + sb0, (uint32_t)slab);
    const rsrc_t rc = make_rsrc(reinterpret_cast<const char *>(Cm) + sb0, (uint32_t)slab);
    const rsrc_t rg = make_rsrc(Gout, g_bytes);
    const int t0 = tau * TT;
    const int row = 64 * band + 16 * w + r;  // tile row of this lane's query token (B operand column)
    const int ti = t0 + row;
    frag cq[NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
        const int n0 = kk * 32 + 8 * kg;
        cq[kk] = Tr::load_frag(rc, oob_if(ti >= T || n0 >= N, (uint32_t)(((ti * G + g) * N + n0) * ES)));
    }
    const size_t tile = (((size_t)b * G + g) * ntiles + tau) * (size_t)(TT * TT);
    // With N = 256 the 64 B rows of a column group (32 KB, which each of the
    // four waves reads whole) are staged in LDS once per work-group as
    // 16-byte pieces: it cuts the tile's L2 reads from 160 to 64 KB. For
    // smaller N the waves load their fragments directly (shorter chain).
    constexpr bool kBLds = N >= 256;
    constexpr int BLD = N + 16 / ES;                 // row length, padded by 16 bytes
    constexpr int PPR = N * ES / 16;                 // 16-byte pieces per row
    // bsh: the caller's LDS, 64 * BLD elements
    for (int cgp = 0; cgp <= band; ++cgp) {  // 64-column groups up to the band's diagonal
        frag bk[4][NK];
        if constexpr (kBLds) {
            if (cgp > 0) __syncthreads();    // the previous group's rows are read
            for (int c = threadIdx.x; c < 64 * PPR; c += 256) {
                const int key = c / PPR, pc = c % PPR;
                const int tj = t0 + 64 * cgp + key;
                *reinterpret_cast<u32x4 *>(bsh + key * BLD + pc * (16 / ES)) =
                    buf_ld128(rb, oob_if(tj >= T, (uint32_t)((tj * G + g) * N * ES + pc * 16)));
            }
            __syncthreads();
#pragma unroll
            for (int kk = 0; kk < NK; ++kk)
#pragma unroll
                for (int cb = 0; cb < 4; ++cb)
                    bk[cb][kk] = Tr::lds_frag(bsh + (16 * cb + r) * BLD + kk * 32 + 8 * kg);
        } else {
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) {
                const int n0 = kk * 32 + 8 * kg;
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) {
                    const int tj = t0 + 64 * cgp + 16 * cb + r;
                    bk[cb][kk] = Tr::load_frag(rb, oob_if(tj >= T || n0 >= N,
                                                          (uint32_t)(((tj * G + g) * N + n0) * ES)));
                }
            }
        }
        // acc[cb][i] = G[row][64 cgp + 16 cb + 4 kg + i]
        f32x4 acc[4];
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < NK; ++kk)
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) acc[cb] = Tr::mma(bk[cb][kk], cq[kk], acc[cb]);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            // causal mask: entries above the diagonal (key after query) are stored as 0
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (64 * cgp + 16 * cb + 4 * kg + i > row) acc[cb][i] = 0.f;
            const uint32_t off = (uint32_t)((tile + row * TT + 64 * cgp + 16 * cb + 4 * kg) * ES);
            if constexpr (ES == 2) {
                const bf16x4 v = {(bf16)acc[cb][0], (bf16)acc[cb][1], (bf16)acc[cb][2], (bf16)acc[cb][3]};
                buf_st64(__builtin_bit_cast(u32x2, v), rg, off);
            } else {
                buf_st128(__builtin_bit_cast(u32x4, acc[cb]), rg, off);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// k_prepare: both preparation jobs in one launch (the first work-groups form
// C B^T tiles, the rest the log-decays); they are independent, so their
// latencies overlap instead of adding up.
// ---------------------------------------------------------------------------
template <typename TI, int Q, int N, int TT>
__global__ __launch_bounds__(256) void k_prepare(PrepArgs a) {
    // one LDS buffer for whichever job the work-group runs (the C B^T job
    // stages B rows only for N >= 256), so that more work-groups fit a CU
    constexpr int kCbBytes = N >= 256 ? 64 * (N + 16 / (int)sizeof(TI)) * (int)sizeof(TI) : 0;
    constexpr int kCsBytes = kCumsumHeads * (Q + 1) * 4;
    __shared__ __attribute__((aligned(16))) char lds[kCbBytes > kCsBytes ? kCbBytes : kCsBytes];
    const int blk = blockIdx.x;
    if (blk < a.cb_blocks) {
        tile_cb<TI, N, TT>(blk, (const TI *)a.B, (const TI *)a.C, (TI *)a.Gbuf, a.T, a.G, a.ntiles, a.g_bytes,
                           a.cu, a.total, reinterpret_cast<TI *>(lds));
    } else {
        dt_cumsum<TI, Q>(blk - a.cb_blocks, (const TI *)a.dt, a.A, a.cs2, a.dtf, a.T, a.H, a.nC, a.Tpad, a.cu,
                         a.total, a.dt_bias, a.softplus, reinterpret_cast<float *>(lds));
    }
}

// ---------------------------------------------------------------------------
// k_chunk_walk
//
// One work-group per (batch, head, column slice) walks the sequence in tiles
// of TT tokens (64 or 128), with the PW x N fp32 state in matrix-core
// accumulators. Its 8 wavefronts take two roles that run side by side on
// every SIMD:
//   output waves (0-3), TT/4 rows of the tile each (16-row blocks w and, for
//     128-token tiles, 7 - w, which balances the triangular diagonal work):
//     C rows and the tile's C B^T rows come from global memory one tile
//     ahead; the state at the tile's start comes from an LDS copy; form the
//     state term, the diagonal block and the skip term; store Y through a
//     per-wave LDS staging area.
//   state waves (4-7), a quarter of the state's rows n each: X, B and
//     log-decays come from global memory two tiles ahead (one when a chunk
//     has an odd tile count); update h with this tile, write h as the next
//     tile's LDS copy, and stage the next tile's X, weighted X (factored
//     tiles) and B^T (weighted by w_j in the other tiles) into the other
//     LDS slots.
// One barrier per tile; a second one where LDS cannot hold two copies of
// B^T or of the state.
// The state is accumulated transposed (h^T[n][p]) so that each lane holds
// four consecutive n of one row p: the LDS copy and the final state are
// written four elements at a time.
// ---------------------------------------------------------------------------
// Largest decay over one tile, in base-2 log units (cs2 before the tile minus
// cs2 at its last token), for which the walk factors the diagonal block's
// weights: the weighted X is then at most dt x 2^64, far inside the fp32 and
// bf16 range. Tiles that decay faster take the per-element weights.
constexpr float kFDMax = 64.f;

template <typename TI, int Q, int PW, int N, int TT, bool kConv = false>
struct WalkCfg {
    static constexpr int ES = Traits<TI>::kBytes;
    static constexpr int NTT = TT / 64;              // 16-row blocks per output wave
    static constexpr int NT = Q / TT;                // tiles per chunk
    static constexpr int KB = TT / 32;               // 32-token k-steps per tile
    static constexpr int PB = PW / 16;
    static constexpr int NB = N / 16;
    static constexpr int NTH = 512;                  // 4 output + 4 state wavefronts
    static constexpr int NBW = (NB + 3) / 4;         // state n-blocks per state wave
    static constexpr int NK = (N + 31) / 32;         // 32-wide k-steps over N
    static constexpr int PAD = 16 / ES;
    static constexpr int X_LD = 2 * TT + PAD;        // X: two tile slots
    static constexpr int BT_LD = TT + PAD;
    static constexpr int HS_LD = NK * 32 + PAD;
    static constexpr int YS_LD = PW + PAD;
    static constexpr int TQ = TT / 4;                // token quads per tile
    static constexpr int UX = TQ * (PW / 8);         // staging units: 4 tokens x 8 columns
    static constexpr int UB = TQ * (N / 8);
    static constexpr int RX = (UX + 255) / 256;      // units per state-wave thread
    static constexpr int RB = (UB + 255) / 256;
    static constexpr bool kHSReg = PB * NK * ES <= 32;  // state fragments held in registers
    static constexpr int XT_OFF = 0;
    static constexpr int X_BYTES = PW * X_LD * ES;
    // walks without the input convolution keep a second, weighted X copy
    // (two slots, the layout of X) for the factored diagonal block, up to
    // N = 128: with N = 256 the state waves, which stage it, are the busier
    // role and the per-element form was measured faster (walk 356 vs 383 us
    // on the 16K-token shape)
    static constexpr bool kXW = !kConv && N <= 128;
    static constexpr int XW_OFF = XT_OFF + X_BYTES;
    static constexpr int YS_OFF = XW_OFF + (kXW ? X_BYTES : 0);
    static constexpr int YS_BYTES = TT * YS_LD * ES;
    static constexpr int CS_OFF = YS_OFF + YS_BYTES;  // 2 x (cs2[Q], cs'[Q]) fp32
    static constexpr int CS_BYTES = 2 * 2 * Q * 4;
    static constexpr int HS_OFF = CS_OFF + CS_BYTES;
    static constexpr int HS_BYTES = PW * HS_LD * ES;
    static constexpr int BT_BYTES = N * BT_LD * ES;
    // the fused input convolution's taps and bias for this slice's columns (fp32)
    static constexpr int CW_BYTES = kConv ? PW * 5 * 4 : 0;
    static constexpr int BASE = HS_OFF + HS_BYTES + BT_BYTES + CW_BYTES;
    static constexpr bool kBT2 = BASE + BT_BYTES <= 160 * 1024;             // double B^T
    static constexpr bool kHS2 = BASE + (kBT2 ? BT_BYTES : 0) + HS_BYTES <= 160 * 1024;
    static constexpr int BT_OFF = HS_OFF + (kHS2 ? 2 : 1) * HS_BYTES;
    static constexpr int CW_OFF = BT_OFF + (kBT2 ? 2 : 1) * BT_BYTES;
    static constexpr int LDS = CW_OFF + CW_BYTES;
    static constexpr bool kFits = LDS <= 160 * 1024 && Q % TT == 0;
    static constexpr bool kMidSync = !kBT2 || !kHS2;
    // loads run two tiles ahead of the staging when a chunk has an even
    // number of tiles (register set of tile t = t % 2, static), else one
    static constexpr int kDepth = (NT % 2 == 0) ? 2 : 1;
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

// kStateOnly: the state waves alone (256 threads), for the first pass of a
// sequence split: each segment's end state from its own entering state.
// kConv: X arrives before the layer's causal convolution (4 taps per
// channel, with bias) and SiLU; the state waves apply both while staging
// each tile, reading the 3 tokens before it as well (zeros before the
// sequence's first token).
template <typename TI, int Q, int PW, int N, int TT, bool kStateOnly, bool kConv>
__global__ __launch_bounds__(kStateOnly ? 256 : 512, 1) void k_chunk_walk(WalkArgs a) {
    using Tr = Traits<TI>;
    using Cfg = WalkCfg<TI, Q, PW, N, TT, kConv>;
    using frag = typename Tr::frag;
    constexpr int ES = Cfg::ES, NT = Cfg::NT, NTT = Cfg::NTT, KB = Cfg::KB, PB = Cfg::PB, NB = Cfg::NB;
    constexpr int NBW = Cfg::NBW, NK = Cfg::NK, TQ = Cfg::TQ;
    constexpr int RX = Cfg::RX, RB = Cfg::RB, UX = Cfg::UX, UB = Cfg::UB;
    constexpr int X_LD = Cfg::X_LD, BT_LD = Cfg::BT_LD, HS_LD = Cfg::HS_LD, YS_LD = Cfg::YS_LD;
    constexpr bool kHSReg = Cfg::kHSReg, kBT2 = Cfg::kBT2, kHS2 = Cfg::kHS2, kMidSync = Cfg::kMidSync;
    __shared__ __attribute__((aligned(16))) char smem[Cfg::LDS];
    TI *XT = reinterpret_cast<TI *>(smem + Cfg::XT_OFF);  // [p][slot*TT + token]
    TI *XW = reinterpret_cast<TI *>(smem + Cfg::XW_OFF);  // weighted X, same layout (kFD)
    TI *YS = reinterpret_cast<TI *>(smem + Cfg::YS_OFF);
    float *CSB = reinterpret_cast<float *>(smem + Cfg::CS_OFF);  // [buf][cs2 Q | cs' Q]
    TI *HSB = reinterpret_cast<TI *>(smem + Cfg::HS_OFF);        // [copy][p][n]
    TI *BTB = reinterpret_cast<TI *>(smem + Cfg::BT_OFF);        // [copy][n][token], weighted
    float *CWL = reinterpret_cast<float *>(smem + Cfg::CW_OFF);  // conv taps [col][4], then bias [col]

    const int H = a.H, G = a.G, T = a.T, nC = a.nC, P = a.P, NS = a.NS;
    const int ntiles = nC * NT;
    // blockIdx -> (b, h, slice of PW columns): consecutive logical indices
    // share an XCD (dispatch goes round-robin over the 8 XCDs), so the slices
    // of a head and the heads of one batch element, which read the same B, C
    // and C B^T, share one L2.
    // logical index = ((b H + h) SL + s) NS + ps, s the sequence segment
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
    // this work-group's chunks, and the state it starts from / ends in
    const SeqRange sq = seq_range(a.cu, a.total, b, T);
    const int nCb = (sq.len + Q - 1) / Q;  // chunks of this element (all nC unless packed)
    const int cb = seg * a.cps, ce = min(cb + a.cps, nCb);
    const int last_tile = max(ce * NT - 1, cb * NT);  // loads past the end reload it
    const size_t bhs = (size_t)bhi;
    // pass 1 (state only) enters every segment but the first with zero; the
    // full walk enters segment s with the scanned state in slot s - 1
    const float *init_mat = (seg == 0) ? (a.init ? a.init + bhs * P * N : nullptr)
                            : kStateOnly ? nullptr
                                         : a.seg + (bhs * (S - 1) * a.segk + seg * a.segk - 1) * P * N;
    float *out_mat = kStateOnly ? a.seg + (bhs * (S - 1) + seg) * P * N
                                : ((seg == S - 1 && a.final_state) ? a.final_state + bhs * P * N : nullptr);

    // factored diagonal block and state update (see kFDMax): the state waves
    // also stage a weighted X copy and stage B^T unweighted
    constexpr bool kFD = !kStateOnly && !kConv && Cfg::kXW;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, scalar
    const bool out_wave = !kStateOnly && wv < 4;
    constexpr int NTH = kStateOnly ? 256 : Cfg::NTH;
    const int w = wv & 3;              // index within the role
    const int st = tid & 255;          // thread index within the role
    const int r = lane & 15, kg = lane >> 4;

    const size_t xslab = (size_t)sq.len * H * P * ES, x0 = (size_t)sq.start * H * P * ES;
    const size_t bslab = (size_t)sq.len * G * N * ES, b0 = (size_t)sq.start * G * N * ES;
    const rsrc_t rx = make_rsrc(reinterpret_cast<const char *>(a.X) + x0, (uint32_t)xslab);
    const rsrc_t ry = make_rsrc(reinterpret_cast<char *>(a.Y) + x0, (uint32_t)xslab);
    const rsrc_t rbm = make_rsrc(reinterpret_cast<const char *>(a.B) + b0, (uint32_t)bslab);
    const rsrc_t rc = make_rsrc(reinterpret_cast<const char *>(a.C) + b0, (uint32_t)bslab);
    const rsrc_t rg = make_rsrc(a.Gbuf, a.g_bytes);
    const float *cs_row = a.cs2 + ((size_t)b * H + h) * a.Tpad;
    const float *cp_row = a.dtf + ((size_t)b * H + h) * a.Tpad;  // cs' = cs2 - log2(dt)
    const float Dh = a.D[h];
    const uint32_t x_tok = (uint32_t)(H * P * ES), b_tok = (uint32_t)(G * N * ES);
    const uint32_t hp0 = (uint32_t)((h * P + p0) * ES);  // this slice's columns within a token row

    // ---- prologue: the log-decays of the first chunk, zero padding of the state copies ----
    for (int k = tid; k < Q; k += NTH) {
        CSB[k] = cs_row[cb * Q + k];
        CSB[Q + k] = cp_row[cb * Q + k];
    }
    if constexpr (kConv) {
        for (int k = tid; k < PW; k += NTH) {
            const int col = h * P + p0 + k;
            *reinterpret_cast<f32x4 *>(CWL + 4 * k) = *reinterpret_cast<const f32x4 *>(a.conv_w + 4 * (size_t)col);
            CWL[4 * PW + k] = a.conv_b ? a.conv_b[col] : 0.f;
        }
        __syncthreads();  // the state waves stage a tile before their first barrier
    }
    if constexpr (N % 32 != 0) {
        constexpr int PADN = NK * 32 - N;
        for (int k = tid; k < (kHS2 ? 2 : 1) * PW * PADN; k += NTH) {
            const int q = k / (PW * PADN), kr = k % (PW * PADN);
            HSB[q * PW * HS_LD + (kr / PADN) * HS_LD + N + kr % PADN] = Tr::from_f32(0.f);
        }
    }

    if (!kStateOnly && out_wave) {
        // ===================== output waves =====================
        // 16-row blocks of the tile: w, and 4 NTT - 1 - w for 128-token tiles
        int rbk[NTT];
#pragma unroll
        for (int j = 0; j < NTT; ++j) rbk[j] = (j == 0) ? w : 4 * NTT - 1 - w;
        uint32_t vc[NTT][NK], vg[NTT][KB];
#pragma unroll
        for (int j = 0; j < NTT; ++j) {
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) {
                const int n0 = kk * 32 + 8 * kg;
                vc[j][kk] = oob_if(n0 >= N, (uint32_t)(16 * rbk[j] + r) * b_tok + (uint32_t)(n0 * ES));
            }
            // C B^T column blocks above the block's diagonal are not needed
#pragma unroll
            for (int k2 = 0; k2 < KB; ++k2)
                vg[j][k2] = oob_if(32 * k2 > 16 * rbk[j] + 15,
                                   (uint32_t)(((16 * rbk[j] + r) * TT + 32 * k2 + 8 * kg) * ES));
        }
        const size_t gbase = ((size_t)b * G + g) * ntiles;
        // C rows and the C B^T rows of the next tile are loaded while this one
        // is computed (C right after its last use, C B^T after the diagonal).
        frag cf[NTT][NK], gd[NTT][KB];
        auto load_c = [&](int tt) __attribute__((always_inline)) {  // C rows of the tile at token tt
            const uint32_t sb = (uint32_t)(tt * G + g) * (uint32_t)(N * ES);
#pragma unroll
            for (int j = 0; j < NTT; ++j)
#pragma unroll
                for (int kk = 0; kk < NK; ++kk) cf[j][kk] = Tr::load_frag_s(rc, vc[j][kk], sb);
        };
        auto load_g = [&](int tau) __attribute__((always_inline)) {  // this wave's rows of the tile's C B^T
            const uint32_t sg = (uint32_t)((gbase + tau) * (size_t)(TT * TT * ES));
#pragma unroll
            for (int j = 0; j < NTT; ++j)
#pragma unroll
                for (int k2 = 0; k2 < KB; ++k2) gd[j][k2] = Tr::load_frag_s(rg, vg[j][k2], sg);
        };
        // same issue order as inside the loop (C rows first), so that the
        // compiler's wait counts at the loop head fit both ways in
        // the gate's z pieces (the 16-byte row pieces this lane stores), loaded
        // a tile ahead like C; without z the resource is empty and they read 0
        constexpr int VPR = PW * ES / 16;           // 16-byte vectors per row
        constexpr int NZ = (16 * VPR + 63) / 64;    // per lane and row block
        const bool gate = a.z != nullptr;
        const rsrc_t rz = make_rsrc(reinterpret_cast<const char *>(a.z) + (gate ? x0 : 0),
                                    gate ? (uint32_t)xslab : 0u);
        u32x4 zq[NTT][NZ];
        uint32_t vz[NZ];
#pragma unroll
        for (int k = 0; k < NZ; ++k) {
            const int v = lane + 64 * k;
            vz[k] = oob_if(v >= 16 * VPR, (uint32_t)(v / VPR) * x_tok + (uint32_t)((v % VPR) * 16));
        }
        auto load_z = [&](int tt) __attribute__((always_inline)) {  // z pieces of the tile at token tt
#pragma unroll
            for (int j = 0; j < NTT; ++j) {
                const uint32_t sz = (uint32_t)(tt + 16 * rbk[j]) * x_tok + hp0;
#pragma unroll
                for (int k = 0; k < NZ; ++k) zq[j][k] = buf_ld128s(rz, vz[k], sz);
            }
        };
        load_c(cb * Q);
        __builtin_amdgcn_sched_barrier(0);
        load_g(cb * NT);
        __builtin_amdgcn_sched_barrier(0);
        load_z(cb * Q);
        frag hsf[kHSReg ? PB : 1][kHSReg ? NK : 1];
        __syncthreads();
        for (int c = cb; c < ce; ++c) {
            const int t0 = c * Q;
            const float *CSL = CSB + ((c - cb) & 1) * 2 * Q;  // cs2 of this chunk
            const float *CPL = CSL + Q;                       // cs' of this chunk
            static_for<NT>([&](auto Ic) __attribute__((always_inline)) {
                constexpr int I = decltype(Ic)::value;
                const int tile0 = I * TT;  // chunk-local
                const int tau = c * NT + I;
                const TI *HSr = HSB + (kHS2 ? (tau & 1) : 0) * PW * HS_LD;
                const TI *XTc = XT + (tau & 1) * TT;
                if constexpr (kHSReg) {
#pragma unroll
                    for (int pb = 0; pb < PB; ++pb)
#pragma unroll
                        for (int kk = 0; kk < NK; ++kk)
                            hsf[pb][kk] = Tr::lds_frag(HSr + (16 * pb + r) * HS_LD + kk * 32 + 8 * kg);
                }
                const float cs_ref = (I > 0) ? CSL[tile0 - 1] : 0.f;
                // state -> output
                f32x4 acc[NTT][PB];
#pragma unroll
                for (int j = 0; j < NTT; ++j)
#pragma unroll
                    for (int pb = 0; pb < PB; ++pb) acc[j][pb] = f32x4{0.f, 0.f, 0.f, 0.f};
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
#pragma unroll
                        for (int j = 0; j < NTT; ++j) acc[j][pb] = Tr::mma(cf[j][kk], hb, acc[j][pb]);
                    }
                }
                // the state copy (and a single B^T copy) may be overwritten
                // from here on
                if constexpr (kMidSync) __syncthreads();
                load_c(min(tau + 1, last_tile) * TT);  // past the end: a harmless reload
                // Diagonal block. Factored tiles split the weight 2^(cs_i - cs'_j) as
                // 2^(cs_i - cs_ref) 2^(cs_ref - cs'_j): the second factor is on the
                // weighted X copy, the first on the whole row after the block (state
                // term included), the mask is already in C B^T, so C B^T goes into the
                // matrix cores as loaded. Other tiles weight C B^T per element and
                // scale the state term before the block. The matrix-core ops and both
                // scalings run on every path (one scaling by 1): only the per-element
                // weighting, which reads no accumulator, sits under the branch.
                const bool fd = kFD && (cs_ref - CSL[tile0 + TT - 1] <= kFDMax);
                float fr[NTT][4];
#pragma unroll
                for (int j = 0; j < NTT; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        fr[j][i] = fast_exp2(CSL[tile0 + 16 * rbk[j] + 4 * kg + i] - cs_ref);
#pragma unroll
                        for (int pb = 0; pb < PB; ++pb) acc[j][pb][i] *= fd ? 1.f : fr[j][i];
                    }
                if (!fd) {
#pragma unroll
                    for (int j = 0; j < NTT; ++j) {
                        const int irow = tile0 + 16 * rbk[j] + r;  // chunk-local token of this lane's A row
                        const float cs_i = CSL[irow];
#pragma unroll
                        for (int k2 = 0; k2 < KB; ++k2) {
                            if (32 * k2 > 16 * rbk[j] + 15) continue;  // wave-uniform: above the diagonal
                            const int j0 = tile0 + 32 * k2 + 8 * kg;
                            const f32x4 cpa = *reinterpret_cast<const f32x4 *>(CPL + j0);
                            const f32x4 cpb = *reinterpret_cast<const f32x4 *>(CPL + j0 + 4);
#pragma unroll
                            for (int e = 0; e < 8; ++e) {
                                const float cpj = e < 4 ? cpa[e] : cpb[e - 4];
                                const float v = Tr::frag_get(gd[j][k2], e) * fast_exp2(cs_i - cpj);
                                Tr::frag_set(gd[j][k2], e, (j0 + e <= irow) ? v : 0.f);
                            }
                        }
                    }
                }
                const TI *XD = (fd ? XW : XT) + (tau & 1) * TT;
#pragma unroll
                for (int j = 0; j < NTT; ++j) {
#pragma unroll
                    for (int k2 = 0; k2 < KB; ++k2) {
                        if (32 * k2 > 16 * rbk[j] + 15) continue;  // wave-uniform: above the diagonal
#pragma unroll
                        for (int pb = 0; pb < PB; ++pb) {
                            const frag xb = Tr::lds_frag(XD + (16 * pb + r) * X_LD + 32 * k2 + 8 * kg);
                            acc[j][pb] = Tr::mma(gd[j][k2], xb, acc[j][pb]);
                        }
                    }
                }
                if constexpr (kFD) {
#pragma unroll
                    for (int j = 0; j < NTT; ++j)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
#pragma unroll
                            for (int pb = 0; pb < PB; ++pb) acc[j][pb][i] *= fd ? fr[j][i] : 1.f;
                }
                load_g(min(tau + 1, last_tile));
                // skip term, staging through this wave's own rows, store
#pragma unroll
                for (int j = 0; j < NTT; ++j) {
#pragma unroll
                    for (int pb = 0; pb < PB; ++pb) {
                        TI xs4[4];
                        lds_load4<TI>(xs4, XTc + (16 * pb + r) * X_LD + 16 * rbk[j] + 4 * kg);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int rl = 16 * rbk[j] + 4 * kg + i;  // tile-local token
                            YS[rl * YS_LD + 16 * pb + r] =
                                Tr::from_f32(acc[j][pb][i] + Dh * Tr::to_f32(xs4[i]));
                        }
                    }
                }
                wave_lds_order();
#pragma unroll
                for (int j = 0; j < NTT; ++j) {
                    const uint32_t sy = (uint32_t)(t0 + tile0 + 16 * rbk[j]) * x_tok + hp0;
#pragma unroll
                    for (int k = 0; k < NZ; ++k) {
                        // lanes past the block's vectors run along (no lane-divergent
                        // branch): clamped row, out-of-range store (dropped)
                        const int v = lane + 64 * k;
                        const bool vin = !(NZ * 64 > 16 * VPR) || v < 16 * VPR;
                        const int rl = min(v / VPR, 15), cv = v % VPR;
                        u32x4 d = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(YS) +
                                                                   (16 * rbk[j] + rl) * YS_LD * ES + cv * 16);
                        if (gate) {  // fused output gate y * silu(z), in fp32
                            if constexpr (ES == 2) {
                                bf16x8 yv = __builtin_bit_cast(bf16x8, d);
                                const bf16x8 zv = __builtin_bit_cast(bf16x8, zq[j][k]);
#pragma unroll
                                for (int e = 0; e < 8; ++e) yv[e] = (bf16)silu_gate((float)yv[e], (float)zv[e]);
                                d = __builtin_bit_cast(u32x4, yv);
                            } else {
                                f32x4 yv = __builtin_bit_cast(f32x4, d);
                                const f32x4 zv = __builtin_bit_cast(f32x4, zq[j][k]);
#pragma unroll
                                for (int e = 0; e < 4; ++e) yv[e] = silu_gate(yv[e], zv[e]);
                                d = __builtin_bit_cast(u32x4, yv);
                            }
                        }
                        buf_st128s(d, ry, oob_if(!vin, (uint32_t)rl * x_tok + (uint32_t)(cv * 16)), sy);
                    }
                }
                load_z(min(tau + 1, last_tile) * TT);
                __syncthreads();
            });
        }
    } else {
        // ===================== state waves =====================
        // staging units are wave-uniform whenever their count is a multiple of 64
        auto x_unit = [&](int k) __attribute__((always_inline)) {
            return (UX % 64 == 0) ? (64 * w + 256 * k < UX) : (st + 256 * k < UX);
        };
        auto b_unit = [&](int k) __attribute__((always_inline)) {
            return (UB % 64 == 0) ? (64 * w + 256 * k < UB) : (st + 256 * k < UB);
        };
        // Every lane issues every load, a lane without a unit at an
        // out-of-range offset (it reads zeros and moves no data), and tiles
        // past the end reload the last one: with no load under a branch, the
        // compiler's wait counts stay exact and loads two tiles ahead stay in
        // flight.
        uint32_t vx[RX], vb[RB];
#pragma unroll
        for (int k = 0; k < RX; ++k) {
            const int u = st + 256 * k;
            vx[k] = oob_if(!x_unit(k), (uint32_t)(4 * (u % TQ)) * x_tok + (uint32_t)(8 * ((u / TQ) % (PW / 8)) * ES));
        }
#pragma unroll
        for (int k = 0; k < RB; ++k) {
            const int u = st + 256 * k;
            vb[k] = oob_if(!b_unit(k), (uint32_t)(4 * (u % TQ)) * b_tok + (uint32_t)(8 * ((u / TQ) % (N / 8)) * ES));
        }
        constexpr int kDepth = Cfg::kDepth;
        frag xr[kDepth][RX][4], br[kDepth][RB][4];
        frag xh[kDepth][RX][kConv ? 3 : 1];  // the 3 tokens before each X unit (conv)
        f32x4 bcp[kDepth][RB];   // cs' of the B unit's 4 tokens
        float xce[kDepth] = {};  // cs2 of the tile's last token
        // (kFD) cs' of the X unit's 4 tokens, and cs2 before the tile: the
        // reference of the weighted X, 0 at a chunk's first tile
        f32x4 xcp[kDepth][kFD ? RX : 1];
        float xcr[kDepth] = {};
        const rsrc_t rcs = make_rsrc(cs_row, (uint32_t)a.Tpad * 4u);
        auto issue_stage = [&](int tt, auto Sc) __attribute__((always_inline)) {  // X, B and log-decays of the tile at token tt
            constexpr int S = decltype(Sc)::value;
            const uint32_t sx = (uint32_t)tt * x_tok + hp0;
            const uint32_t sb = (uint32_t)(tt * G + g) * (uint32_t)(N * ES);
#pragma unroll
            for (int k = 0; k < RX; ++k) {
#pragma unroll
                for (int i = 0; i < 4; ++i) xr[S][k][i] = Tr::load_frag_s(rx, vx[k] + i * x_tok, sx);
                if constexpr (kConv) {
                    const int u = st + 256 * k;
                    const int row0 = tt + 4 * (u % TQ) - 3;  // token of halo row 0
                    const uint32_t col = hp0 + (uint32_t)(8 * ((u / TQ) % (PW / 8)) * ES);
#pragma unroll
                    for (int i = 0; i < 3; ++i)
                        xh[S][k][i] = Tr::load_frag(
                            rx, oob_if(!x_unit(k) || row0 + i < 0, (uint32_t)(row0 + i) * x_tok + col));
                }
            }
            // a vector load: a scalar one would hold up every LDS wait (both
            // count in lgkmcnt) until it returns
            xce[S] = __builtin_bit_cast(float, buf_ld32(rcs, (uint32_t)(tt + TT - 1) * 4u));
            if constexpr (kFD) {
                const float ref = __builtin_bit_cast(float, buf_ld32(rcs, (uint32_t)max(tt - 1, 0) * 4u));
                xcr[S] = (tt % Q == 0) ? 0.f : ref;
#pragma unroll
                for (int k = 0; k < RX; ++k)
                    xcp[S][k] = *reinterpret_cast<const f32x4 *>(cp_row + tt + 4 * ((st + 256 * k) % TQ));
            }
#pragma unroll
            for (int k = 0; k < RB; ++k) {
#pragma unroll
                for (int i = 0; i < 4; ++i) br[S][k][i] = Tr::load_frag_s(rbm, vb[k] + i * b_tok, sb);
                bcp[S][k] = *reinterpret_cast<const f32x4 *>(cp_row + tt + 4 * ((st + 256 * k) % TQ));
            }
        };
        auto stage = [&](auto Sc, int slot) __attribute__((always_inline)) {  // into X slot `slot` and the matching B^T copy
            constexpr int S = decltype(Sc)::value;
            TI *BT = BTB + (kBT2 ? slot : 0) * N * BT_LD;
            // Where the units do not fill whole wavefronts, every lane runs the
            // staging (no lane-divergent branch) and lanes without a unit write
            // into the rows' padding columns, which nothing reads.
#pragma unroll
            for (int k = 0; k < RX; ++k)
                if (UX % 64 != 0 || x_unit(k)) {
                    const int u = st + 256 * k;
                    const int tq = u % TQ, po = (u / TQ) % (PW / 8);
                    const int xcol = x_unit(k) ? slot * TT + 4 * tq : 2 * TT;  // padding: 2 TT .. 2 TT + PAD - 1
                    if constexpr (kConv) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const int c = 8 * po + e;
                            const f32x4 wv = *reinterpret_cast<const f32x4 *>(CWL + 4 * c);
                            const float bv = CWL[4 * PW + c];
                            float xv[7];  // tokens 4 tq - 3 .. 4 tq + 3 of this column
#pragma unroll
                            for (int i = 0; i < 3; ++i) xv[i] = Tr::frag_get(xh[S][k][i], e);
#pragma unroll
                            for (int i = 0; i < 4; ++i) xv[3 + i] = Tr::frag_get(xr[S][k][i], e);
                            float yv[4];
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const float v = bv + wv[0] * xv[i] + wv[1] * xv[i + 1] + wv[2] * xv[i + 2] +
                                                wv[3] * xv[i + 3];
                                yv[i] = v * __builtin_amdgcn_rcpf(1.f + fast_exp2(-kLog2e * v));
                            }
                            lds_store4<TI>(XT + c * X_LD + xcol, Tr::from_f32(yv[0]), Tr::from_f32(yv[1]),
                                           Tr::from_f32(yv[2]), Tr::from_f32(yv[3]));
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            lds_store4<TI>(XT + (8 * po + e) * X_LD + xcol, xr[S][k][0][e], xr[S][k][1][e],
                                           xr[S][k][2][e], xr[S][k][3][e]);
                        if constexpr (kFD) {
                            // x_j 2^(cs_ref - cs'_j) = dt_j x_j 2^(cs_ref - cs_j), at most
                            // dt_j x_j 2^kFDMax in the tiles that use it
                            if (xcr[S] - xce[S] <= kFDMax) {
                                float cw[4];
#pragma unroll
                                for (int i = 0; i < 4; ++i) cw[i] = fast_exp2(xcr[S] - xcp[S][k][i]);
#pragma unroll
                                for (int e = 0; e < 8; ++e)
                                    lds_store4<TI>(XW + (8 * po + e) * X_LD + xcol,
                                                   Tr::from_f32(Tr::frag_get(xr[S][k][0], e) * cw[0]),
                                                   Tr::from_f32(Tr::frag_get(xr[S][k][1], e) * cw[1]),
                                                   Tr::from_f32(Tr::frag_get(xr[S][k][2], e) * cw[2]),
                                                   Tr::from_f32(Tr::frag_get(xr[S][k][3], e) * cw[3]));
                            }
                        }
                    }
                }
            // factored tiles take B^T as it is (their weights are on X)
            const bool braw = kFD && (xcr[S] - xce[S] <= kFDMax);
            // (the same padding rule as for X: B^T rows have TT + PAD columns)
#pragma unroll
            for (int k = 0; k < RB; ++k)
                if ((UB % 64 != 0 || b_unit(k)) && braw) {
                    const int u = st + 256 * k;
                    const int tq = u % TQ, no = (u / TQ) % (N / 8);
                    const int bcol = b_unit(k) ? 4 * tq : TT;
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        lds_store4<TI>(BT + (8 * no + e) * BT_LD + bcol, br[S][k][0][e], br[S][k][1][e],
                                       br[S][k][2][e], br[S][k][3][e]);
                } else if (UB % 64 != 0 || b_unit(k)) {
                    const int u = st + 256 * k;
                    const int tq = u % TQ, no = (u / TQ) % (N / 8);
                    const int bcol = b_unit(k) ? 4 * tq : TT;
                    // the state update's weights w_j = exp2(cs_e - cs'_j) <= dt_j
                    float sc[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) sc[i] = fast_exp2(xce[S] - bcp[S][k][i]);
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        lds_store4<TI>(BT + (8 * no + e) * BT_LD + bcol,
                                       Tr::from_f32(Tr::frag_get(br[S][k][0], e) * sc[0]),
                                       Tr::from_f32(Tr::frag_get(br[S][k][1], e) * sc[1]),
                                       Tr::from_f32(Tr::frag_get(br[S][k][2], e) * sc[2]),
                                       Tr::from_f32(Tr::frag_get(br[S][k][3], e) * sc[3]));
                }
        };
        // transposed state: hacc[pb][j][i] = h[p = 16pb + r][n = 16(w + 4j) + 4kg + i]
        f32x4 hacc[PB][NBW];
        auto write_hs = [&](TI *HSw) __attribute__((always_inline)) {
#pragma unroll
            for (int pb = 0; pb < PB; ++pb)
#pragma unroll
                for (int j = 0; j < NBW; ++j) {
                    const int nb = w + 4 * j;
                    if (nb < NB)
                        lds_store4<TI>(HSw + (16 * pb + r) * HS_LD + 16 * nb + 4 * kg,
                                       Tr::from_f32(hacc[pb][j][0]), Tr::from_f32(hacc[pb][j][1]),
                                       Tr::from_f32(hacc[pb][j][2]), Tr::from_f32(hacc[pb][j][3]));
                }
        };
#pragma unroll
        for (int pb = 0; pb < PB; ++pb)
#pragma unroll
            for (int j = 0; j < NBW; ++j) {
                const int nb = w + 4 * j;
                f32x4 v = {0.f, 0.f, 0.f, 0.f};
                if (init_mat && nb < NB)
                    v = *reinterpret_cast<const f32x4 *>(init_mat + (p0 + 16 * pb + r) * N + 16 * nb + 4 * kg);
                hacc[pb][j] = v;
            }
        const int tile_b = cb * NT;  // first tile
        if constexpr (!kStateOnly) write_hs(HSB + (kHS2 ? (tile_b & 1) : 0) * PW * HS_LD);
        issue_stage(tile_b * TT, std::integral_constant<int, 0>{});
        stage(std::integral_constant<int, 0>{}, tile_b & 1);
        if constexpr (kDepth == 2) issue_stage(min(tile_b + 1, last_tile) * TT, std::integral_constant<int, 1>{});
        __syncthreads();
        float csn = 0.f, cpn = 0.f;
        for (int c = cb; c < ce; ++c) {
            const int t0 = c * Q;
            const float *CSL = CSB + ((c - cb) & 1) * 2 * Q;  // cs2 of this chunk
            static_for<NT>([&](auto Ic) __attribute__((always_inline)) {
                constexpr int I = decltype(Ic)::value;
                const int tile0 = I * TT;
                const int tau = c * NT + I;
                const int slot = tau & 1;
                if constexpr (I == 0) {
                    // the next chunk's log-decays (Q <= 256: one per thread),
                    // issued first and written at the chunk's last tile
                    const int kn = (c + 1 < ce ? t0 + Q : t0) + min(st, Q - 1);
                    csn = cs_row[kn];
                    cpn = cp_row[kn];
                }
                issue_stage(min(tau + kDepth, last_tile) * TT,
                            std::integral_constant<int, kDepth == 2 ? (I & 1) : 0>{});
                const TI *BT = BTB + (kBT2 ? slot : 0) * N * BT_LD;
                const float cs_ref = (I > 0) ? CSL[tile0 - 1] : 0.f;
                const float dec = fast_exp2(CSL[tile0 + TT - 1] - cs_ref);
                // factored tile: h_e = dec (h + B^T Xw); else h_e = dec h + Bw^T X.
                // Both scalings always run (one of them by 1): a branch next to the
                // matrix-core ops left the accumulators read too early on one path.
                const bool fd = kFD && (cs_ref - CSL[tile0 + TT - 1] <= kFDMax);
                const float pre = fd ? 1.f : dec, post = fd ? dec : 1.f;
#pragma unroll
                for (int pb = 0; pb < PB; ++pb)
#pragma unroll
                    for (int j = 0; j < NBW; ++j) hacc[pb][j] *= pre;
                const TI *XS = (fd ? XW : XT) + slot * TT;
#pragma unroll
                for (int k2 = 0; k2 < KB; ++k2) {
                    frag xa[PB];
#pragma unroll
                    for (int pb = 0; pb < PB; ++pb)
                        xa[pb] = Tr::lds_frag(XS + (16 * pb + r) * X_LD + 32 * k2 + 8 * kg);
#pragma unroll
                    for (int j = 0; j < NBW; ++j) {
                        const int nb = w + 4 * j;
                        if (nb < NB) {
                            const frag bb = Tr::lds_frag(BT + (16 * nb + r) * BT_LD + 32 * k2 + 8 * kg);
#pragma unroll
                            for (int pb = 0; pb < PB; ++pb) hacc[pb][j] = Tr::mma(bb, xa[pb], hacc[pb][j]);
                        }
                    }
                }
                if constexpr (kFD) {
#pragma unroll
                    for (int pb = 0; pb < PB; ++pb)
#pragma unroll
                        for (int j = 0; j < NBW; ++j) hacc[pb][j] *= post;
                }
                // a single B^T copy, or a single state copy, is read up to here
                if constexpr (kMidSync) __syncthreads();
                if constexpr (I == NT - 1) {
                    if (c + 1 < ce && st < Q) {
                        float *CSN = CSB + ((c + 1 - cb) & 1) * 2 * Q;
                        CSN[st] = csn;
                        CSN[Q + st] = cpn;
                    }
                }
                if constexpr (!kStateOnly) write_hs(HSB + (kHS2 ? ((tau + 1) & 1) : 0) * PW * HS_LD);
                // (after the last tile this stages a reload into slots nobody reads)
                stage(std::integral_constant<int, kDepth == 2 ? ((I + 1) & 1) : 0>{}, (tau + 1) & 1);
                __syncthreads();
            });
        }
        if (out_mat) {
#pragma unroll
            for (int pb = 0; pb < PB; ++pb)
#pragma unroll
                for (int j = 0; j < NBW; ++j) {
                    const int nb = w + 4 * j;
                    if (nb < NB)
                        *reinterpret_cast<f32x4 *>(out_mat + (p0 + 16 * pb + r) * N + 16 * nb + 4 * kg) =
                            hacc[pb][j];
                }
        }
    }
}

// ---------------------------------------------------------------------------
// k_seg_scan: between the two passes of a sequence split. Pass 1 left, for
// each segment s < S - 1, the state at its end when entered with zero (with
// the caller's initial state for s = 0). The state entering segment s + 1 is
//   E_0 = end_0,   E_s = 2^{D_s} E_{s-1} + end_s,
// D_s the segment's total log-decay (the sum of its chunks' last cs2), i.e.
// the state passing of the chunked method at segment granularity. Rewritten in
// place: slot s ends up holding the state entering segment s + 1. One thread
// per 4 state elements. (Where the pre-pass halves the walk's segments, the
// segments here are those halves.)
// ---------------------------------------------------------------------------
static __global__ __launch_bounds__(256) void k_seg_scan(float *__restrict__ seg, const float *__restrict__ cs2,
                                                  int64_t bh_count, int PN, int S, int cps, int nC, int Q,
                                                  int Tpad) {
    const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // f32x4 index
    const int per = PN / 4;
    if (v >= bh_count * per) return;
    const int64_t bhi = v / per;
    const int e = (int)(v - bhi * per);
    const float *cs = cs2 + bhi * Tpad;
    f32x4 *base = reinterpret_cast<f32x4 *>(seg + bhi * (int64_t)(S - 1) * PN) + e;
    const int64_t stride = PN / 4;
    f32x4 E = base[0];
    // four segments at a time: their states and total decays are loaded
    // together, then chained (past the last segment a repeat, not stored)
    for (int s0 = 1; s0 < S - 1; s0 += 4) {
        f32x4 sl[4];
        float D[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int s = min(s0 + k, S - 2);
            sl[k] = base[(int64_t)s * stride];
            float d = 0.f;
#pragma unroll 8
            for (int c = s * cps; c < min((s + 1) * cps, nC); ++c) d += cs[c * Q + Q - 1];
            D[k] = d;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (s0 + k < S - 1) {
                E = fast_exp2(D[k]) * E + sl[k];
                base[(int64_t)(s0 + k) * stride] = E;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// host side: the plan (column slices, tile size) and the launches
// ---------------------------------------------------------------------------
template <typename TI, int Q, int PW, int N, int TT, bool kConv = false>
static constexpr bool fits() {
    if constexpr (Q % TT != 0) {
        return false;
    } else {
        return WalkCfg<TI, Q, PW, N, TT, kConv>::kFits;
    }
}

// The tile: 64 tokens. (128-token tiles, which halve the per-tile barriers,
// were measured slower on every benchmark shape: the cost per tile grows with
// the work, not with the number of tiles.)
template <typename TI, int Q, int PW, int N>
static int tile_of() {
    if (fits<TI, Q, PW, N, 64>()) return 64;
    return 0;
}

template <typename TI, int Q, int PW>
static int tile_n(int64_t N) {
    switch (N) {
        case 16: return tile_of<TI, Q, PW, 16>();
        case 32: return tile_of<TI, Q, PW, 32>();
        case 64: return tile_of<TI, Q, PW, 64>();
        case 128: return tile_of<TI, Q, PW, 128>();
        case 256: return tile_of<TI, Q, PW, 256>();
        default: return 0;
    }
}

template <typename TI, int Q>
static int tile_p(int64_t PW, int64_t N) {
    switch (PW) {
        case 16: return tile_n<TI, Q, 16>(N);
        case 32: return tile_n<TI, Q, 32>(N);
        case 64: return tile_n<TI, Q, 64>(N);
        case 128: return tile_n<TI, Q, 128>(N);
        default: return 0;
    }
}

template <typename TI>
static int tile_q(int64_t Q, int64_t PW, int64_t N) {
    switch (Q) {
        case 64: return tile_p<TI, 64>(PW, N);
        case 128: return tile_p<TI, 128>(PW, N);
        case 256: return tile_p<TI, 256>(PW, N);
        default: return 0;
    }
}

// Work-groups per head, each taking P / ns of the head's columns (and the
// matching rows of the state). One work-group fills a CU, so heads are split
// only while there are fewer walks than CUs; a slice keeps at least 16
// columns. Splitting further was measured slower: the slices of a head each
// stage the whole B tile and build the whole masked C B^T block.
constexpr int kCUs = 256;

#ifndef SSD_CONV_TU
int fwd_plan(ssd_dtype dt, int64_t batch, int64_t H, int64_t P, int64_t N, int64_t Q, int64_t nC,
             bool segments, WalkPlan *plan) {
    const int64_t walks = batch * H;
    // Long sequences with few heads: split the sequence into S segments (at
    // least two chunks each) so that more, shorter walks fill the CUs; then
    // split heads' columns while walks are still fewer than CUs.
    int S = 1;
    while (segments && walks * 2 * S <= kCUs && nC / (2 * S) >= 2) S *= 2;
    while (S > 1 && (S - 1) * ((nC + S - 1) / S) >= nC) S /= 2;  // no empty segment
    int ns = 1;
    while (ns < 4 && walks * S * 2 * ns <= kCUs && P % (2 * ns) == 0 && P / (2 * ns) >= 16) ns *= 2;
    int tt = dt == SSD_BF16 ? tile_q<bf16>(Q, P / ns, N) : tile_q<float>(Q, P / ns, N);
    // the plan must not depend on the batch for a shape to be supported: the
    // unsplit head has to fit too
    const int tt1 = dt == SSD_BF16 ? tile_q<bf16>(Q, P, N) : tile_q<float>(Q, P, N);
    if (!tt || !tt1) return -1;
    plan->ns = ns;
    plan->tt = tt;
    plan->S = S;
    plan->cps = (int)((nC + S - 1) / S);
    // The end-state pre-pass takes each segment but the last as two halves
    // where its chunks split evenly: twice the work-groups, each with half the
    // tiles, for a pre-pass whose time is the length of its walks.
    plan->segk = (S > 1 && plan->cps % 2 == 0) ? 2 : 1;
    return 0;
}

#endif  // SSD_CONV_TU

template <typename TI, int Q, int N, int TT>
static ssd_status run_prepare(const FwdArgs &f, hipStream_t s) {
    PrepArgs a;
    a.dt = f.dt; a.B = f.B; a.C = f.C; a.A = f.A; a.Gbuf = f.Gbuf; a.cs2 = f.cs2; a.dtf = f.dtf;
    a.T = (int)f.T; a.H = (int)f.H; a.G = (int)f.G; a.nC = (int)f.nC; a.Tpad = (int)f.Tpad;
    a.cu = f.cu; a.total = (int)f.total;
    a.dt_bias = f.dt_bias; a.softplus = f.softplus;
    a.ntiles = (int)(f.Tpad / TT);
    a.g_bytes = (uint32_t)f.g_bytes;
    // the backward reads no C B^T tiles
    a.cb_blocks = f.no_g ? 0 : (int)(f.batch * a.ntiles * f.G * (TT / 64));
    const int64_t hblocks = (f.H + kCumsumHeads - 1) / kCumsumHeads;
    const int64_t blocks = a.cb_blocks + f.batch * hblocks * f.nC;
    return launch(k_prepare<TI, Q, N, TT>, dim3((unsigned)blocks), dim3(256), s, a) == hipSuccess
               ? SSD_OK
               : SSD_ERR_HIP;
}

// A split sequence (S > 1) takes three launches: the state-only walk of
// segments 0..S-2, the scan of their end states, the full walk of all S
// segments each from its entering state.
template <typename TI, int Q, int PW, int N, int TT, bool kConv>
static ssd_status run_walk_c(const FwdArgs &f, hipStream_t s) {
    if constexpr (!fits<TI, Q, PW, N, TT, kConv>()) {
        return SSD_ERR_UNSUPPORTED;
    } else {
        WalkArgs wa;
        wa.X = f.X; wa.B = f.B; wa.C = f.C; wa.Y = f.Y; wa.Gbuf = f.Gbuf;
        wa.cs2 = f.cs2; wa.dtf = f.dtf; wa.D = f.D; wa.init = f.init; wa.final_state = f.final_state;
        wa.batch = (int)f.batch; wa.T = (int)f.T; wa.H = (int)f.H; wa.G = (int)f.G; wa.nC = (int)f.nC;
        wa.Tpad = (int)f.Tpad; wa.P = (int)f.P; wa.NS = f.ns; wa.g_bytes = (uint32_t)f.g_bytes;
        wa.S = f.S; wa.cps = f.cps; wa.seg = f.seg;
        wa.segk = kConv ? 1 : f.segk;
        wa.cu = f.cu; wa.total = (int)f.total; wa.z = f.z;
        wa.conv_w = f.conv_w; wa.conv_b = f.conv_b;
        const int64_t heads = f.batch * f.H * f.ns;
        if (f.S > 1) {
            // the pre-pass and the scan run over wa.segk sub-segments per
            // segment (all segments but the last): SP - 1 of them, cpp chunks each
            const int SP = (f.S - 1) * wa.segk + 1, cpp = f.cps / wa.segk;
            wa.SL = f.S - 1;
            if constexpr (kConv) {
                // the segments' end states need the convolved X: the state-only walk
                if (launch(k_chunk_walk<TI, Q, PW, N, TT, true, kConv>, dim3((unsigned)(heads * wa.SL)), dim3(256),
                           s, wa) != hipSuccess)
                    return SSD_ERR_HIP;
            } else {
                FwdArgs fs = f;
                fs.S = SP;
                fs.cps = cpp;
                const ssd_status st = launch_seg_states(fs, s);
                if (st != SSD_OK) return st;
            }
            const int64_t n4 = f.batch * f.H * f.P * f.N / 4;
            if (SP > 2 && launch(k_seg_scan, dim3((unsigned)((n4 + 255) / 256)), dim3(256), s, f.seg,
                                 (const float *)f.cs2, f.batch * f.H, (int)(f.P * f.N), SP, cpp, (int)f.nC,
                                 (int)f.Q, (int)f.Tpad) != hipSuccess)
                return SSD_ERR_HIP;
        }
        if (walk_rs_supported(f)) return launch_walk_rs(f, s);
        wa.SL = f.S;
        return launch(k_chunk_walk<TI, Q, PW, N, TT, false, kConv>, dim3((unsigned)(heads * f.S)), dim3(512), s,
                      wa) == hipSuccess
                   ? SSD_OK
                   : SSD_ERR_HIP;
    }
}

template <typename TI, int Q, int PW, int N, bool kConv>
static ssd_status walk_t(const FwdArgs &f, hipStream_t s) {
    switch (f.tt) {
        case 64: return run_walk_c<TI, Q, PW, N, 64, kConv>(f, s);
        default: return SSD_ERR_UNSUPPORTED;
    }
}

template <typename TI, int Q, int PW, bool kConv>
static ssd_status walk_n(const FwdArgs &f, hipStream_t s) {
    switch (f.N) {
        case 16: return walk_t<TI, Q, PW, 16, kConv>(f, s);
        case 32: return walk_t<TI, Q, PW, 32, kConv>(f, s);
        case 64: return walk_t<TI, Q, PW, 64, kConv>(f, s);
        case 128: return walk_t<TI, Q, PW, 128, kConv>(f, s);
        case 256: return walk_t<TI, Q, PW, 256, kConv>(f, s);
        default: return SSD_ERR_UNSUPPORTED;
    }
}

template <typename TI, int Q, bool kConv>
static ssd_status walk_p(const FwdArgs &f, hipStream_t s) {
    switch (f.P / f.ns) {
        case 16: return walk_n<TI, Q, 16, kConv>(f, s);
        case 32: return walk_n<TI, Q, 32, kConv>(f, s);
        case 64: return walk_n<TI, Q, 64, kConv>(f, s);
        case 128: return walk_n<TI, Q, 128, kConv>(f, s);
        default: return SSD_ERR_UNSUPPORTED;
    }
}

template <typename TI, bool kConv>
static ssd_status walk_q(const FwdArgs &f, hipStream_t s) {
    switch (f.Q) {
        case 64: return walk_p<TI, 64, kConv>(f, s);
        case 128: return walk_p<TI, 128, kConv>(f, s);
        case 256: return walk_p<TI, 256, kConv>(f, s);
        default: return SSD_ERR_UNSUPPORTED;
    }
}

#ifdef SSD_CONV_TU
// This translation unit (ssd_walk_conv.hip) holds only the walks with the
// fused input convolution, so that they compile in parallel with the rest.
ssd_status launch_walk_conv(const FwdArgs &f, hipStream_t s) {
    return f.dtype == SSD_BF16 ? walk_q<bf16, true>(f, s) : walk_q<float, true>(f, s);
}
#else

template <typename TI, int Q, int N>
static ssd_status prepare_t(const FwdArgs &f, hipStream_t s) {
    switch (f.tt) {
        case 64: return run_prepare<TI, Q, N, 64>(f, s);
        default: return SSD_ERR_UNSUPPORTED;
    }
}

template <typename TI, int Q>
static ssd_status prepare_n(const FwdArgs &f, hipStream_t s) {
    switch (f.N) {
        case 16: return prepare_t<TI, Q, 16>(f, s);
        case 32: return prepare_t<TI, Q, 32>(f, s);
        case 64: return prepare_t<TI, Q, 64>(f, s);
        case 128: return prepare_t<TI, Q, 128>(f, s);
        case 256: return prepare_t<TI, Q, 256>(f, s);
        default: return SSD_ERR_UNSUPPORTED;
    }
}

template <typename TI>
static ssd_status prepare_q(const FwdArgs &f, hipStream_t s) {
    switch (f.Q) {
        case 64: return prepare_n<TI, 64>(f, s);
        case 128: return prepare_n<TI, 128>(f, s);
        case 256: return prepare_n<TI, 256>(f, s);
        default: return SSD_ERR_UNSUPPORTED;
    }
}

template <typename TI, int Q, int PW>
static bool conv_fits_n(int64_t N) {
    switch (N) {
        case 16: return fits<TI, Q, PW, 16, 64, true>();
        case 32: return fits<TI, Q, PW, 32, 64, true>();
        case 64: return fits<TI, Q, PW, 64, 64, true>();
        case 128: return fits<TI, Q, PW, 128, 64, true>();
        case 256: return fits<TI, Q, PW, 256, 64, true>();
        default: return false;
    }
}

template <typename TI, int Q>
static bool conv_fits_q(int64_t PW, int64_t N) {
    switch (PW) {
        case 16: return conv_fits_n<TI, Q, 16>(N);
        case 32: return conv_fits_n<TI, Q, 32>(N);
        case 64: return conv_fits_n<TI, Q, 64>(N);
        case 128: return conv_fits_n<TI, Q, 128>(N);
        default: return false;
    }
}

bool walk_conv_fits(ssd_dtype dt, int64_t Q, int64_t PW, int64_t N) {
    auto q = [&](auto T0) -> bool {
        using TI = decltype(T0);
        switch (Q) {
            case 64: return conv_fits_q<TI, 64>(PW, N);
            case 128: return conv_fits_q<TI, 128>(PW, N);
            case 256: return conv_fits_q<TI, 256>(PW, N);
            default: return false;
        }
    };
    return dt == SSD_BF16 ? q(bf16{}) : q(float{});
}

ssd_status launch_prepare(const FwdArgs &f, hipStream_t s) {
    return f.dtype == SSD_BF16 ? prepare_q<bf16>(f, s) : prepare_q<float>(f, s);
}

ssd_status launch_walk(const FwdArgs &f, hipStream_t s) {
    if (f.conv_w) return launch_walk_conv(f, s);
    return f.dtype == SSD_BF16 ? walk_q<bf16, false>(f, s) : walk_q<float, false>(f, s);
}
#endif  // SSD_CONV_TU

}  // namespace ssd
