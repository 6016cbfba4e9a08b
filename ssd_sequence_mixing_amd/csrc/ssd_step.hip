// One recurrent decode step for gfx950: the O(1)-per-token inference form of
// the SSM ("Transformer vs Mamba/SSM: the next step of the architecture",
// why it matters: each step only updates a fixed-size state).
//
//   a = exp(dt[b,h] A[h]);  s[p,n] <- a s[p,n] + dt x[p] B[g,n];
//   y[p] = sum_n s[p,n] C[g,n] + D[h] x[p]
//
// optionally with the layer's prologue and epilogue fused in: dt =
// softplus(dt + dt_bias[h]), the input x <- SiLU(b + w . [x_{t-3}, x_{t-2},
// x_{t-1}, x_t]) of the layer's causal convolution (the 3 earlier raw inputs
// kept in a rolling conv state, shifted by this step) and y <- y * silu(z[p]).
//
// The state is the only large operand: the kernel streams it once in and
// once out with 16-byte non-temporal accesses (it is not reused by this
// step, so it should not displace anything in the caches). A row of N fp32
// values is split over N/4 lanes; the dot product with C is reduced across
// those lanes with cross-lane shuffles. Each work-group covers RPB rows of
// one (batch, head), so the head's scalars (dt, A, D, group) are uniform
// and every lane keeps two rows' loads in flight.
#include "ssd_common.h"
#include "ssd_internal.h"

namespace ssd {

constexpr int kStepThreads = 256;
constexpr int kStepUnroll = 2;

template <typename TI, int N>
struct StepShape {
    static constexpr int TPR = N / 4;                 // lanes per state row
    static constexpr int RPW = 64 / TPR;              // rows per wavefront per pass
    static constexpr int RPB = (kStepThreads / 64) * RPW * kStepUnroll;  // rows per work-group
};

template <typename TI, int N>
__global__ __launch_bounds__(kStepThreads) void k_step(StepArgs a, int pblocks) {
    using Tr = Traits<TI>;
    using S = StepShape<TI, N>;
    constexpr int TPR = S::TPR, RPW = S::RPW, RPB = S::RPB;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int sub = lane / TPR, c4 = lane % TPR;
    const int P = (int)a.P, H = (int)a.H, G = (int)a.G;
    // work-group -> (batch*head, block of rows); all of it scalar
    const int64_t bh = blockIdx.x / pblocks;
    const int pb = blockIdx.x - (int)(bh * pblocks);
    const int64_t bb = bh / H;
    const int h = (int)(bh - bb * H);
    const int g = (h * G) / H;
    float dtv = Tr::to_f32(reinterpret_cast<const TI *>(a.dt)[bh]);
    if (a.dt_bias || a.softplus) dtv = dt_prologue(dtv, a.dt_bias ? a.dt_bias[h] : 0.f, a.softplus);
    const float dec = fast_exp2(dtv * a.A[h] * kLog2e);
    const float Dh = a.D[h];
    float *srow = a.state + bh * P * N;

    int p[kStepUnroll];
    f32x4 s[kStepUnroll];
#pragma unroll
    for (int u = 0; u < kStepUnroll; ++u) {
        p[u] = pb * RPB + (u * (kStepThreads / 64) + w) * RPW + sub;
        s[u] = (p[u] < P)
                   ? __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(srow + (int64_t)p[u] * N) + c4)
                   : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const TI *bp = reinterpret_cast<const TI *>(a.B) + (bb * G + g) * N + 4 * c4;
    const TI *cp = reinterpret_cast<const TI *>(a.C) + (bb * G + g) * N + 4 * c4;
    float bv[4], cv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        bv[e] = Tr::to_f32(bp[e]);
        cv[e] = Tr::to_f32(cp[e]);
    }
#pragma unroll
    for (int u = 0; u < kStepUnroll; ++u) {
        const bool ok = p[u] < P;
        float xv = ok ? Tr::to_f32(reinterpret_cast<const TI *>(a.x)[bh * P + p[u]]) : 0.f;
        if (a.conv_w && ok) {
            // channel c = h P + p: x' = SiLU(b + w0 s0 + w1 s1 + w2 s2 + w3 x), in fp32 and
            // rounded to the storage type (as the forward stages it); the conv
            // state then holds (s1, s2, x). Every lane of the row reads it, one writes it,
            // after the reads have been used.
            const int64_t ch = (int64_t)h * P + p[u];
            TI *cst = reinterpret_cast<TI *>(a.conv_state) + (bb * H * P + ch) * 3;
            const TI s1 = cst[1], s2 = cst[2];
            const float s0 = Tr::to_f32(cst[0]);
            const f32x4 wv = *reinterpret_cast<const f32x4 *>(a.conv_w + 4 * ch);
            const float v = (a.conv_b ? a.conv_b[ch] : 0.f) + wv[0] * s0 + wv[1] * Tr::to_f32(s1) +
                            wv[2] * Tr::to_f32(s2) + wv[3] * xv;
            const float xa = Tr::to_f32(Tr::from_f32(v / (1.f + expf(-v))));
            if (c4 == 0) {
                cst[0] = s1;
                cst[1] = s2;
                cst[2] = Tr::from_f32(xv);
            }
            xv = xa;
        }
        const float uin = dtv * xv;
        f32x4 sn;
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sn[e] = dec * s[u][e] + uin * bv[e];
            part += sn[e] * cv[e];
        }
        if (ok) __builtin_nontemporal_store(sn, reinterpret_cast<f32x4 *>(srow + (int64_t)p[u] * N) + c4);
#pragma unroll
        for (int off = TPR / 2; off > 0; off >>= 1) part += __shfl_xor(part, off, 64);
        if (ok && c4 == 0) {
            float yv = part + Dh * xv;
            if (a.z) yv = silu_gate(yv, Tr::to_f32(reinterpret_cast<const TI *>(a.z)[bh * P + p[u]]));
            reinterpret_cast<TI *>(a.y)[bh * P + p[u]] = Tr::from_f32(yv);
        }
    }
}

template <typename TI, int N>
static ssd_status run_step(const StepArgs &a, hipStream_t s) {
    constexpr int RPB = StepShape<TI, N>::RPB;
    const int pblocks = (int)((a.P + RPB - 1) / RPB);
    const int64_t blocks = a.batch * a.H * pblocks;
    return launch(k_step<TI, N>, dim3((unsigned)blocks), dim3(kStepThreads), s, a, pblocks) ==
                   hipSuccess
               ? SSD_OK
               : SSD_ERR_HIP;
}

template <typename TI>
static ssd_status step_n(const StepArgs &a, hipStream_t s) {
    switch (a.N) {
        case 4: return run_step<TI, 4>(a, s);
        case 8: return run_step<TI, 8>(a, s);
        case 16: return run_step<TI, 16>(a, s);
        case 32: return run_step<TI, 32>(a, s);
        case 64: return run_step<TI, 64>(a, s);
        case 128: return run_step<TI, 128>(a, s);
        case 256: return run_step<TI, 256>(a, s);
        default: return SSD_ERR_UNSUPPORTED;
    }
}

ssd_status launch_step(const StepArgs &a, hipStream_t s) {
    return a.dtype == SSD_BF16 ? step_n<bf16>(a, s) : step_n<float>(a, s);
}

}  // namespace ssd
