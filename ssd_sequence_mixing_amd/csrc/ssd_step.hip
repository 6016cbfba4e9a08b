// One recurrent decode step for gfx950: the O(1)-per-token inference form of
// the SSM ("Transformer vs Mamba/SSM: the next step of the architecture",
// why it matters: each step only updates a fixed-size state).
//
//   a = exp(dt[b,h] A[h]);  s[p,n] <- a s[p,n] + dt x[p] B[g,n];
//   y[p] = sum_n s[p,n] C[g,n] + D[h] x[p]
//
// The state is the only large operand: the kernel streams it once in and
// once out with 16-byte accesses. A row of N fp32 values is split over N/4
// lanes; the dot product with C is reduced across those lanes with
// cross-lane shuffles. Each thread keeps UNROLL rows' loads in flight.
#include "ssd_common.h"
#include "ssd_internal.h"

namespace ssd {

template <typename TI, int N, int UNROLL>
__global__ __launch_bounds__(256) void k_step(StepArgs a, int64_t rows) {
    using Tr = Traits<TI>;
    constexpr int ES = Tr::kBytes;
    constexpr int TPR = N / 4;          // lanes per state row
    constexpr int RPW = 64 / TPR;       // rows per wavefront per pass
    constexpr int RPB = 4 * RPW * UNROLL;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int sub = lane / TPR, c4 = lane % TPR;
    const int P = (int)a.P, H = (int)a.H, G = (int)a.G;
    const int64_t row0 = (int64_t)blockIdx.x * RPB;

    f32x4 s[UNROLL];
    int64_t rr[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
        rr[u] = row0 + (int64_t)(u * 4 + w) * RPW + sub;
        if (rr[u] < rows)
            s[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(a.state + rr[u] * N) + c4);
        else
            s[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
        const int64_t R = rr[u];
        const bool ok = R < rows;
        const int64_t Rc = ok ? R : 0;
        const int64_t bh = Rc / P;
        const int p = (int)(Rc - bh * P);
        const int64_t bb = bh / H;
        const int h = (int)(bh - bb * H);
        const int g = (h * G) / H;
        const float dtv = Tr::to_f32(reinterpret_cast<const TI *>(a.dt)[bh]);
        const float xv = Tr::to_f32(reinterpret_cast<const TI *>(a.x)[bh * P + p]);
        const float dec = fast_exp2(dtv * a.A[h] * kLog2e);
        const float uin = dtv * xv;
        const TI *bp = reinterpret_cast<const TI *>(a.B) + (bb * G + g) * N + 4 * c4;
        const TI *cp = reinterpret_cast<const TI *>(a.C) + (bb * G + g) * N + 4 * c4;
        float bv[4], cv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            bv[e] = Tr::to_f32(bp[e]);
            cv[e] = Tr::to_f32(cp[e]);
        }
        f32x4 sn;
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sn[e] = dec * s[u][e] + uin * bv[e];
            part += sn[e] * cv[e];
        }
        if (ok) __builtin_nontemporal_store(sn, reinterpret_cast<f32x4 *>(a.state + R * N) + c4);
#pragma unroll
        for (int off = TPR / 2; off > 0; off >>= 1) part += __shfl_xor(part, off, 64);
        if (ok && c4 == 0) {
            const float yv = part + a.D[h] * xv;
            reinterpret_cast<TI *>(a.y)[bh * P + p] = Tr::from_f32(yv);
        }
    }
}

template <typename TI, int N>
static ssd_status run_step(const StepArgs &a, hipStream_t s) {
    constexpr int UNROLL = 4;
    constexpr int RPB = 4 * (64 / (N / 4)) * UNROLL;
    const int64_t rows = a.batch * a.H * a.P;
    const int64_t blocks = (rows + RPB - 1) / RPB;
    return launch(k_step<TI, N, UNROLL>, dim3((unsigned)blocks), dim3(256), s, a, rows) == hipSuccess
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
