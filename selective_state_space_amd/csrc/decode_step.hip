// decode_step: one token of the recurrence, state updated in place,
//     dA = exp(A_h dt);  state[p][:] <- dA state[p][:] + (dt x[p]) B;
//     y[p] = state[p][:] . C + D_h x[p]      (y uses the updated state).
//
// "Optimizing Nemotron v3 Super in TensorRT-LLM", section 6.1 "The SSU Math"
// (the update for one head, batch x heads independent) and 6.2-6.4 (the
// eager form makes several HBM round trips of the state; one fused pass that
// reads and writes each state element once is the goal; wide vector loads
// of the state and an in-register reduction for y).  "mamba-metal: running
// Mamba on Apple Silicon", section on O(L) incremental decoding (the per-token
// step is elementwise on the carried state).
//
// The step moves the whole fp32 state through HBM once in each direction, so
// it is bandwidth-bound.  One workgroup of 4 wavefronts per (b, h); each
// wavefront owns 16 rows p.  A row of N floats is covered by N/4 lanes with
// 16-byte loads (one wavefront iteration moves 1 KB of contiguous state),
// and all of a lane's rows are loaded before any is used, so 4 (N = 128) or
// 8 (N = 64) independent 16-byte loads per lane are in flight.  y[p] is the
// sum over the N/4 lanes of a row, formed with xor shuffles inside the
// wavefront: no LDS, no atomics.  B_t and C_t of the head's group (N values)
// are read once per lane as 4-element vectors.  y is written fp32 (for bf16
// inputs too: a bf16 y would carry a rounding of up to 2^-8 |y|).
//
// Optionally (sections 6.1 and 6.3 of the same page): dt <- dt + dt_bias_h,
// then dt <- log(1 + e^dt) where dt <= 20; and y <- y * silu(z) after the D
// term (GATE: z is loaded with x, up front, like every other operand).

#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

namespace {

template <typename Tio>
__device__ __forceinline__ float4 load4(const Tio *p);
template <>
__device__ __forceinline__ float4 load4<float>(const float *p) {
    return *reinterpret_cast<const float4 *>(p);
}
template <>
__device__ __forceinline__ float4 load4<uint16_t>(const uint16_t *p) {
    const uint2 v = *reinterpret_cast<const uint2 *>(p);
    return make_float4(bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y));
}
__device__ __forceinline__ float load1(const float *p) { return *p; }
__device__ __forceinline__ float load1(const uint16_t *p) { return bf16_to_f32(*p); }

template <int N, typename Tio, bool GATE>
__global__ __launch_bounds__(256) void decode_step_kernel(
    float *__restrict__ state, const Tio *__restrict__ x, const float *__restrict__ dt,
    const Tio *__restrict__ B, const Tio *__restrict__ C, const float *__restrict__ A,
    const float *__restrict__ D, float *__restrict__ y, const float *__restrict__ dt_bias,
    int32_t softplus, const Tio *__restrict__ z, int32_t H, int32_t G) {
    constexpr int P = 64;
    constexpr int LPR = N / 4;         // lanes per state row
    constexpr int RPI = 64 / LPR;      // rows per wavefront iteration
    constexpr int ITER = 16 / RPI;     // iterations per wavefront (16 rows)
    const int64_t bh = blockIdx.x;
    const int64_t b = bh / H;
    const int32_t h = (int32_t)(bh % H);
    const int32_t g = h / (H / G);
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int sub = lane % LPR, rw = lane / LPR;

    float dtv = dt[bh];
    if (dt_bias) dtv += dt_bias[h];
    if (softplus && dtv <= 20.f) dtv = log1pf(expf(dtv));
    const float dA = fast_exp2(A[h] * dtv * kLog2e);
    const float Dh = D[h];
    const float4 Bv = load4(B + (b * G + g) * N + 4 * sub);
    const float4 Cv = load4(C + (b * G + g) * N + 4 * sub);

    float *st = state + bh * (int64_t)(P * N);
    float4 sv[ITER];
    float xv[ITER], zv[ITER];
#pragma unroll
    for (int k = 0; k < ITER; ++k) {
        const int p = 16 * wave + RPI * k + rw;
        sv[k] = load_nt(st + p * N + 4 * sub);
        xv[k] = load1(x + bh * P + p);
        if constexpr (GATE) zv[k] = load1(z + bh * P + p);
    }
#pragma unroll
    for (int k = 0; k < ITER; ++k) {
        const int p = 16 * wave + RPI * k + rw;
        const float u = dtv * xv[k];
        float4 ns;
        ns.x = dA * sv[k].x + u * Bv.x;
        ns.y = dA * sv[k].y + u * Bv.y;
        ns.z = dA * sv[k].z + u * Bv.z;
        ns.w = dA * sv[k].w + u * Bv.w;
        store_nt(st + p * N + 4 * sub, ns);
        float part = ns.x * Cv.x + ns.y * Cv.y + ns.z * Cv.z + ns.w * Cv.w;
#pragma unroll
        for (int off = LPR / 2; off > 0; off >>= 1) part += __shfl_xor(part, off, 64);
        float out = part + Dh * xv[k];
        if constexpr (GATE) out *= fast_silu(zv[k]);
        if (sub == 0) y[bh * P + p] = out;
    }
}

template <int N, typename Tio>
hipError_t launch_dec_t(const Shape &s, float *state, const void *x, const float *dt,
                        const void *B, const void *C, const float *A, const float *D, void *y,
                        const float *dt_bias, int softplus, const void *z, hipStream_t st) {
    const uint64_t nblk = (uint64_t)s.Bt * s.H;
    if (z)
        hipLaunchKernelGGL((decode_step_kernel<N, Tio, true>), dim3((uint32_t)nblk), dim3(256), 0,
                           st, state, (const Tio *)x, dt, (const Tio *)B, (const Tio *)C, A, D,
                           (float *)y, dt_bias, (int32_t)softplus, (const Tio *)z, (int32_t)s.H,
                           (int32_t)s.G);
    else
        hipLaunchKernelGGL((decode_step_kernel<N, Tio, false>), dim3((uint32_t)nblk), dim3(256),
                           0, st, state, (const Tio *)x, dt, (const Tio *)B, (const Tio *)C, A,
                           D, (float *)y, dt_bias, (int32_t)softplus, (const Tio *)nullptr,
                           (int32_t)s.H, (int32_t)s.G);
    return hipGetLastError();
}

template <int N>
hipError_t launch_dec(const Shape &s, float *state, const void *x, const float *dt, const void *B,
                      const void *C, const float *A, const float *D, void *y,
                      const float *dt_bias, int softplus, const void *z, hipStream_t st) {
    if (s.bf16)
        return launch_dec_t<N, uint16_t>(s, state, x, dt, B, C, A, D, y, dt_bias, softplus, z,
                                         st);
    return launch_dec_t<N, float>(s, state, x, dt, B, C, A, D, y, dt_bias, softplus, z, st);
}

}  // namespace

hipError_t launch_decode_step(const Shape &s, float *state, const void *x, const float *dt,
                              const void *B, const void *C, const float *A, const float *D,
                              void *y, const float *dt_bias, int softplus, const void *z,
                              hipStream_t st) {
    if (s.Bt == 0) return hipSuccess;
    if (s.N == 64) return launch_dec<64>(s, state, x, dt, B, C, A, D, y, dt_bias, softplus, z, st);
    if (s.N == 128)
        return launch_dec<128>(s, state, x, dt, B, C, A, D, y, dt_bias, softplus, z, st);
    return hipErrorInvalidValue;
}

}  // namespace ssd
