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
// inputs too: a bf16 y would carry a rounding of up to 2^-8 |y|), or in bf16
// when the caller asks for y in the io dtype.
//
// Optionally (sections 6.1 and 6.3 of the same page): dt <- dt + dt_bias_h,
// then dt <- log(1 + e^dt) where dt <= 20; and y <- y * silu(z) after the D
// term (GATE: z is loaded with x, up front, like every other operand).

#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

namespace {

template <int N, typename Tio, bool GATE>
__global__ __launch_bounds__(256) void decode_step_kernel(
    float *__restrict__ state, const Tio *__restrict__ x, const float *__restrict__ dt,
    const Tio *__restrict__ B, const Tio *__restrict__ C, const float *__restrict__ A,
    const float *__restrict__ D, void *__restrict__ y, const float *__restrict__ dt_bias,
    int32_t softplus, const Tio *__restrict__ z, int32_t H, int32_t G, int32_t ybf) {
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
        part = group_sum<LPR>(part);   // the row's sum, in its last lane
        float out = part + Dh * xv[k];
        if constexpr (GATE) out *= fast_silu(zv[k]);
        if (sub == LPR - 1) store_y1(y, bh * P + p, out, ybf != 0);
    }
}

// ---------------------------------------------------------------------------
// decode_multi: K tokens per sequence in one launch ("Optimizing Nemotron v3
// Super in TensorRT-LLM", sections 10.3 and 10.4: the multi-token state update
// of speculative decoding).  Same work split as decode_step -- one workgroup
// per (b, h), the lane's slice of the state in registers -- but the state
// stays in registers across the K steps, so it is read once and written at
// most once per call instead of once per token.  SNAP writes the state after
// every step (the per-step snapshots, [Bt, K, H, P, N]); TREE restarts step k
// from the snapshot of step parent[b, k] when that is an earlier step (a
// draft tree; other values continue from step k - 1).  The snapshot is read
// back by the same lanes that wrote it, so no synchronisation is needed.
// Without update the state is only read (the verification pass).
template <int N, typename Tio, bool GATE>
struct TokenIn {
    static constexpr int ITER = 16 / (64 / (N / 4));
    float dtv;
    float4 Bv, Cv;
    float xv[ITER], zv[ITER];
};

template <int N, typename Tio, bool GATE, bool SNAP, bool TREE>
__global__ __launch_bounds__(256) void decode_multi_kernel(
    float *__restrict__ state, const Tio *__restrict__ x, const float *__restrict__ dt,
    const Tio *__restrict__ B, const Tio *__restrict__ C, const float *__restrict__ A,
    const float *__restrict__ D, void *__restrict__ y, const float *__restrict__ dt_bias,
    int32_t softplus, const Tio *__restrict__ z, float *__restrict__ snaps,
    const int32_t *__restrict__ parent, int32_t update, int32_t H, int32_t G, int32_t K,
    int32_t ybf) {
    constexpr int P = 64;
    constexpr int LPR = N / 4;         // lanes per state row
    constexpr int RPI = 64 / LPR;      // rows per wavefront iteration
    constexpr int ITER = 16 / RPI;     // rows per lane
    const int64_t bh = blockIdx.x;
    const int64_t b = bh / H;
    const int32_t h = (int32_t)(bh % H);
    const int32_t g = h / (H / G);
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int sub = lane % LPR, rw = lane / LPR;
    const float a2 = A[h] * kLog2e, Dh = D[h];
    const float bias = dt_bias ? dt_bias[h] : 0.f;
    int rowoff[ITER];                  // this lane's rows p, as offsets into a [P][N] state
#pragma unroll
    for (int i = 0; i < ITER; ++i) rowoff[i] = (16 * wave + RPI * i + rw) * N + 4 * sub;

    // the small per-token operands of step k (B, C of the head's group)
    auto load_tok = [&](int k, TokenIn<N, Tio, GATE> &in) {
        const int64_t tk = b * K + k;
        const int64_t th = tk * H + h;
        in.dtv = dt[th];
        in.Bv = load4(B + (tk * G + g) * N + 4 * sub);
        in.Cv = load4(C + (tk * G + g) * N + 4 * sub);
#pragma unroll
        for (int i = 0; i < ITER; ++i) {
            const int p = 16 * wave + RPI * i + rw;
            in.xv[i] = load1(x + th * P + p);
            if constexpr (GATE) in.zv[i] = load1(z + th * P + p);
        }
    };

    const float *st_in = state + bh * (int64_t)(P * N);
    float4 sv[ITER];
#pragma unroll
    for (int i = 0; i < ITER; ++i) sv[i] = load_nt(st_in + rowoff[i]);
    TokenIn<N, Tio, GATE> cur, nxt;
    load_tok(0, cur);
    for (int k = 0; k < K; ++k) {
        const int64_t th = (b * K + k) * H + h;
        load_tok(min(k + 1, K - 1), nxt);   // the next step's operands, in flight now
        if constexpr (TREE) {
            const int par = k > 0 ? parent[b * K + k] : -1;   // uniform over the workgroup
            if (par >= 0 && par < k) {
                const float *sp = snaps + ((b * K + par) * H + h) * (int64_t)(P * N);
#pragma unroll
                for (int i = 0; i < ITER; ++i)
                    sv[i] = *reinterpret_cast<const float4 *>(sp + rowoff[i]);
            }
        }
        float dtv = cur.dtv + bias;
        if (softplus && dtv <= 20.f) dtv = log1pf(expf(dtv));
        const float dA = fast_exp2(a2 * dtv);
        float *sn = SNAP ? snaps + th * (int64_t)(P * N) : nullptr;
#pragma unroll
        for (int i = 0; i < ITER; ++i) {
            const float u = dtv * cur.xv[i];
            sv[i].x = dA * sv[i].x + u * cur.Bv.x;
            sv[i].y = dA * sv[i].y + u * cur.Bv.y;
            sv[i].z = dA * sv[i].z + u * cur.Bv.z;
            sv[i].w = dA * sv[i].w + u * cur.Bv.w;
            if constexpr (SNAP) store_nt(sn + rowoff[i], sv[i]);
            float part = sv[i].x * cur.Cv.x + sv[i].y * cur.Cv.y + sv[i].z * cur.Cv.z +
                         sv[i].w * cur.Cv.w;
            part = group_sum<LPR>(part);   // the row's sum, in its last lane
            float out = part + Dh * cur.xv[i];
            if constexpr (GATE) out *= fast_silu(cur.zv[i]);
            if (sub == LPR - 1) store_y1(y, th * P + 16 * wave + RPI * i + rw, out, ybf != 0);
        }
        cur = nxt;
    }
    if (update && K > 0) {
        float *st_out = state + bh * (int64_t)(P * N);
#pragma unroll
        for (int i = 0; i < ITER; ++i) store_nt(st_out + rowoff[i], sv[i]);
    }
}

template <int N, typename Tio, bool GATE>
hipError_t launch_multi_g(const Shape &s, const MultiArgs &m, hipStream_t st) {
    const uint32_t nblk = (uint32_t)((uint64_t)s.Bt * s.H);
    const Tio *z = (const Tio *)m.z;
#define SSD_MULTI_LAUNCH(SNAP, TREE)                                                          \
    hipLaunchKernelGGL((decode_multi_kernel<N, Tio, GATE, SNAP, TREE>), dim3(nblk), dim3(256), \
                       0, st, m.state, (const Tio *)m.x, m.dt, (const Tio *)m.B,              \
                       (const Tio *)m.C, m.A, m.D, m.y, m.dt_bias, (int32_t)m.softplus, z,     \
                       m.snaps, m.parent, (int32_t)m.update, (int32_t)s.H, (int32_t)s.G,      \
                       (int32_t)s.T, (int32_t)s.ybf16)
    if (m.parent)
        SSD_MULTI_LAUNCH(true, true);
    else if (m.snaps)
        SSD_MULTI_LAUNCH(true, false);
    else
        SSD_MULTI_LAUNCH(false, false);
#undef SSD_MULTI_LAUNCH
    return hipGetLastError();
}

template <int N, typename Tio>
hipError_t launch_multi_t(const Shape &s, const MultiArgs &m, hipStream_t st) {
    if (m.z) return launch_multi_g<N, Tio, true>(s, m, st);
    return launch_multi_g<N, Tio, false>(s, m, st);
}

template <int N>
hipError_t launch_multi_n(const Shape &s, const MultiArgs &m, hipStream_t st) {
    if (s.bf16) return launch_multi_t<N, uint16_t>(s, m, st);
    return launch_multi_t<N, float>(s, m, st);
}

template <int N, typename Tio>
hipError_t launch_dec_t(const Shape &s, float *state, const void *x, const float *dt,
                        const void *B, const void *C, const float *A, const float *D, void *y,
                        const float *dt_bias, int softplus, const void *z, hipStream_t st) {
    const uint64_t nblk = (uint64_t)s.Bt * s.H;
    if (z)
        hipLaunchKernelGGL((decode_step_kernel<N, Tio, true>), dim3((uint32_t)nblk), dim3(256), 0,
                           st, state, (const Tio *)x, dt, (const Tio *)B, (const Tio *)C, A, D,
                           y, dt_bias, (int32_t)softplus, (const Tio *)z, (int32_t)s.H,
                           (int32_t)s.G, (int32_t)s.ybf16);
    else
        hipLaunchKernelGGL((decode_step_kernel<N, Tio, false>), dim3((uint32_t)nblk), dim3(256),
                           0, st, state, (const Tio *)x, dt, (const Tio *)B, (const Tio *)C, A,
                           D, y, dt_bias, (int32_t)softplus, (const Tio *)nullptr,
                           (int32_t)s.H, (int32_t)s.G, (int32_t)s.ybf16);
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

hipError_t launch_decode_multi(const Shape &s, const MultiArgs &m, hipStream_t st) {
    if (s.Bt == 0 || s.T == 0) return hipSuccess;
    if (s.N == 64) return launch_multi_n<64>(s, m, st);
    if (s.N == 128) return launch_multi_n<128>(s, m, st);
    return hipErrorInvalidValue;
}

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
