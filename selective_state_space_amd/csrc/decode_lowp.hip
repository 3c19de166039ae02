// decode_lowp: the decode step on a state kept in HBM at 16 bits per element
// ("Optimizing Nemotron v3 Super in TensorRT-LLM", section 6.5, and the
// state types of section 6.6's dispatch table):
//   FMT_F16_RN  fp16, round to nearest even;
//   FMT_F16_SR  fp16, stochastic rounding: |x| + (r / 2^13) ulp16(|x|),
//               rounded toward zero and saturated at 65504, with r a 13-bit
//               field of a Philox-4x32 word (the round count is a parameter;
//               one block per 8 consecutive elements of a row, counter = the
//               flat index (b, h, p, n) of the first, key = the 64-bit seed;
//               element n takes word (n mod 8) / 2, bits 0..12 for even n and
//               16..28 for odd n);
//   FMT_BF16    bf16, round to nearest even;
//   FMT_INT16   int16 codes with one fp32 decode scale per row p: after the
//               update, encode = 32767 / max|row| and decode = 1 / encode (both
//               IEEE fp32 divisions), codes = round-half-even(x * encode); an
//               all-zero row stores codes 0 and scale 0.
// The update and y are those of the fp32 decode step (y from the updated
// state before it is rounded for storage); only the load and the store of the
// state change, so the step moves 2 bytes per state element each way instead
// of 4.  A workgroup per (b, h); a row of N elements over N/8 lanes with
// 16-byte accesses (8 elements a lane, so one Philox block per lane and row);
// the row sums and the int16 row maximum are DPP reductions over those
// lanes.
//
// Philox-4x32 follows its published definition (Salmon, Moraes, Dror, Shaw,
// "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11): rounds of two
// 32x32 -> 64-bit products (multipliers 0xD2511F53, 0xCD9E8D57), a
// swap-and-xor with the key and a Weyl increment of the key.  Generating the
// bits costs ALU time (ten rounds: 20 integer multiplies per block, one
// block per 8 elements), which is why each word serves two elements.

#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

namespace {

enum { FMT_F16_RN = 0, FMT_F16_SR = 1, FMT_BF16 = 2, FMT_INT16 = 3 };

// NB Philox blocks advanced together (independent chains for the issue
// slots); counters (lo, hi, 0, 0), key (k0, k1).  Returns c[i][0..3].
template <int NB>
__device__ __forceinline__ void philox4x32(uint32_t (&c)[NB][4], uint32_t k0, uint32_t k1,
                                           int rounds) {
    for (int r = 0; r < rounds; ++r) {
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const uint64_t p0 = (uint64_t)c[i][0] * 0xD2511F53u;   // one 64-bit product each
            const uint64_t p1 = (uint64_t)c[i][2] * 0xCD9E8D57u;
            const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[i][1] ^ k0;
            const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[i][3] ^ k1;
            c[i][0] = n0;
            c[i][1] = (uint32_t)p1;
            c[i][2] = n2;
            c[i][3] = (uint32_t)p0;
        }
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
}

__device__ __forceinline__ float half_bits_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

__device__ __forceinline__ uint32_t f32_to_half_rn(float x) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}

// Stochastic rounding to fp16 with a 13-bit random integer r (see above).
__device__ __forceinline__ uint32_t f32_to_half_sr(float x, uint32_t r) {
    const uint32_t ux = __float_as_uint(x);
    const uint32_t sgn = (ux >> 16) & 0x8000u;
    const uint32_t ua = ux & 0x7FFFFFFFu;
    // |x| >= 2^-14: fp32 keeps 13 bits below fp16's ulp; the carry of the
    // added random bits is the round away from zero
    const uint32_t ut = (ua + r) & ~0x1FFFu;
    const uint32_t hn = ut >= 0x47800000u ? 0x7BFFu : (ut >> 13) - (112u << 10);
    // below, fp16 is subnormal: with |x| 2^24 = n + f (n whole, 0 <= f < 1) the
    // result is n units of 2^-24, or n + 1 where f 2^13 >= 2^13 - r, that is
    // floor((floor(|x| 2^37) + r) / 2^13) (|x| 2^37 < 2^23 is exact in fp32 and
    // the conversion truncates; a carry into 2^10 units is the smallest normal)
    const uint32_t hs = ((uint32_t)(__uint_as_float(ua) * 0x1p37f) + r) >> 13;
    return (ua >= 0x38800000u ? hn : hs) | sgn;
}

template <int N, typename Tio, bool GATE, int FMT>
__global__ __launch_bounds__(256) void decode_lowp_kernel(
    uint16_t *__restrict__ state, float *__restrict__ scale, const Tio *__restrict__ x,
    const float *__restrict__ dt, const Tio *__restrict__ B, const Tio *__restrict__ C,
    const float *__restrict__ A, const float *__restrict__ D, void *__restrict__ y,
    const float *__restrict__ dt_bias, int32_t softplus, const Tio *__restrict__ z,
    uint32_t seed_lo, uint32_t seed_hi, int32_t rounds, int32_t H, int32_t G, int32_t ybf) {
    constexpr int P = 64;
    constexpr int EPL = 8;             // state elements per lane (16 bytes)
    constexpr int LPR = N / EPL;       // lanes per state row
    constexpr int RPI = 64 / LPR;      // rows per wavefront iteration
    constexpr int ITER = 16 / RPI;     // rows per lane
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
    float bb[EPL], cc[EPL];
    {
        const Tio *Bp = B + (b * G + g) * N + EPL * sub, *Cp = C + (b * G + g) * N + EPL * sub;
        const float4 b0 = load4(Bp), b1 = load4(Bp + 4), c0 = load4(Cp), c1 = load4(Cp + 4);
        const float bv[EPL] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
        const float cv[EPL] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            bb[e] = bv[e];
            cc[e] = cv[e];
        }
    }

    uint16_t *st = state + bh * (int64_t)(P * N);
    uint4 sv[ITER];
    float xv[ITER], zv[ITER], sc[ITER];
#pragma unroll
    for (int k = 0; k < ITER; ++k) {
        const int p = 16 * wave + RPI * k + rw;
        sv[k] = load_nt8(st + p * N + EPL * sub);
        xv[k] = load1(x + bh * P + p);
        if constexpr (GATE) zv[k] = load1(z + bh * P + p);
        if constexpr (FMT == FMT_INT16) sc[k] = scale[bh * P + p];
    }
    // the random bits of this lane's 8 elements in each of its rows: one
    // Philox block per row, each word serving two elements
    uint32_t rb[FMT == FMT_F16_SR ? ITER : 1][4];
    if constexpr (FMT == FMT_F16_SR) {
#pragma unroll
        for (int k = 0; k < ITER; ++k) {
            const uint64_t first = (uint64_t)(bh * P + 16 * wave + RPI * k + rw) * N + EPL * sub;
            rb[k][0] = (uint32_t)first;
            rb[k][1] = (uint32_t)(first >> 32);
            rb[k][2] = 0u;
            rb[k][3] = 0u;
        }
        philox4x32<ITER>(rb, seed_lo, seed_hi, rounds);
    }
#pragma unroll
    for (int k = 0; k < ITER; ++k) {
        const int p = 16 * wave + RPI * k + rw;
        const uint32_t wd[4] = {sv[k].x, sv[k].y, sv[k].z, sv[k].w};
        float s[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const uint32_t w = (e & 1) ? wd[e >> 1] >> 16 : wd[e >> 1] & 0xffffu;
            if constexpr (FMT == FMT_BF16)
                s[e] = __uint_as_float(w << 16);
            else if constexpr (FMT == FMT_INT16)
                s[e] = (float)(int16_t)w * sc[k];
            else
                s[e] = half_bits_to_f32(w);
        }
        const float u = dtv * xv[k];
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            s[e] = dA * s[e] + u * bb[e];
            part = fmaf(s[e], cc[e], part);
        }
        part = group_sum<LPR>(part);   // the row's sum, in every lane of the row
        float out = part + Dh * xv[k];
        if constexpr (GATE) out *= fast_silu(zv[k]);
        if (sub == LPR - 1) store_y1(y, bh * P + p, out, ybf != 0);

        uint32_t o[EPL];
        if constexpr (FMT == FMT_BF16) {
#pragma unroll
            for (int e = 0; e < EPL; e += 2) {
                const uint32_t w = pack_bf16x2(s[e], s[e + 1]);
                o[e] = w & 0xffffu;
                o[e + 1] = w >> 16;
            }
        } else if constexpr (FMT == FMT_F16_RN) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) o[e] = f32_to_half_rn(s[e]);
        } else if constexpr (FMT == FMT_F16_SR) {
#pragma unroll
            for (int e = 0; e < EPL; ++e)
                o[e] = f32_to_half_sr(s[e], (rb[k][e >> 1] >> (16 * (e & 1))) & 0x1FFFu);
        } else {   // FMT_INT16
            float m = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) m = fmaxf(m, fabsf(s[e]));
            m = group_max<LPR>(m);
            const bool zero = m == 0.f;
            const float enc = 32767.f / (zero ? 1.f : m);
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const float q = fminf(fmaxf(rintf(s[e] * enc), -32767.f), 32767.f);
                o[e] = zero ? 0u : (uint32_t)(uint16_t)(int16_t)q;
            }
            if (sub == 0) scale[bh * P + p] = zero ? 0.f : 1.f / enc;
        }
        store_nt(st + p * N + EPL * sub, make_uint4(o[0] | (o[1] << 16), o[2] | (o[3] << 16),
                                                    o[4] | (o[5] << 16), o[6] | (o[7] << 16)));
    }
}

template <int N, typename Tio, bool GATE>
hipError_t launch_lowp_g(const Shape &s, const LowpArgs &a, hipStream_t st) {
    const uint32_t nblk = (uint32_t)((uint64_t)s.Bt * s.H);
    const uint32_t slo = (uint32_t)a.seed, shi = (uint32_t)(a.seed >> 32);
#define SSD_LOWP_LAUNCH(FMT)                                                                     \
    hipLaunchKernelGGL((decode_lowp_kernel<N, Tio, GATE, FMT>), dim3(nblk), dim3(256), 0, st,     \
                       (uint16_t *)a.state, a.scale, (const Tio *)a.x, a.dt, (const Tio *)a.B,    \
                       (const Tio *)a.C, a.A, a.D, a.y, a.dt_bias, (int32_t)a.softplus,           \
                       (const Tio *)a.z, slo, shi, (int32_t)a.philox_rounds, (int32_t)s.H, \
                       (int32_t)s.G, (int32_t)s.ybf16)
    switch (a.format) {
    case LOWP_F16:
        if (a.philox_rounds > 0)
            SSD_LOWP_LAUNCH(FMT_F16_SR);
        else
            SSD_LOWP_LAUNCH(FMT_F16_RN);
        break;
    case LOWP_BF16: SSD_LOWP_LAUNCH(FMT_BF16); break;
    case LOWP_INT16: SSD_LOWP_LAUNCH(FMT_INT16); break;
    default: return hipErrorInvalidValue;
    }
#undef SSD_LOWP_LAUNCH
    return hipGetLastError();
}

template <int N, typename Tio>
hipError_t launch_lowp_t(const Shape &s, const LowpArgs &a, hipStream_t st) {
    if (a.z) return launch_lowp_g<N, Tio, true>(s, a, st);
    return launch_lowp_g<N, Tio, false>(s, a, st);
}

template <int N>
hipError_t launch_lowp_n(const Shape &s, const LowpArgs &a, hipStream_t st) {
    if (s.bf16) return launch_lowp_t<N, uint16_t>(s, a, st);
    return launch_lowp_t<N, float>(s, a, st);
}

}  // namespace

hipError_t launch_decode_lowp(const Shape &s, const LowpArgs &a, hipStream_t st) {
    if (s.Bt == 0) return hipSuccess;
    if (s.N == 64) return launch_lowp_n<64>(s, a, st);
    if (s.N == 128) return launch_lowp_n<128>(s, a, st);
    return hipErrorInvalidValue;
}

}  // namespace ssd
