// chunk_state: the state one chunk contributes on its own,
//     S_c[p][n] = sum_j x_j[p] * w_j * B_j[n],   w_j = dt_j * exp2(G_last - G_j).
//
// "Accelerating Mamba-2 with High-Performance Forward Pass Kernels in NVIDIA
// CUDA Tile", section "Mamba-2 architecture" (the jump formula with the decay
// in log space: h_{t+T} = exp(G_last) h_t + (exp(G_last - G) . B)^T X) and
// section "Kernel 2" (the same product per chunk, operands scaled by dt and
// the decay before the matrix product).  Every exponent G_last - G_j is <= 0.
//
// bf16 path (MFMA): one workgroup per (b, h, chunk), one wavefront per 64
// state columns, heads fastest in the launch order (and kept on one XCD) so
// the group's B tile is served from L2 to all heads that share it.  The
// product is X^T diag(w) B with K = tokens, so both operands are read along
// their slow axis.  Instead of an LDS transpose, each lane loads 8-byte row
// segments (4 bf16) of 8 tokens and transposes them in registers into MFMA
// operands (v_mfma_f32_16x16x32_bf16, 8 bf16 of K per lane):
//   A operand, row m of MFMA s   = p = 4m + s        (64 rows in 4 MFMAs)
//   B operand, col m of MFMA sn  = n = 64t + 4m + sn (64 columns per wavefront)
// The weights w are folded into x (64 wide rather than N wide).  x*w is not
// exact in bf16, and rounding it once costs up to 2^-9 of every term of S --
// enough, where |S| runs far above its rms, to break a 2e-2 rms bound on the
// final state -- so it is carried as a bf16 head plus a bf16 remainder (two
// MFMAs, ~16 significant bits); B itself is exact.  The next 32-token slab is
// loaded while the current one is multiplied.  Accumulation is fp32; S is
// written fp32, 16 bytes a lane.
//
// fp32 path (VALU): one workgroup per (b, h, chunk); 32-token slices of X, B
// and w staged in LDS; each thread owns one n and 64*N/256 values of p.

#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

namespace {

template <int L, int N>
__global__ __launch_bounds__(N) void chunk_state_bf16_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ B,
    const float *__restrict__ Gws, const float *__restrict__ DTws, float *__restrict__ S,
    int64_t T, int32_t H, int32_t G, int32_t nc, uint32_t nblk) {
    constexpr int P = 64;
    const uint32_t lid = xcd_remap(blockIdx.x, nblk);
    const int32_t h = lid % H;
    const int32_t c = (lid / H) % nc;
    const int64_t b = lid / ((uint32_t)H * nc);
    const int32_t g = h / (H / G);
    const int t = threadIdx.x >> 6;          // this wavefront's 64 columns: n = 64t ..
    const int lane = threadIdx.x & 63;
    const int m = lane & 15, q = lane >> 4;

    const int64_t bhc = ((int64_t)b * H + h) * nc + c;
    const float *Gp = Gws + bhc * L;
    const float *Dp = DTws + bhc * L;
    const float glast = Gp[L - 1];

    // acc[s][sn]: rows p = 4M + s (M = 4q + i), columns n = 64t + 4m + sn
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[i][k] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint2 xr[8], br[8];
    auto load = [&](int ks) {
        const int j0 = 32 * ks + 8 * q;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int64_t tok = (int64_t)c * L + j0 + r;
            const bool ok = tok < T;
            const int64_t bt = b * T + tok;
            xr[r] = ok ? *reinterpret_cast<const uint2 *>(x + (bt * H + h) * P + 4 * m)
                       : make_uint2(0u, 0u);
            br[r] = ok ? *reinterpret_cast<const uint2 *>(B + (bt * G + g) * N + 64 * t + 4 * m)
                       : make_uint2(0u, 0u);
        }
    };
    load(0);
    for (int ks = 0; ks < L / 32; ++ks) {
        const int j0 = 32 * ks + 8 * q;  // this lane's 8 tokens: j0 .. j0+7
        float w[8];
        {
            const float4 g0 = *reinterpret_cast<const float4 *>(Gp + j0);
            const float4 g1 = *reinterpret_cast<const float4 *>(Gp + j0 + 4);
            const float4 d0 = *reinterpret_cast<const float4 *>(Dp + j0);
            const float4 d1 = *reinterpret_cast<const float4 *>(Dp + j0 + 4);
            w[0] = d0.x * fast_exp2(glast - g0.x);
            w[1] = d0.y * fast_exp2(glast - g0.y);
            w[2] = d0.z * fast_exp2(glast - g0.z);
            w[3] = d0.w * fast_exp2(glast - g0.w);
            w[4] = d1.x * fast_exp2(glast - g1.x);
            w[5] = d1.y * fast_exp2(glast - g1.y);
            w[6] = d1.z * fast_exp2(glast - g1.z);
            w[7] = d1.w * fast_exp2(glast - g1.w);
        }
        // A operands: x * w transposed (row m of MFMA s is p = 4m + s), split
        // into a bf16 head and the bf16 rounding of the remainder, so the
        // product carries ~16 significant bits; B is exact in bf16.
        bf16x8 ahi[4], alo[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            uint4 vh, vl;
            uint32_t *wh = reinterpret_cast<uint32_t *>(&vh);
            uint32_t *wl = reinterpret_cast<uint32_t *>(&vl);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const uint32_t a0 = (s < 2) ? xr[2 * rr].x : xr[2 * rr].y;
                const uint32_t a1 = (s < 2) ? xr[2 * rr + 1].x : xr[2 * rr + 1].y;
                const float e0 = ((s & 1) ? bf16_hi(a0) : bf16_lo(a0)) * w[2 * rr];
                const float e1 = ((s & 1) ? bf16_hi(a1) : bf16_lo(a1)) * w[2 * rr + 1];
                const uint32_t hw = pack_bf16x2(e0, e1);
                wh[rr] = hw;
                wl[rr] = pack_bf16x2(e0 - bf16_lo(hw), e1 - bf16_hi(hw));
            }
            ahi[s] = as_bf16x8(vh);
            alo[s] = as_bf16x8(vl);
        }
        // B operands: B rows transposed (column m of MFMA sn is n = 64t + 4m + sn)
        bf16x8 bfr[4];
#pragma unroll
        for (int sn = 0; sn < 4; ++sn) {
            uint4 v;
            uint32_t *vw = reinterpret_cast<uint32_t *>(&v);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const uint32_t a0 = (sn < 2) ? br[2 * rr].x : br[2 * rr].y;
                const uint32_t a1 = (sn < 2) ? br[2 * rr + 1].x : br[2 * rr + 1].y;
                vw[rr] = (sn & 1) ? pair_hi(a0, a1) : pair_lo(a0, a1);
            }
            bfr[sn] = as_bf16x8(v);
        }
        if (ks + 1 < L / 32) load(ks + 1);   // next slab in flight during the MFMAs
#pragma unroll
        for (int sn = 0; sn < 4; ++sn)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                acc[s][sn] = mfma16x16x32(ahi[s], bfr[sn], acc[s][sn]);
                acc[s][sn] = mfma16x16x32(alo[s], bfr[sn], acc[s][sn]);
            }
    }

    // D layout: lane holds rows M = 4q + i (i = 0..3) of column m.
    float *Sp = S + bhc * (int64_t)(P * N);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int p = 4 * (4 * q + i) + s;
            const float4 v = make_float4(acc[s][0][i], acc[s][1][i], acc[s][2][i], acc[s][3][i]);
            *reinterpret_cast<float4 *>(Sp + p * N + 64 * t + 4 * m) = v;
        }
}

template <int L, int N>
__global__ __launch_bounds__(256) void chunk_state_f32_kernel(
    const float *__restrict__ x, const float *__restrict__ B, const float *__restrict__ Gws,
    const float *__restrict__ DTws, float *__restrict__ S, int64_t T, int32_t H, int32_t G,
    int32_t nc, uint32_t nblk) {
    constexpr int P = 64;
    constexpr int KT = 32;                // tokens per LDS slice
    constexpr int PR = 256 / N;           // thread rows over p
    constexpr int NP = P / PR;            // p values per thread
    __shared__ float xs[KT][P + 1];
    __shared__ float bs[KT][N + 1];
    __shared__ float ws[KT];

    const uint32_t lid = xcd_remap(blockIdx.x, nblk);
    const int32_t h = lid % H;
    const int32_t c = (lid / H) % nc;
    const int64_t b = lid / ((uint32_t)H * nc);
    const int32_t g = h / (H / G);
    const int tid = threadIdx.x;
    const int n = tid % N, pr = tid / N;

    const int64_t bhc = ((int64_t)b * H + h) * nc + c;
    const float *Gp = Gws + bhc * L;
    const float *Dp = DTws + bhc * L;
    const float glast = Gp[L - 1];

    float acc[NP];
#pragma unroll
    for (int k = 0; k < NP; ++k) acc[k] = 0.f;

    for (int j0 = 0; j0 < L; j0 += KT) {
        for (int e = tid; e < KT * P; e += 256) {
            const int j = e / P, p = e % P;
            const int64_t tok = (int64_t)c * L + j0 + j;
            xs[j][p] = tok < T ? x[((b * T + tok) * H + h) * P + p] : 0.f;
        }
        for (int e = tid; e < KT * N; e += 256) {
            const int j = e / N, nn = e % N;
            const int64_t tok = (int64_t)c * L + j0 + j;
            bs[j][nn] = tok < T ? B[((b * T + tok) * G + g) * N + nn] : 0.f;
        }
        if (tid < KT) ws[tid] = Dp[j0 + tid] * fast_exp2(glast - Gp[j0 + tid]);
        __syncthreads();
#pragma unroll 4
        for (int j = 0; j < KT; ++j) {
            const float wb = ws[j] * bs[j][n];
#pragma unroll
            for (int k = 0; k < NP; ++k) acc[k] += xs[j][pr + PR * k] * wb;
        }
        __syncthreads();
    }
    float *Sp = S + bhc * (int64_t)(P * N);
#pragma unroll
    for (int k = 0; k < NP; ++k) Sp[(pr + PR * k) * N + n] = acc[k];
}

template <int L, int N>
hipError_t launch_cs(const Shape &s, const void *x, const void *B, const float *Gws,
                     const float *DTws, float *S, hipStream_t st) {
    const uint64_t nblk = (uint64_t)s.Bt * s.nc * s.H;
    if (s.bf16) {
        hipLaunchKernelGGL((chunk_state_bf16_kernel<L, N>), dim3((uint32_t)nblk), dim3(N), 0, st,
                           (const uint16_t *)x, (const uint16_t *)B, Gws, DTws, S, s.T,
                           (int32_t)s.H, (int32_t)s.G, (int32_t)s.nc, (uint32_t)nblk);
    } else {
        hipLaunchKernelGGL((chunk_state_f32_kernel<L, N>), dim3((uint32_t)nblk), dim3(256), 0, st,
                           (const float *)x, (const float *)B, Gws, DTws, S, s.T, (int32_t)s.H,
                           (int32_t)s.G, (int32_t)s.nc, (uint32_t)nblk);
    }
    return hipGetLastError();
}

template <int L>
hipError_t launch_cs_n(const Shape &s, const void *x, const void *B, const float *Gws,
                       const float *DTws, float *S, hipStream_t st) {
    if (s.N == 64) return launch_cs<L, 64>(s, x, B, Gws, DTws, S, st);
    if (s.N == 128) return launch_cs<L, 128>(s, x, B, Gws, DTws, S, st);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_chunk_state(const Shape &s, const void *x, const void *B, const float *Gws,
                              const float *DTws, float *S, hipStream_t st) {
    if (s.Bt == 0 || s.nc == 0) return hipSuccess;
    switch (s.L) {
    case 64: return launch_cs_n<64>(s, x, B, Gws, DTws, S, st);
    case 128: return launch_cs_n<128>(s, x, B, Gws, DTws, S, st);
    case 256: return launch_cs_n<256>(s, x, B, Gws, DTws, S, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ssd
