// chunk_scan: the output of each chunk from the state entering it,
//     y_i = exp2(G_i) C_i h_prev^T
//           + sum_{j <= i} exp2(G_i - G_j) (C_i . B_j) dt_j x_j  +  D x_i.
//
// "Accelerating Mamba-2 with High-Performance Forward Pass Kernels in NVIDIA
// CUDA Tile", section "Mamba-2 architecture" (Y = exp(G) C h + (exp(G - G^T)
// . C B^T . M) X + D X, M the causal mask including the diagonal) and
// section "Kernel 3" (C B^T never leaves the chip; the pairwise decay and the
// causal mask are applied to it before the second product; the positive
// exponents above the diagonal are discarded before they can overflow).  The
// "mamba3" kernel card ("Method") folds the causal weight and the decay into
// the drain of the first product's accumulator.
//
// bf16 path (MFMA, v_mfma_f32_16x16x32_bf16): one workgroup of 4 wavefronts
// per (b, h, chunk), heads fastest and kept on one XCD so B and C of the
// group come from L2.  A wavefront owns 16-row blocks of the chunk, paired
// (I, L/16-1-I) so that every wavefront has the same number of causal tiles.
// For a row block I (rows i0 = 16 I ...):
//   1. inter:  acc = C_I h_prev^T (K = N).  C rows are the A operand as
//      loaded (16 bytes a lane); h_prev rows (N contiguous) are the B operand
//      as loaded.  Output column m of MFMA s is p = 4m + s.
//   2. rows scaled by exp2(G_i).
//   3. intra: per 32-token step, two 16x16 tiles of (C B^T)^T = B C^T are
//      formed with MFMA (A = B rows, B = the C fragments of step 1).  The
//      accumulator layout of a transposed tile (lane m: column i, rows j =
//      4q..4q+3) is exactly a 4-element K slice of an A operand for row i,
//      so the drain -- times exp2(G_i - G_j) dt_j, select j <= i, round to
//      bf16 -- leaves the A operand of the second product in place, with no
//      LDS round trip.  The matching B operand (x rows of the same 8 tokens,
//      4 p per lane) is transposed in registers.  Tiles above the diagonal
//      are skipped.
//   4. y += D x, stored as bf16 (8 bytes a lane and row).
//
// fp32 path (VALU): one workgroup per (b, h, chunk), 16-row tiles: the
// decayed, masked C B^T rows are built in LDS, then each thread forms y for
// one p and four rows.

#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

namespace {

template <int L, int N>
__device__ __forceinline__ void scan_row_block(
    int I, const uint16_t *__restrict__ x, const uint16_t *__restrict__ Bm,
    const uint16_t *__restrict__ Cm, const float *__restrict__ Gp, const float *__restrict__ Dp,
    const uint16_t *__restrict__ Hp, uint16_t *__restrict__ y, float Dh, int64_t T, int64_t t0,
    int64_t b, int32_t h, int32_t H, int32_t g, int32_t G, int m, int q) {
    constexpr int P = 64;
    constexpr int NK = N / 32;  // K steps over n
    const int i0 = 16 * I;

    // C rows i0 + m, n = 32 kn + 8q .. +7: A operand of the inter product
    // and B operand of the B C^T tiles.
    uint4 cf[NK];
    {
        const int64_t tok = t0 + i0 + m;
        const bool ok = tok < T;
        const uint16_t *cp = Cm + ((b * T + tok) * G + g) * N + 8 * q;
#pragma unroll
        for (int kn = 0; kn < NK; ++kn)
            cf[kn] = ok ? *reinterpret_cast<const uint4 *>(cp + 32 * kn) : make_uint4(0, 0, 0, 0);
    }

    f32x4 acc[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) acc[s] = f32x4{0.f, 0.f, 0.f, 0.f};

    // 1. inter: acc[s][e] = sum_n C[i0+4q+e][n] h_prev[4m+s][n]
#pragma unroll
    for (int kn = 0; kn < NK; ++kn) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const uint4 hv =
                *reinterpret_cast<const uint4 *>(Hp + (4 * m + s) * N + 32 * kn + 8 * q);
            acc[s] = mfma16x16x32(as_bf16x8(cf[kn]), as_bf16x8(hv), acc[s]);
        }
    }
    // 2. rows i = i0 + 4q + e scaled by exp2(G_i)
    {
        const float4 gi = *reinterpret_cast<const float4 *>(Gp + i0 + 4 * q);
        const float sc[4] = {fast_exp2(gi.x), fast_exp2(gi.y), fast_exp2(gi.z), fast_exp2(gi.w)};
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[s][e] *= sc[e];
    }

    // 3. intra
    const float gcol = Gp[i0 + m];  // G of this lane's column i = i0 + m
    for (int jb2 = 0; 2 * jb2 <= I; ++jb2) {
        uint32_t cbw[2][2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int J = 2 * jb2 + u;
            if (J <= I) {
                f32x4 cbt = f32x4{0.f, 0.f, 0.f, 0.f};
                const int64_t tok = t0 + 16 * J + m;
                const bool ok = tok < T;
                const uint16_t *bp = Bm + ((b * T + tok) * G + g) * N + 8 * q;
#pragma unroll
                for (int kn = 0; kn < NK; ++kn) {
                    const uint4 bv = ok ? *reinterpret_cast<const uint4 *>(bp + 32 * kn)
                                        : make_uint4(0, 0, 0, 0);
                    cbt = mfma16x16x32(as_bf16x8(bv), as_bf16x8(cf[kn]), cbt);
                }
                // cbt[e] = (C B^T)[i = i0 + m][j = 16J + 4q + e]
                const float4 gj = *reinterpret_cast<const float4 *>(Gp + 16 * J + 4 * q);
                const float4 dj = *reinterpret_cast<const float4 *>(Dp + 16 * J + 4 * q);
                const float gjv[4] = {gj.x, gj.y, gj.z, gj.w};
                const float djv[4] = {dj.x, dj.y, dj.z, dj.w};
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float d = fminf(gcol - gjv[e], 0.f);
                    const float val = cbt[e] * fast_exp2(d) * djv[e];
                    const bool keep = (J < I) || (4 * q + e <= m);
                    v[e] = keep ? val : 0.f;
                }
                cbw[u][0] = pack_bf16x2(v[0], v[1]);
                cbw[u][1] = pack_bf16x2(v[2], v[3]);
            } else {
                cbw[u][0] = 0u;
                cbw[u][1] = 0u;
            }
        }
        const uint4 aw = make_uint4(cbw[0][0], cbw[0][1], cbw[1][0], cbw[1][1]);
        const bf16x8 af = as_bf16x8(aw);

        // x rows for the same K slots: slot r < 4 -> j = 32 jb2 + 4q + r,
        // slot r >= 4 -> j = 32 jb2 + 16 + 4q + (r - 4); 4 p (4m .. 4m+3) each.
        const bool second = (2 * jb2 + 1) <= I;
        uint2 xr[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int jl = 32 * jb2 + ((r < 4) ? 0 : 16) + 4 * q + (r & 3);
            const int64_t tok = t0 + jl;
            const bool ok = (tok < T) && (r < 4 || second);
            xr[r] = ok ? *reinterpret_cast<const uint2 *>(x + ((b * T + tok) * H + h) * P + 4 * m)
                       : make_uint2(0u, 0u);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            uint4 v;
            uint32_t *vw = reinterpret_cast<uint32_t *>(&v);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const uint32_t a0 = (s < 2) ? xr[2 * rr].x : xr[2 * rr].y;
                const uint32_t a1 = (s < 2) ? xr[2 * rr + 1].x : xr[2 * rr + 1].y;
                vw[rr] = (s & 1) ? pair_hi(a0, a1) : pair_lo(a0, a1);
            }
            acc[s] = mfma16x16x32(af, as_bf16x8(v), acc[s]);
        }
    }

    // 4. y = acc + D x for rows i0 + 4q + e, p = 4m .. 4m+3
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int64_t tok = t0 + i0 + 4 * q + e;
        if (tok < T) {
            const int64_t off = ((b * T + tok) * H + h) * P + 4 * m;
            const uint2 xv = *reinterpret_cast<const uint2 *>(x + off);
            uint2 o;
            o.x = pack_bf16x2(acc[0][e] + Dh * bf16_lo(xv.x), acc[1][e] + Dh * bf16_hi(xv.x));
            o.y = pack_bf16x2(acc[2][e] + Dh * bf16_lo(xv.y), acc[3][e] + Dh * bf16_hi(xv.y));
            *reinterpret_cast<uint2 *>(y + off) = o;
        }
    }
}

template <int L, int N>
__global__ __launch_bounds__(256) void chunk_scan_bf16_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ Bm,
    const uint16_t *__restrict__ Cm, const float *__restrict__ D, const float *__restrict__ Gws,
    const float *__restrict__ DTws, const uint16_t *__restrict__ hprev, uint16_t *__restrict__ y,
    int64_t T, int32_t H, int32_t G, int32_t nc, uint32_t nblk) {
    constexpr int P = 64;
    constexpr int NB = L / 16;
    const uint32_t lid = xcd_remap(blockIdx.x, nblk);
    const int32_t h = lid % H;
    const int32_t c = (lid / H) % nc;
    const int64_t b = lid / ((uint32_t)H * nc);
    const int32_t g = h / (H / G);
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int m = lane & 15, q = lane >> 4;

    const int64_t bhc = ((int64_t)b * H + h) * nc + c;
    const float *Gp = Gws + bhc * L;
    const float *Dp = DTws + bhc * L;
    const uint16_t *Hp = hprev + bhc * (int64_t)(P * N);
    const float Dh = D[h];
    const int64_t t0 = (int64_t)c * L;

    if constexpr (NB == 4) {
        scan_row_block<L, N>(wave, x, Bm, Cm, Gp, Dp, Hp, y, Dh, T, t0, b, h, H, g, G, m, q);
    } else {
        for (int pi = wave; pi < NB / 2; pi += 4) {
            scan_row_block<L, N>(pi, x, Bm, Cm, Gp, Dp, Hp, y, Dh, T, t0, b, h, H, g, G, m, q);
            scan_row_block<L, N>(NB - 1 - pi, x, Bm, Cm, Gp, Dp, Hp, y, Dh, T, t0, b, h, H, g, G,
                                 m, q);
        }
    }
}

template <int L, int N>
__global__ __launch_bounds__(256) void chunk_scan_f32_kernel(
    const float *__restrict__ x, const float *__restrict__ Bm, const float *__restrict__ Cm,
    const float *__restrict__ D, const float *__restrict__ Gws, const float *__restrict__ DTws,
    const float *__restrict__ hprev, float *__restrict__ y, int64_t T, int32_t H, int32_t G,
    int32_t nc, uint32_t nblk) {
    constexpr int P = 64;
    constexpr int RT = 16;  // rows per tile
    __shared__ float hs[P][N + 1];
    __shared__ float cs[RT][N + 1];
    __shared__ float cb[RT][L + 1];

    const uint32_t lid = xcd_remap(blockIdx.x, nblk);
    const int32_t h = lid % H;
    const int32_t c = (lid / H) % nc;
    const int64_t b = lid / ((uint32_t)H * nc);
    const int32_t g = h / (H / G);
    const int tid = threadIdx.x;
    const int p = tid % P, rq = tid / P;

    const int64_t bhc = ((int64_t)b * H + h) * nc + c;
    const float *Gp = Gws + bhc * L;
    const float *Dp = DTws + bhc * L;
    const float *Hp = hprev + bhc * (int64_t)(P * N);
    const float Dh = D[h];
    const int64_t t0 = (int64_t)c * L;

    for (int e = tid; e < P * N; e += 256) hs[e / N][e % N] = Hp[e];

    for (int i0 = 0; i0 < L; i0 += RT) {
        __syncthreads();
        for (int e = tid; e < RT * N; e += 256) {
            const int ii = e / N, n = e % N;
            const int64_t tok = t0 + i0 + ii;
            cs[ii][n] = tok < T ? Cm[((b * T + tok) * G + g) * N + n] : 0.f;
        }
        __syncthreads();
        // decayed, masked C B^T rows of this tile
        const int jmax = i0 + RT;  // columns j < jmax can be causal
        for (int e = tid; e < RT * jmax; e += 256) {
            const int ii = e / jmax, j = e % jmax;
            const int i = i0 + ii;
            float v = 0.f;
            const int64_t tj = t0 + j;
            if (j <= i && tj < T) {
                const float *bp = Bm + ((b * T + tj) * G + g) * N;
                float dot = 0.f;
                for (int n = 0; n < N; ++n) dot += cs[ii][n] * bp[n];
                v = dot * fast_exp2(fminf(Gp[i] - Gp[j], 0.f)) * Dp[j];
            }
            cb[ii][j] = v;
        }
        __syncthreads();
        for (int ii = rq; ii < RT; ii += 4) {
            const int i = i0 + ii;
            const int64_t tok = t0 + i;
            if (tok >= T) continue;
            float inter = 0.f;
            for (int n = 0; n < N; ++n) inter += cs[ii][n] * hs[p][n];
            float acc = fast_exp2(Gp[i]) * inter;
            for (int j = 0; j <= i; ++j) {
                const int64_t tj = t0 + j;
                if (tj >= T) break;
                acc += cb[ii][j] * x[((b * T + tj) * H + h) * P + p];
            }
            const int64_t off = ((b * T + tok) * H + h) * P + p;
            y[off] = acc + Dh * x[off];
        }
    }
}

template <int L, int N>
hipError_t launch_scan(const Shape &s, const void *x, const void *B, const void *C,
                       const float *D, const float *Gws, const float *DTws, const void *hprev,
                       void *y, hipStream_t st) {
    const uint64_t nblk = (uint64_t)s.Bt * s.nc * s.H;
    if (s.bf16)
        hipLaunchKernelGGL((chunk_scan_bf16_kernel<L, N>), dim3((uint32_t)nblk), dim3(256), 0, st,
                           (const uint16_t *)x, (const uint16_t *)B, (const uint16_t *)C, D, Gws,
                           DTws, (const uint16_t *)hprev, (uint16_t *)y, s.T, (int32_t)s.H,
                           (int32_t)s.G, (int32_t)s.nc, (uint32_t)nblk);
    else
        hipLaunchKernelGGL((chunk_scan_f32_kernel<L, N>), dim3((uint32_t)nblk), dim3(256), 0, st,
                           (const float *)x, (const float *)B, (const float *)C, D, Gws, DTws,
                           (const float *)hprev, (float *)y, s.T, (int32_t)s.H, (int32_t)s.G,
                           (int32_t)s.nc, (uint32_t)nblk);
    return hipGetLastError();
}

template <int L>
hipError_t launch_scan_n(const Shape &s, const void *x, const void *B, const void *C,
                         const float *D, const float *Gws, const float *DTws, const void *hprev,
                         void *y, hipStream_t st) {
    if (s.N == 64) return launch_scan<L, 64>(s, x, B, C, D, Gws, DTws, hprev, y, st);
    if (s.N == 128) return launch_scan<L, 128>(s, x, B, C, D, Gws, DTws, hprev, y, st);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_chunk_scan(const Shape &s, const void *x, const void *B, const void *C,
                             const float *D, const float *Gws, const float *DTws,
                             const void *hprev, void *y, hipStream_t st) {
    if (s.Bt == 0 || s.nc == 0) return hipSuccess;
    switch (s.L) {
    case 64: return launch_scan_n<64>(s, x, B, C, D, Gws, DTws, hprev, y, st);
    case 128: return launch_scan_n<128>(s, x, B, C, D, Gws, DTws, hprev, y, st);
    case 256: return launch_scan_n<256>(s, x, B, C, D, Gws, DTws, hprev, y, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ssd
